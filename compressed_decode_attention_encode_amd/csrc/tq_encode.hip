// TurboQuant encode kernels for gfx950.
//
// Rotated Lloyd-Max encode (keys with the QJL sketch; rotated-LM values; MSE-only keys):
//   TurboQuant vLLM guide (kwkr.cn), section 2, steps 1-3 and 5; TurboQuant-MLX page
//   (pomoai.com), core technique items 1-3.
// Group-32 symmetric values: TurboQuant vLLM guide, section 2, step 4.
// Per-block affine 8-bit keys: vllm-metal TurboQuant guide (wmrh.cn), quantisation
//   principle table (per-block scale, no rotation).
//
// Rotated Lloyd-Max encode, work decomposition: every wave of a persistent work-group walks
// 32-token blocks of the (batch, kv-head) slices on its own.  The rotation y = H diag(s) x
// runs on the matrix cores: with H_d = H_{d/32} (x) H_32 (Sylvester order, high index bits
// outer), each 32-feature input block goes through one 32 x 32 Hadamard product
// (v_mfma_f32_32x32x16_{f16,bf16}; the +-1 entries, with the rotation's sign flips folded
// in, and the fp16/bf16 inputs are exact operands, so only the float32 sums round), and the
// H_{d/32} stage combines the blocks' outputs inside each lane.  The Hadamard rows are fed
// in a permuted order so that lane l ends up holding the 16 contiguous coordinates
// 32 b + 16 (l / 32) + r (r = 0..15) of token l % 32 for every block b: the Lloyd-Max
// decision, the code packing and the residual all work on contiguous coordinates.
// The QJL projection z = S r (keys) is a second matrix-core product: the residual, split
// into fp16 hi + lo halves (every product with the fp16 S exact, ~21 significant bits
// carried), is already in the B-operand layout in the lanes' registers, and S is read from
// LDS as the A operand in the matching order, with its rows permuted like H's so that each
// lane's accumulators are 16 contiguous projection outputs (16 sign bits).
#include <type_traits>

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------
// Rotated Lloyd-Max encode.  QJL = true: keys (codes + QJL signs + fp16 (n, gamma));
// QJL = false: rotated values or MSE-only keys (codes + fp32 n).
// ---------------------------------------------------------------------------------

// Decisions work on y, thresholds and centroids scaled by the table's cell unit U = 2^e
// (exact), at least 2^6 for keys: the residual then enters the fp16 split as |r| U, where
// its low half stays a normal fp16 number for all but the smallest residuals (those keep an
// absolute error below 2^-24 / U); decisions are unchanged, the projection's sign needs no
// rescaling and gamma = sqrt(sum r'^2) / U.
constexpr int kKeyTabMinExp = 6;

// floor(x) as int32 in one instruction (NaN gives 0, values outside the int range saturate).
__device__ __forceinline__ int floor_i32(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
// Cell table of the Lloyd-Max decision.  Measure y in units of 2^-e of the unit
// coordinate, with e the smallest exponent from e_min on at which the scaled thresholds
// fall into different unit cells [j, j + 1) (so each cell holds at most one of them).  The
// entry of cell j then gives that threshold (+inf if the cell has none), the index
// #{i : t_i < j} of the cell's lower end and the centroids on both sides of the threshold:
// idx(y) = #{i : t_i < y} = entry.base + (y > entry.t) for every y in the cell, with one
// table read and one comparison instead of a search.  Scaling by 2^e is exact, so decisions
// and residuals are those of the unscaled arithmetic.  Codebooks whose thresholds crowd
// closer than 2^-kTabMaxExp (or are not ascending) return -1: the kernel then still builds
// the table at 2^kTabMaxExp (every read stays inside it) but decides each block again by
// counting the thresholds below y.
constexpr int kTabMaxExp = 7;
constexpr int kTabEntries = 2 * (1 << kTabMaxExp) + 2;   // cells j = -(U + 1) .. U, U = 2^e
struct __attribute__((aligned(16))) TabEntry {
  float t;         // threshold inside the cell, or +inf
  uint32_t base;   // #{i : t_i < j}
  float c_lo, c_hi;
};

template <int L>
__device__ int table_exponent(const float* __restrict__ thr, int e_min) {
  for (int e = e_min; e <= kTabMaxExp; ++e) {
    const float u = (float)(1 << e);
    bool ok = true;
    float prev = floorf(thr[0] * u);
    for (int i = 1; i < L - 1; ++i) {
      const float f = floorf(thr[i] * u);
      ok = ok && f > prev;           // false for NaN as well
      prev = f;
    }
    if (ok) return e;
  }
  return -1;
}

// Entry of cell j = e - (U + 1) for U = 2^te (thresholds and centroids scaled by U).
template <int L>
__device__ TabEntry table_entry(const float* __restrict__ thr, const float* __restrict__ cent, int e, int te) {
  const float u = (float)(1 << te);
  const float j = (float)(e - ((1 << te) + 1));
  uint32_t base = 0u;
  float t_in = __builtin_huge_valf();
  for (int i = 0; i < L - 1; ++i) {
    const float t = thr[i] * u;
    if (t < j) ++base;
    else if (t < j + 1.f) t_in = t;
  }
  return {t_in, base, cent[base] * u, cent[base + 1 < (uint32_t)L ? base + 1 : base] * u};
}

// Row of H_32 (or of S within a 32-row block) fed to matrix row m: the accumulator of
// register r in lane l (matrix row 8 (r / 4) + 4 (l / 32) + r % 4) then holds output
// 16 (l / 32) + r.
__host__ __device__ constexpr int rot_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// 32 x 32 x 16 matrix-core product with 16-bit operands of the input type.
template <int DT>
__device__ __forceinline__ floatx16 mfma_in(uint4 a, uint4 b, floatx16 c) {
  if constexpr (DT == TQ_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0,
                                                  0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  }
}

__device__ __forceinline__ floatx16 mfma_f16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// c + lo^2 + hi^2 of a pair of 16-bit inputs (exact products, float32 sum).
template <int DT>
__device__ __forceinline__ float sq2(uint32_t x, float c) {
  if constexpr (DT == TQ_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), __builtin_bit_cast(f16x2_t, x), c, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, x), c, false);
  }
}

// Values of lanes l and l ^ 32 for every lane: .lo = the lane-half-0 value (lanes 0..31),
// .hi = the lane-half-1 value (lanes 32..63), in both halves (one permlane32 swap).
struct HalfPair {
  uint32_t lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {(uint32_t)p[0], (uint32_t)p[1]};
}

// Waves per work-group, and waves per SIMD the registers are budgeted for: keys at d = 256
// hold 128 residual registers through the projection and their S fills most of a CU's LDS,
// so they run one wave per SIMD (one group per CU) without spilling.
template <int D>
constexpr int rot_waves() { return 4; }
template <int D, bool QJL>
constexpr int rot_waves_per_simd() { return D <= 64 ? (QJL ? 3 : 4) : ((D >= 256 && QJL) ? 1 : 2); }

template <int D, int KB, int DT, bool QJL>
__global__ void __launch_bounds__(64 * rot_waves<D>()) __attribute__((amdgpu_waves_per_eu(rot_waves_per_simd<D, QJL>())))
encode_lm_kernel(const uint16_t* __restrict__ x, int T, int mb_per_slice, int n_mb, int dst_offset, int cap,
                 const float* __restrict__ cent, const float* __restrict__ thr,
                 const uint32_t* __restrict__ sign_mask, const uint16_t* __restrict__ S,
                 uint32_t* __restrict__ codes_out, uint32_t* __restrict__ signs_out,
                 uint32_t* __restrict__ aux_out) {
  constexpr int NB = D / 32;                       // 32-feature blocks
  constexpr int NK = D / 16;                       // 16-feature input operand blocks
  constexpr int NW = rot_waves<D>();
  constexpr int L = 1 << KB;
  constexpr int PER = (KB == 3) ? 10 : 32 / KB;   // codes per word
  constexpr int WK = (D + PER - 1) / PER;          // words per row
  constexpr int CW = (16 * KB + 31) / 32;          // words of a lane's 16-code chunk
  constexpr int SP = D + 8;                        // LDS row stride of S (halves)
  constexpr bool kPrefetch = D <= 128 || QJL;       // next block's inputs held in registers
  static_assert(NB >= 2 && NB <= 8, "head_dim 64..256");

  __shared__ uint4 s_h[NB * 2 * kWave];            // rotation A operands, per (block, k-half, lane)
  __shared__ float s_cent[16];
  __shared__ TabEntry s_tab[kTabEntries];
  __shared__ __attribute__((aligned(16))) uint16_t s_S[QJL ? D * SP : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;                         // lane half
  const int col = lane & 31;                       // token within the 32-token block

  // A operands of the rotation: lane l, k-half kb of block b holds
  // H_32[rot_row(l % 32)][16 kb + 8 (l / 32) + i] * s[32 b + 16 kb + 8 (l / 32) + i], i = 0..7
  for (int e = tid; e < NB * 2 * kWave; e += kWave * NW) {
    const int l = e & 63, kb = (e >> 6) & 1, b = e >> 7;
    const int row = rot_row(l & 31);
    const uint32_t one = (DT == TQ_F16) ? 0x3C00u : 0x3F80u;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t pair = 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 16 * kb + 8 * (l >> 5) + 2 * q + u;
        const int j = 32 * b + c;
        const uint32_t neg = (uint32_t)(__popc(row & c) & 1) ^ ((sign_mask[j >> 5] >> (j & 31)) & 1u);
        pair |= (one | (neg << 15)) << (16 * u);
      }
      w[q] = pair;
    }
    s_h[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // decision units: U = 2^te per unit coordinate
  const int te0 = table_exponent<L>(thr, QJL ? kKeyTabMinExp : 0);
  const bool crowded = te0 < 0;                    // uniform over the launch
  const int te = crowded ? kTabMaxExp : te0;
  const int U = 1 << te;
  const float uf = (float)U, inv_uf = 1.f / (float)U;   // exact
  for (int e = tid; e < 2 * U + 2; e += kWave * NW) s_tab[e] = table_entry<L>(thr, cent, e, te);
  if (tid < L) s_cent[tid] = cent[tid] * uf;
  if constexpr (QJL) {
    for (int e = tid; e < D * D / 8; e += kWave * NW) {
      const int r = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint4*>(&s_S[r * SP + 8 * c8]) = reinterpret_cast<const uint4*>(S)[e];
    }
  }
  __syncthreads();
  const TabEntry* tab0 = s_tab + (U + 1);          // entry of cell j at tab0[j]
  // -1 kept opaque so that r - (float)hi stays a multiply-add with an fp16 operand
  // (v_fma_mix_f32) instead of a conversion and a subtraction
  float neg_one = -1.f;
  asm volatile("" : "+v"(neg_one));

  // this lane's S row offset (QJL A operands): row rot_row(col) of each 32-row block,
  // columns 16 h + 8 j of each 32-feature block
  const int s_base = rot_row(col) * SP + 16 * h;

  // input operands: xr[k] = features 16 k + 8 h .. + 7 of token col (B layout)
  auto load = [&](int mb, uint4 (&dst)[NK]) {
    const int slice = mb / mb_per_slice;
    const int t = min((mb % mb_per_slice) * 32 + col, T - 1);     // rows past T repeat the last one
    const uint4* src = reinterpret_cast<const uint4*>(x + ((size_t)slice * T + t) * D + 8 * h);
#pragma unroll
    for (int k = 0; k < NK; ++k) dst[k] = src[2 * k];
  };

  const int first = blockIdx.x * NW + wave;
  const int stride = gridDim.x * NW;
  uint4 xr[NK];
  if (first < n_mb) load(first, xr);

  for (int mb = first; mb < n_mb; mb += stride) {
    const int slice = mb / mb_per_slice;
    const int t0 = (mb % mb_per_slice) * 32;
    const bool valid = col < T - t0;
    const size_t row = (size_t)slice * cap + dst_offset + t0 + col;

    if constexpr (!kPrefetch) load(mb, xr);

    // ---- norm of the input ---------------------------------------------------------
    // keys: float32 sums of exact squares (n stored as fp16); values / MSE keys: float64,
    // so the stored float32 n is the correctly rounded norm
    float n;
    double ss64 = 0.0;
    float ss32 = 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const uint32_t w4[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (QJL) {
          ss32 = sq2<DT>(w4[q], ss32);
        } else {
          const double a = (double)in_to_f32<DT>(w4[q] & 0xFFFFu), b = (double)in_to_f32<DT>(w4[q] >> 16);
          ss64 = fma(a, a, ss64);
          ss64 = fma(b, b, ss64);
        }
      }
    }

    // bf16 inputs span the float32 exponent range: a float32 sum of squares can underflow
    // (|x| below ~1e-19, down to the subnormals) and the rotated sums can overflow (|x|
    // above ~1e37).  Such a token (rare; never a zero vector) is rescaled by a power of two --
    // exact for every input, and the codes depend only on the direction -- before the
    // rotation; its norm is divided back.  fp16 inputs never need it.
    float inv_s = 1.f;
    if constexpr (DT == TQ_BF16) {
      bool odd;
      if constexpr (QJL) {
        const HalfPair p = half_pair(__float_as_uint(ss32));
        const float tot = __uint_as_float(p.lo) + __uint_as_float(p.hi);
        odd = !(tot >= 0x1p-100f && tot <= 0x1p100f);
      } else {
        const uint64_t u = (uint64_t)__double_as_longlong(ss64);
        const HalfPair plo = half_pair((uint32_t)u), phi = half_pair((uint32_t)(u >> 32));
        const double tot = __longlong_as_double((long long)(((uint64_t)phi.lo << 32) | plo.lo)) +
                           __longlong_as_double((long long)(((uint64_t)phi.hi << 32) | plo.hi));
        odd = !(tot >= 0x1p-100 && tot <= 0x1p100);
      }
      if (__builtin_amdgcn_ballot_w64(odd) != 0) {
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const uint32_t w4[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            amax = fmaxf(amax, fmaxf(fabsf(in_to_f32<DT>(w4[q] & 0xFFFFu)), fabsf(in_to_f32<DT>(w4[q] >> 16))));
        }
        const HalfPair pm = half_pair(__float_as_uint(amax));
        amax = fmaxf(__uint_as_float(pm.lo), __uint_as_float(pm.hi));
        const bool need = odd && amax > 0.f;
        int e = 0;
        (void)frexpf(need ? amax : 1.f, &e);
        const int k2 = need ? 1 - e : 0;            // scaled maximum in [2, 4)
        inv_s = ldexpf(1.f, -k2);                   // may be subnormal: the stored fp16 n rounds to 0 then
        if constexpr (QJL) ss32 = 0.f;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          uint32_t w4[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a = ldexpf(in_to_f32<DT>(w4[q] & 0xFFFFu), k2);
            const float b = ldexpf(in_to_f32<DT>(w4[q] >> 16), k2);
            w4[q] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);   // exact in bf16
            if constexpr (QJL) ss32 = sq2<DT>(w4[q], ss32);
          }
          xr[k] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
      }
    }

    // ---- rotation: one Hadamard product per 32-feature block, then H_{d/32} in-lane ----
    floatx16 y[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      y[b] = floatx16{};
      y[b] = mfma_in<DT>(s_h[(2 * b) * kWave + lane], xr[2 * b], y[b]);
      y[b] = mfma_in<DT>(s_h[(2 * b + 1) * kWave + lane], xr[2 * b + 1], y[b]);
      if constexpr (D >= 256) __builtin_amdgcn_sched_barrier(0);   // two A operands live at a time
    }
    if constexpr (kPrefetch) {
      if (mb + stride < n_mb) load(mb + stride, xr);     // in flight through the rest of the block
    }
#pragma unroll
    for (int s = 1; s < NB; s <<= 1) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if ((b & s) == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = y[b][r], c = y[b + s][r];
            y[b][r] = a + c;
            y[b + s][r] = a - c;
          }
        }
      }
    }
    float scale;
    if constexpr (QJL) {
      const HalfPair p = half_pair(__float_as_uint(ss32));
      const float ns = sqrtf(__uint_as_float(p.lo) + __uint_as_float(p.hi));   // norm of the (rescaled) input
      n = ns * inv_s;
      scale = (ns > 0.f) ? uf / (sqrtf((float)D) * ns) : 0.f;
    } else {
      const uint64_t u = (uint64_t)__double_as_longlong(ss64);
      const HalfPair plo = half_pair((uint32_t)u), phi = half_pair((uint32_t)(u >> 32));
      const double n64 = sqrt(__longlong_as_double((long long)(((uint64_t)phi.lo << 32) | plo.lo)) +
                              __longlong_as_double((long long)(((uint64_t)phi.hi << 32) | plo.hi)));
      n = (float)n64;
      scale = (n64 > 0.0) ? (float)((double)uf / (sqrt((double)D) * n64 / (double)inv_s)) : 0.f;
    }

    // ---- Lloyd-Max decision, packed codes, residual --------------------------------
    uint32_t cw[NB][CW];
    uint32_t rh[QJL ? NB : 1][8], rl[QJL ? NB : 1][8];
    float gg = 0.f;
    // block b's codes (and residual halves), with g accumulated over its coordinates: by
    // the cell table, or (COUNT) by counting the thresholds below y.  idx = #{i : t_i < y};
    // the float32 y differs from the exact one by ~1e-7, so a decision can change only next
    // to a threshold
    auto decide = [&](const int b, float g, auto count_tag) -> float {
      constexpr bool COUNT = decltype(count_tag)::value;
      // table path: entries are read kAhead coordinates ahead of their use (a ring in
      // registers), so the LDS latency hides behind the work on earlier coordinates
      using Ent = std::conditional_t<QJL, TabEntry, float2>;   // values need (t, base) only
      constexpr int kAhead = 4;
      float ysv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ysv[i] = y[b][i] * scale;
      auto fetch = [&](int i) -> Ent {
        // |ys| <= U (1 + 1e-6): y is the unnormalised rotation of x (|y| <= sqrt(d) |x|) and
        // scale = U / (sqrt(d) |x|), so floor(ys) lies in [-(U + 1), U] and no clamp is
        // needed.  ys is NaN only when the input norm is not finite (scale 0): the
        // conversion then gives 0, or a saturated value whose offset wraps to cell 0 / -1
        // (16 x 2^31 = 0 and 16 (2^31 - 1) = -16 modulo 2^32), so every read stays inside
        // the table.
        return *reinterpret_cast<const Ent*>(tab0 + floor_i32(ysv[i]));
      };
      Ent ring[kAhead];
      if constexpr (!COUNT) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i) ring[i] = fetch(i);
      }
#pragma unroll
      for (int i = 0; i < CW; ++i) cw[b][i] = 0u;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float rr[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = r + u;
          const float ys = ysv[i];
          uint32_t idx;
          float c = 0.f;                             // centroid (keys: for the residual)
          if constexpr (COUNT) {
            // against the unscaled thresholds (uniform loads; ys / U is exact)
            const float yu = ys * inv_uf;
            idx = 0u;
#pragma unroll
            for (int k = 0; k < L - 1; ++k) idx += (thr[k] < yu) ? 1u : 0u;
            if constexpr (QJL) c = s_cent[idx];
          } else {
            const Ent e = ring[i % kAhead];
            if (i + kAhead < 16) ring[i % kAhead] = fetch(i + kAhead);
            // idx (and c) taken while the comparison is live (else every mask waits for the
            // packing); the volatile statement also keeps the reads in this order
            if constexpr (QJL) {
              const bool up = ys > e.t;
              idx = e.base + (up ? 1u : 0u);
              c = up ? e.c_hi : e.c_lo;
              asm volatile("" : "+v"(idx), "+v"(c));
            } else {
              idx = __float_as_uint(e.y) + ((ys > e.x) ? 1u : 0u);
              asm volatile("" : "+v"(idx));
            }
          }
          const int bit = KB * i;
          cw[b][bit >> 5] |= idx << (bit & 31);
          if ((bit & 31) + KB > 32) cw[b][(bit >> 5) + 1] |= idx >> (32 - (bit & 31));
          if constexpr (QJL) {
            rr[u] = ys - c;
            g = fmaf(rr[u], rr[u], g);
          }
        }
        if constexpr (QJL) {
          // hi = fp16(r) and lo = fp16(r - hi), both rounded toward zero (r - hi is exact in
          // float32: one mixed-precision multiply-add per coordinate)
          const auto hi = __builtin_amdgcn_cvt_pkrtz(rr[0], rr[1]);
          const auto lo = __builtin_amdgcn_cvt_pkrtz(fmaf((float)hi[0], neg_one, rr[0]), fmaf((float)hi[1], neg_one, rr[1]));
          rh[b][r / 2] = __builtin_bit_cast(uint32_t, hi);
          rl[b][r / 2] = __builtin_bit_cast(uint32_t, lo);
        }
      }
      return g;
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (crowded) gg = decide(b, gg, std::true_type{});
      else gg = decide(b, gg, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);     // block b's rotated values die here
    }

    // ---- store the codes: a lane holds codes 32 b + 16 h .. + 15 of its token ----------
    if constexpr (KB == 2) {
      if (valid) {
#pragma unroll
        for (int b = 0; b < NB; ++b) codes_out[row * WK + 2 * b + h] = cw[b][0];
      }
    } else if constexpr (KB == 4) {
      if (valid) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          *reinterpret_cast<uint2*>(codes_out + row * WK + 4 * b + 2 * h) = make_uint2(cw[b][0], cw[b][1]);
      }
    } else {
      // 3-bit codes, ten per word: both lane halves assemble the token's whole 3d-bit
      // stream (block b: the half-0 lane's 48 bits, then the half-1 lane's), then word w =
      // bits 30 w .. 30 w + 29; the half-0 lane stores the even words, the half-1 lane the odd
      constexpr int NS = 3 * NB;
      uint32_t st[NS + 1];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const HalfPair a = half_pair(cw[b][0]);   // low 32 bits of each half's chunk
        const HalfPair c = half_pair(cw[b][1]);   // high 16 bits
        st[3 * b] = a.lo;
        st[3 * b + 1] = (c.lo & 0xFFFFu) | (a.hi << 16);
        st[3 * b + 2] = (a.hi >> 16) | (c.hi << 16);
      }
      st[NS] = 0u;
#pragma unroll
      for (int w = 0; w < WK; ++w) {
        const int bb = 30 * w;
        const uint32_t word = __builtin_amdgcn_alignbit(st[(bb >> 5) + 1], st[bb >> 5], (uint32_t)(bb & 31)) & 0x3FFFFFFFu;
        if (valid && (w & 1) == h) codes_out[row * WK + w] = word;
      }
    }

    if constexpr (QJL) {
      const HalfPair p = half_pair(__float_as_uint(gg));
      const float g = sqrtf(__uint_as_float(p.lo) + __uint_as_float(p.hi)) * inv_uf;
      if (valid && h == 0) {
        const uint32_t nb16 = __builtin_bit_cast(uint16_t, (_Float16)n);
        const uint32_t gb16 = __builtin_bit_cast(uint16_t, (_Float16)g);
        aux_out[row] = nb16 | (gb16 << 16);
      }

      // ---- QJL projection z = S r on the matrix cores, 16 sign bits per lane and block --
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        floatx16 z = {};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint4 a = *reinterpret_cast<const uint4*>(&s_S[s_base + 32 * nb * SP + 32 * b + 8 * j]);
            z = mfma_f16(a, make_uint4(rh[b][4 * j], rh[b][4 * j + 1], rh[b][4 * j + 2], rh[b][4 * j + 3]), z);
            z = mfma_f16(a, make_uint4(rl[b][4 * j], rl[b][4 * j + 1], rl[b][4 * j + 2], rl[b][4 * j + 3]), z);
          }
        }
        // register r holds output 32 nb + 16 h + r; stored bit = (z >= 0), from the sign bit
        // (shifted in from the top register down: bit r = sign of z[r])
        uint32_t neg = 0u;
#pragma unroll
        for (int r = 15; r >= 0; --r) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(z[r]), 31);
        const HalfPair p2 = half_pair(~neg & 0xFFFFu);
        if (valid && h == (nb & 1)) signs_out[row * NB + nb] = p2.lo | (p2.hi << 16);
        __builtin_amdgcn_sched_barrier(0);   // one output block's operands live at a time
      }
    } else {
      if (valid && h == 0) aux_out[row] = __float_as_uint(n);
    }
  }
}

// ---------------------------------------------------------------------------------
// Group-32 symmetric values and per-block affine 8-bit keys: four lanes per 32-element
// group, 8 elements (one 16-byte load) per lane, so consecutive lanes read consecutive
// 16 bytes; the group's max / min is reduced across the lane quad with DPP moves.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __uint_as_float(xor_lanes_u32<1>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(xor_lanes_u32<2>(__float_as_uint(v))));
}
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, __uint_as_float(xor_lanes_u32<1>(__float_as_uint(v))));
  return fminf(v, __uint_as_float(xor_lanes_u32<2>(__float_as_uint(v))));
}

template <int DT>
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, float (&v)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = in_to_f32<DT>(w[k] & 0xFFFFu);
    v[2 * k + 1] = in_to_f32<DT>(w[k] >> 16);
  }
}

// Symmetric group quantiser.  The level boundaries tau_k = Delta (k - L/2) are exact in
// float32 (an fp16 Delta times a small integer), so the float32 estimate of
// rne(v/Delta + (L-1)/2) is corrected by two exact comparisons; a value exactly on a
// boundary goes to the even level, as round-half-to-even does.
__device__ __forceinline__ bool passes(float v, float tau, int k) {
  return (k & 1) ? (v > tau) : (v >= tau);
}

// Thread-to-data map of the group kernels: grid.y walks the (batch, kv-head) slices, and a
// work-group covers kGroupItems * 256 consecutive 8-element parts of one slice; item u of
// a thread is part  blockIdx.x * 256 * kGroupItems + 256 u + threadIdx.x, so each item's
// loads are coalesced and all of a thread's loads are in flight before any is used.
// A part count per slice of T * d / 8 is a multiple of 4 and every item offset is a
// multiple of 64: a lane quad (one 32-group) is entirely inside or outside the slice.
constexpr int kGroupItems = 4;

template <int D, int VB, int DT>
__global__ void __launch_bounds__(256)
encode_group_kernel(const uint16_t* __restrict__ x, int T, int slices, int dst_offset, int cap,
                    uint32_t* __restrict__ codes_out, uint16_t* __restrict__ scale_out) {
  constexpr int G = D / 32;
  constexpr int L = 1 << VB;
  constexpr int WV = D * VB / 32;
  const int parts = T * (D / 8);
  for (int slice = blockIdx.y; slice < slices; slice += gridDim.y) {
    const uint16_t* xs = x + (size_t)slice * T * D;
    const size_t row_s = (size_t)slice * cap + dst_offset;
    float v[kGroupItems][8];
#pragma unroll
    for (int u = 0; u < kGroupItems; ++u) {
      const int p = (blockIdx.x * kGroupItems + u) * 256 + threadIdx.x;
      if (p < parts) {
        load8<DT>(xs + (size_t)p * 8, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kGroupItems; ++u) {
      const int p = (blockIdx.x * kGroupItems + u) * 256 + threadIdx.x;
      const int sub = p & 3, g = (p >> 2) % G, t = p / (D / 8);
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
      amax = quad_max(amax);
      // Delta = fp16(2 amax / (L-1)): amax is an fp16/bf16 value, so the exact quotient has
      // a repeating binary fraction (k/3 or k/15) that stays >= 1/30 of an fp16 ulp away
      // from a rounding tie; the float32 product with the rounded reciprocal (error ~1e-7
      // relative) therefore rounds to the same fp16 value as the exact quotient.
      const uint32_t dbits = __builtin_bit_cast(uint16_t, (_Float16)(2.0f * amax * (1.0f / (float)(L - 1))));
      const float delta = f16_to_f32(dbits);
      const float inv = (delta > 0.f) ? 1.0f / delta : 0.f;
      const float off = 0.5f * (float)(L - 1);
      uint32_t code = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ve = v[u][e];
        // x = v/Delta + (L-1)/2 to within 2^-20; only an x within 2^-16 of a half-integer
        // (a level boundary, exact ties included) needs the exact test
        const float x = fmaf(ve, inv, off);
        const float kr = rintf(x);
        float kf = fminf(fmaxf(kr, 0.f), (float)(L - 1));
        if (fabsf(fabsf(x - kr) - 0.5f) < 0x1p-16f || delta == 0.f) {
          if (delta == 0.f) {
            kf = (ve > 0.f) ? (float)(L - 1) : ((ve < 0.f) ? 0.f : (float)(L / 2));
          } else {
            // boundary b sits between levels b-1 and b at v = Delta (b - L/2), exact in float32
            const float bf = rintf(x + 0.5f);
            const int bi = (int)bf;
            kf = passes(ve, delta * (bf - (float)(L / 2)), bi) ? bf : bf - 1.f;
            kf = fminf(fmaxf(kf, 0.f), (float)(L - 1));
          }
        }
        code |= (uint32_t)kf << (VB * e);
      }
      if (p < parts) {
        const size_t row = row_s + t;
        if constexpr (VB == 4) {
          codes_out[row * WV + g * 4 + sub] = code;                     // 8 codes = one word
        } else {
          reinterpret_cast<uint16_t*>(codes_out + row * WV + g * 2)[sub] = (uint16_t)code;   // half a word
        }
        if (sub == 0) scale_out[row * G + g] = (uint16_t)dbits;
      }
    }
  }
}

// Per-block affine 8-bit keys, and group-32 min/max values at 2 or 4 bits (benchmark page,
// compression details): the same quantiser with L - 1 = 255, 3 or 15.  Boundaries
// m + a (q -+ 1/2) are exact in float64 for fp16 a and m, so a float32 estimate of
// rne((k - m)/a) is corrected by two exact float64 comparisons (ties to even).
__device__ __forceinline__ bool passes64(double v, double tau, int k) {
  return (k & 1) ? (v > tau) : (v >= tau);
}

template <int D, int DT, int QB = 8>
__global__ void __launch_bounds__(256)
encode_affine8_kernel(const uint16_t* __restrict__ x, int T, int slices, int dst_offset, int cap,
                      uint32_t* __restrict__ codes_out, uint32_t* __restrict__ aux_out) {
  static_assert(QB == 8 || QB == 5 || QB == 4 || QB == 2, "8/5/4/2-bit keys, 2/4-bit values");
  constexpr int G = D / 32;
  constexpr int TOP = (1 << QB) - 1;
  const int parts = T * (D / 8);
  for (int slice = blockIdx.y; slice < slices; slice += gridDim.y) {
    const uint16_t* xs = x + (size_t)slice * T * D;
    const size_t row_s = (size_t)slice * cap + dst_offset;
    float v[kGroupItems][8];
#pragma unroll
    for (int u = 0; u < kGroupItems; ++u) {
      const int p = (blockIdx.x * kGroupItems + u) * 256 + threadIdx.x;
      if (p < parts) {
        load8<DT>(xs + (size_t)p * 8, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kGroupItems; ++u) {
      const int p = (blockIdx.x * kGroupItems + u) * 256 + threadIdx.x;
      const int sub = p & 3, g = (p >> 2) % G, t = p / (D / 8);
      float lo = v[u][0], hi = v[u][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) { lo = fminf(lo, v[u][e]); hi = fmaxf(hi, v[u][e]); }
      lo = quad_min(lo);
      hi = quad_max(hi);
      // a = fp16((hi - lo)/255): the difference is exact in float64; the quotient's binary
      // fraction repeats with period 8 (1/255), far from an fp16 rounding tie, so rounding
      // the float64 product to float32 and then to fp16 gives the exactly rounded result.
      // (for 3 and 15 the float64 quotient rounds straight to fp16: its exact value is a
      // terminating binary fraction (then exact in float64) or at least 2^-53 relatively away
      // from an fp16 tie)
      const uint32_t abits = (QB == 8)
          ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)(((double)hi - (double)lo) * (1.0 / 255.0)))
          : f64_to_f16_rne(((double)hi - (double)lo) / (double)TOP);
      const uint32_t mbits = __builtin_bit_cast(uint16_t, (_Float16)lo);
      const double a = (double)f16_to_f32(abits);
      const double m = (double)f16_to_f32(mbits);
      const float inva = (a > 0.0) ? (float)(1.0 / a) : 0.f;
      const float mf = (float)m;
      uint32_t words[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ve = v[u][e];
        // x = (v - m)/a to within ~2^-14 absolute (|x| <= 256); only an x within 2^-11 of
        // a half-integer (a level boundary, exact ties included) needs the exact test
        const float x = (ve - mf) * inva;
        const float qr = rintf(x);
        float qf = fminf(fmaxf(qr, 0.f), (float)TOP);
        if (fabsf(fabsf(x - qr) - 0.5f) < 0x1p-11f && a > 0.0) {
          // boundary b between levels b-1 and b at m + a (b - 1/2), exact in float64
          const float bf = rintf(x + 0.5f);
          qf = passes64((double)ve, fma(a, (double)bf - 0.5, m), (int)bf) ? bf : bf - 1.f;
          qf = fminf(fmaxf(qf, 0.f), (float)TOP);
        }
        if constexpr (QB == 8) {
          words[e >> 2] |= (uint32_t)qf << (8 * (e & 3));
        } else if constexpr (QB == 5) {
          words[0] |= ((uint32_t)qf & 15u) << (4 * e);        // low nibble
          words[1] |= ((uint32_t)qf >> 4) << (8 * sub + e);    // fifth bit, at the group's bit 8 sub + e
        } else {
          words[0] |= (uint32_t)qf << (QB * e);
        }
      }
      if constexpr (QB == 5) words[1] |= xor_lanes_u32<1>(words[1]), words[1] |= xor_lanes_u32<2>(words[1]);
      if (p < parts) {
        const size_t row = row_s + t;
        if constexpr (QB == 8) {
          *reinterpret_cast<uint2*>(codes_out + row * (D / 4) + 8 * g + 2 * sub) = make_uint2(words[0], words[1]);
        } else if constexpr (QB == 5) {
          // row: D/8 words of low nibbles, then D/32 words of fifth bits
          constexpr int W5 = D / 8 + D / 32;
          codes_out[row * W5 + g * 4 + sub] = words[0];
          if (sub == 0) codes_out[row * W5 + D / 8 + g] = words[1];
        } else if constexpr (QB == 4) {
          codes_out[row * (D / 8) + g * 4 + sub] = words[0];                                  // 8 codes = one word
        } else {
          reinterpret_cast<uint16_t*>(codes_out + row * (D / 16) + g * 2)[sub] = (uint16_t)words[0];   // half a word
        }
        if (sub == 0) aux_out[row * G + g] = abits | (mbits << 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Launchers and the compiled set
// ---------------------------------------------------------------------------------
namespace {

int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int D, int KB, int DT, bool QJL>
int lm_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, encode_lm_kernel<D, KB, DT, QJL>, 64 * rot_waves<D>(), 0) !=
            hipSuccess ||
        b <= 0)
      b = 1;
    return b;
  }();
  return n;
}

template <int D, int KB, int DT, bool QJL>
hipError_t run_lm(const tq_layout& Lay, const tq_state& S, const void* x, int batch, int T, int dst,
                  const tq_cache& C, hipStream_t st, bool values) {
  const int slices = batch * Lay.n_kv_heads;
  const int mbps = ceil_div(T, 32);
  const long n_mb = (long)slices * mbps;
  if (n_mb > 0x7FFFFFFFL) return hipErrorInvalidValue;
  // persistent: as many groups as fit on the device at once (each stages the rotation
  // operands, and S for keys, in LDS once); every wave walks 32-token blocks with a stride
  // of the grid's wave count
  constexpr int NW = rot_waves<D>();
  const int grid = (int)std::min<long>((n_mb + NW - 1) / NW, (long)device_cus() * lm_blocks_per_cu<D, KB, DT, QJL>());
  if (values) {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(64 * NW), 0, st,
                       (const uint16_t*)x, T, mbps, (int)n_mb, dst, C.capacity, S.v_centroids, S.v_thresholds,
                       S.v_signs, (const uint16_t*)nullptr, (uint32_t*)C.v_codes, (uint32_t*)nullptr,
                       (uint32_t*)C.v_aux);
  } else {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(64 * NW), 0, st,
                       (const uint16_t*)x, T, mbps, (int)n_mb, dst, C.capacity, S.k_centroids, S.k_thresholds,
                       S.k_signs, QJL ? S.qjl : (const uint16_t*)nullptr, (uint32_t*)C.k_codes,
                       QJL ? (uint32_t*)C.k_signs : (uint32_t*)nullptr, (uint32_t*)C.k_aux);
  }
  return hipGetLastError();
}

// 16-bit keys (MLX page, V-only mode): the rows are stored as given, one 16-byte chunk per
// thread, from the contiguous input into slots [dst, dst + T) of each slice.
__global__ void __launch_bounds__(256) encode_copy16_kernel(const uint4* __restrict__ x, int T, long slices, int dst,
                                                           int cap, int row16, uint4* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= slices * T * row16) return;
  const int c = (int)(i % row16);
  const long rt = i / row16;
  const int t = (int)(rt % T);
  const long s = rt / T;
  out[((s * cap) + dst + t) * row16 + c] = x[i];
}

// Grid of the group kernels: x covers one slice's parts, y the slices (looped past 65535).
inline dim3 group_grid(int slices, int T, int D) {
  const long parts = (long)T * (D / 8);
  const long per_block = 256L * kGroupItems;
  return dim3((unsigned)((parts + per_block - 1) / per_block), (unsigned)std::min(slices, 65535));
}

template <int D, int VB, int DT>
hipError_t run_group(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                     hipStream_t st) {
  const int slices = batch * Lay.n_kv_heads;
  hipLaunchKernelGGL((encode_group_kernel<D, VB, DT>), group_grid(slices, T, D), dim3(256), 0, st,
                     (const uint16_t*)x, T, slices, dst, C.capacity, (uint32_t*)C.v_codes, (uint16_t*)C.v_aux);
  return hipGetLastError();
}

// group-32 min/max values: the affine quantiser at v_bits
template <int D, int QB, int DT>
hipError_t run_minmax_v(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                        hipStream_t st) {
  const int slices = batch * Lay.n_kv_heads;
  hipLaunchKernelGGL((encode_affine8_kernel<D, DT, QB>), group_grid(slices, T, D), dim3(256), 0, st,
                     (const uint16_t*)x, T, slices, dst, C.capacity, (uint32_t*)C.v_codes, (uint32_t*)C.v_aux);
  return hipGetLastError();
}

template <int D, int DT, int QB>
hipError_t run_affine(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                      hipStream_t st) {
  const int slices = batch * Lay.n_kv_heads;
  hipLaunchKernelGGL((encode_affine8_kernel<D, DT, QB>), group_grid(slices, T, D), dim3(256), 0, st,
                     (const uint16_t*)x, T, slices, dst, C.capacity, (uint32_t*)C.k_codes, (uint32_t*)C.k_aux);
  return hipGetLastError();
}

// Dispatch on (d, bits, dtype) to a compiled instantiation; returns false when none exists.
#define TQ_D_SWITCH(d, ...)                                   \
  switch (d) {                                                \
    case 64: { constexpr int DD = 64; __VA_ARGS__ } break;    \
    case 128: { constexpr int DD = 128; __VA_ARGS__ } break;  \
    case 256: { constexpr int DD = 256; __VA_ARGS__ } break;  \
    default: break;                                           \
  }
// the same with head_dim 512 (the generic group / affine / copy kernels)
#define TQ_D5_SWITCH(d, ...)                                  \
  switch (d) {                                                \
    case 64: { constexpr int DD = 64; __VA_ARGS__ } break;    \
    case 128: { constexpr int DD = 128; __VA_ARGS__ } break;  \
    case 256: { constexpr int DD = 256; __VA_ARGS__ } break;  \
    case 512: { constexpr int DD = 512; __VA_ARGS__ } break;  \
    default: break;                                           \
  }
#define TQ_DT_SWITCH(dt, ...)                                 \
  switch (dt) {                                               \
    case TQ_F16: { constexpr int DTT = TQ_F16; __VA_ARGS__ } break; \
    case TQ_BF16: { constexpr int DTT = TQ_BF16; __VA_ARGS__ } break; \
    default: break;                                           \
  }
#define TQ_B_SWITCH(b, ...)                                   \
  switch (b) {                                                \
    case 2: { constexpr int BB = 2; __VA_ARGS__ } break;      \
    case 3: { constexpr int BB = 3; __VA_ARGS__ } break;      \
    case 4: { constexpr int BB = 4; __VA_ARGS__ } break;      \
    default: break;                                           \
  }

}  // namespace

bool encode_k_compiled(const tq_layout& L) {
  const bool d_ok = L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256 || L.head_dim == 512;
  const bool dt_ok = L.in_dtype == TQ_F16 || L.in_dtype == TQ_BF16;
  if (L.k_kind == TQ_K_LM_QJL || L.k_kind == TQ_K_LM_MSE) return d_ok && dt_ok && L.k_bits >= 2 && L.k_bits <= 4;
  if (L.k_kind == TQ_K_AFFINE8)
    return d_ok && dt_ok && (L.k_bits == 8 || L.k_bits == 5 || L.k_bits == 4 || L.k_bits == 2);
  if (L.k_kind == TQ_K_F16) return d_ok && dt_ok && L.k_bits == 16;
  return false;
}

bool encode_v_compiled(const tq_layout& L) {
  const bool d_ok = L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256 || L.head_dim == 512;
  const bool dt_ok = L.in_dtype == TQ_F16 || L.in_dtype == TQ_BF16;
  if (L.v_kind == TQ_V_GROUP_SYM || L.v_kind == TQ_V_GROUP_ASYM) return d_ok && dt_ok && (L.v_bits == 2 || L.v_bits == 4);
  if (L.v_kind == TQ_V_LM_ROT) return d_ok && dt_ok && L.v_bits >= 2 && L.v_bits <= 4;
  return false;
}

hipError_t launch_encode_k(const tq_layout& L, const tq_state& S, const void* k, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st) {
  hipError_t err = hipErrorInvalidValue;
  if (L.head_dim == 512 && (L.k_kind == TQ_K_LM_QJL || L.k_kind == TQ_K_LM_MSE))
    return launch_encode_lm512(L, S, k, batch, n_tokens, dst_offset, C, st, false);
  if (L.k_kind == TQ_K_LM_QJL) {
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.k_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, true>(L, S, k, batch, n_tokens, dst_offset, C, st, false));)))
  } else if (L.k_kind == TQ_K_F16) {
    const long slices = (long)batch * L.n_kv_heads;
    const int row16 = L.head_dim / 8;
    const long chunks = slices * n_tokens * row16;
    hipLaunchKernelGGL(encode_copy16_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                       (const uint4*)k, n_tokens, slices, dst_offset, C.capacity, row16, (uint4*)C.k_codes);
    err = hipGetLastError();
  } else if (L.k_kind == TQ_K_LM_MSE) {
    // the rotated-LM kernel without the QJL stage (fp32 n in the aux plane), key state
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.k_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, false>(L, S, k, batch, n_tokens, dst_offset, C, st, false));)))
  } else {
    TQ_D5_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        switch (L.k_bits) {
          case 8: err = (run_affine<DD, DTT, 8>(L, k, batch, n_tokens, dst_offset, C, st)); break;
          case 5: err = (run_affine<DD, DTT, 5>(L, k, batch, n_tokens, dst_offset, C, st)); break;
          case 4: err = (run_affine<DD, DTT, 4>(L, k, batch, n_tokens, dst_offset, C, st)); break;
          case 2: err = (run_affine<DD, DTT, 2>(L, k, batch, n_tokens, dst_offset, C, st)); break;
          default: break;
        }))
  }
  return err;
}

hipError_t launch_encode_v(const tq_layout& L, const tq_state& S, const void* v, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st) {
  hipError_t err = hipErrorInvalidValue;
  if (L.head_dim == 512 && L.v_kind == TQ_V_LM_ROT)
    return launch_encode_lm512(L, S, v, batch, n_tokens, dst_offset, C, st, true);
  if (L.v_kind == TQ_V_GROUP_SYM) {
    TQ_D5_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        if (L.v_bits == 2) err = (run_group<DD, 2, DTT>(L, v, batch, n_tokens, dst_offset, C, st));
        else err = (run_group<DD, 4, DTT>(L, v, batch, n_tokens, dst_offset, C, st));))
  } else if (L.v_kind == TQ_V_GROUP_ASYM) {
    TQ_D5_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        if (L.v_bits == 2) err = (run_minmax_v<DD, 2, DTT>(L, v, batch, n_tokens, dst_offset, C, st));
        else err = (run_minmax_v<DD, 4, DTT>(L, v, batch, n_tokens, dst_offset, C, st));))
  } else {
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.v_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, false>(L, S, v, batch, n_tokens, dst_offset, C, st, true));)))
  }
  return err;
}

}  // namespace tq

// TurboQuant encode kernels for gfx950.
//
// Rotated Lloyd-Max encode (keys with the QJL sketch; rotated-LM values):
//   TurboQuant vLLM guide (kwkr.cn), section 2, steps 1-3 and 5; TurboQuant-MLX page
//   (pomoai.com), core technique items 1-3.
// Group-32 symmetric values: TurboQuant vLLM guide, section 2, step 4.
// Per-block affine 8-bit keys: vllm-metal TurboQuant guide (wmrh.cn), quantisation
//   principle table (per-block scale, no rotation).
//
// Work decomposition (rotated-LM kernel): a persistent work-group walks 64-token tiles
// of the (batch, kv-head) slices, prefetching the next tile's inputs into registers while
// it computes the current one.  Each vector is handled by P = d/32 consecutive lanes,
// each holding 32 coordinates: the first five butterfly stages of the Walsh-Hadamard
// transform stay inside a lane, the remaining log2(P) stages go across lanes with DPP
// exchanges.  Keys rotate in float64, so n, gamma and every decision match a float64
// evaluation; values rotate in float32 (only their decisions depend on it, and those
// move only within a float32 ulp of a threshold) with a float64 norm.  Codes are packed
// in registers and stored straight from the lanes.
// The QJL projection Z = R S^T (64 x d times d x d) is a dense contraction and runs on
// the fp16 matrix cores (v_mfma_f32_32x32x16_f16): S is stored at fp16 resolution, the
// float32 residual is split into fp16 hi + lo halves, and Z accumulates S*hi + S*lo in
// float32 -- every product exact, the residual carried to ~21 significant bits -- at two
// fp16 MFMAs instead of sixteen float32 ones per k-block of 16.  Each of the d/32 waves
// keeps its 32 rows of S in VGPRs for the whole kernel and reads the residual tile from
// LDS; each lane packs the sign bits of its accumulators.
#include <type_traits>

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------------
// Rotated Lloyd-Max encode.  QJL = true: keys (codes + QJL signs + fp16 (n, gamma));
// QJL = false: rotated values (codes + fp32 n).
// ---------------------------------------------------------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// Keys work on y, thresholds and centroids scaled by 2^12 (exact): the residual then
// enters the fp16 split as |r| 2^12 < 4096, where the low half of nearly every coordinate
// stays a normal fp16 number; decisions are unchanged, the projection's sign needs no
// rescaling and gamma = sqrt(sum r'^2) 2^-12 exactly.
constexpr double kKeyScale = 4096.0;

// Number of positive thresholds p_0 < p_1 < ... below |y| (binary search over the L/2
// magnitude cells of the symmetric codebook).
template <int KB>
__device__ __forceinline__ uint32_t magnitude_cell(float ay, const float (&p)[(1 << KB) / 2 - 1]) {
  if constexpr (KB == 2) {
    return ay > p[0] ? 1u : 0u;
  } else if constexpr (KB == 3) {
    const uint32_t c1 = ay > p[1] ? 1u : 0u;
    const uint32_t c2 = ay > (c1 ? p[2] : p[0]) ? 1u : 0u;
    return 2u * c1 + c2;
  } else {
    const uint32_t c1 = ay > p[3] ? 1u : 0u;
    const uint32_t c2 = ay > (c1 ? p[5] : p[1]) ? 1u : 0u;
    const float t3 = c1 ? (c2 ? p[6] : p[4]) : (c2 ? p[2] : p[0]);
    const uint32_t c3 = ay > t3 ? 1u : 0u;
    return 4u * c1 + 2u * c2 + c3;
  }
}

// Coordinates per lane (a vector spans d / coordinates lanes).  32: five butterfly stages
// inside a lane and a 64-VGPR float64 rotation state.  (16 per lane fits a third wave per
// SIMD but adds a cross-lane stage; measured no faster at d = 64 and slower at d = 128.)
template <int D>
constexpr int lm_coords() { return 32; }

template <int D, int KB, int DT, bool QJL>
__global__ void __launch_bounds__(64 * D / lm_coords<D>()) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
encode_lm_kernel(const uint16_t* __restrict__ x, int T, int tiles_per_slice, int n_tiles,
                 int dst_offset, int cap,
                 const float* __restrict__ cent, const float* __restrict__ thr,
                 const uint32_t* __restrict__ sign_mask, const uint16_t* __restrict__ S,
                 uint32_t* __restrict__ codes_out, uint32_t* __restrict__ signs_out,
                 uint32_t* __restrict__ aux_out) {
  // keys: float64 rotation and residual, so n, gamma and every decision agree with a
  // float64 evaluation; values: float32 rotation (only the decisions depend on it) and a
  // float64 norm
  using W = typename std::conditional<QJL, double, float>::type;
  constexpr int C = lm_coords<D>();        // coordinates per lane
  constexpr int P = D / C;                 // lanes per vector (= waves per group)
  constexpr int NT = 64 * P;               // threads: one 64-token tile
  constexpr int L = 1 << KB;
  constexpr int PER = (KB == 3) ? 10 : 32 / KB;   // codes per word
  constexpr int WK = (D + PER - 1) / PER;          // words per row
  constexpr int SW = D / 32;                       // sign words per row (= MFMA n-blocks)
  constexpr int RH = D + 8;                        // LDS row stride of the residual halves
  constexpr int NKB = D / 16;                      // MFMA k-blocks
  constexpr int LW = C * KB / 32;                  // whole stream words of a lane's codes
  constexpr int LSH = (C * KB) % 32;               // bits of a partial last stream word
  constexpr int MPW = 2 * SW / P;                  // projection m-blocks per wave
  static_assert(P >= 2 && P <= 16 && NT <= 1024, "lane split");
  static_assert(MPW == 1 || MPW == 2, "each wave takes one n-block and one or both m-blocks");

  __shared__ double s_cent[16];
  __shared__ __attribute__((aligned(16))) uint32_t s_xm[P * (C / 2)];
  __shared__ __attribute__((aligned(16))) _Float16 s_rhi[QJL ? kTile * RH : 8];
  __shared__ __attribute__((aligned(16))) _Float16 s_rlo[QJL ? kTile * RH : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int vec = tid / P;     // vector within the tile
  const int part = tid % P;    // which C coordinates

  constexpr double kPre = QJL ? kKeyScale : 1.0;
  if (tid < L) s_cent[tid] = (double)cent[tid] * kPre;
  if (tid < P * (C / 2)) {
    // sign flips as xor masks on pairs of packed 16-bit inputs: coordinate C p + 2 i at
    // bit 15, C p + 2 i + 1 at bit 31
    const int pp = tid / (C / 2), i = tid % (C / 2);
    const int j = C * pp + 2 * i;
    const uint32_t sm = sign_mask[j >> 5] >> (j & 31);
    s_xm[tid] = ((sm & 1u) << 15) | (((sm >> 1) & 1u) << 31);
  }
  // symmetric codebook: t[L/2-1] = 0 and t[L/2-1+i] = -t[L/2-1-i]; only the positive
  // thresholds are compared, against |y|
  float thp[L / 2 - 1];
#pragma unroll
  for (int i = 0; i < L / 2 - 1; ++i) thp[i] = thr[L / 2 + i] * (float)kPre;

  // QJL: wave w computes projection outputs 32 nb .. 32 nb + 31 (nb = w % SW) for the
  // 32-token m-blocks mb0 .. mb0 + MPW - 1 (mb0 = w / SW).  Its rows of S, fp16, as MFMA A
  // operands: lane l holds S[32 nb + l % 32][16 kb + 8 (l / 32) + i], i = 0..7.
  const int nb = wave % SW, mb0 = wave / SW;
  half8 sop[QJL ? NKB : 1];
  if constexpr (QJL) {
    const uint16_t* srow = S + (size_t)(32 * nb + (lane & 31)) * D + 8 * (lane >> 5);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sop[kb] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(srow + 16 * kb));
  }

  // 3-bit codes: word kw holds codes 10 kw .. 10 kw + 9, so words straddle the lanes'
  // C-code ranges.  A lane writes the words that start in its range, kw0 .. kw1, taking
  // the first bits of the next lane's stream where a word runs past its own.
  const int kw0 = (C * part + PER - 1) / PER;
  const int kw1 = min((C * part + C - 1) / PER, WK - 1);
  const int b0 = KB * (PER * kw0 - C * part);     // bit offset of word kw0 in the lane's stream

  auto load_tile = [&](int tile, uint4 (&raw)[C / 8]) {
    const int slice = tile / tiles_per_slice;
    const int t0 = (tile % tiles_per_slice) * kTile;
    if (tile < n_tiles && vec < min(kTile, T - t0)) {
      const uint4* src = reinterpret_cast<const uint4*>(x + ((size_t)slice * T + t0 + vec) * D + C * part);
#pragma unroll
      for (int i = 0; i < C / 8; ++i) raw[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < C / 8; ++i) raw[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  uint4 raw[C / 8];
  load_tile(blockIdx.x, raw);
  __syncthreads();

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int slice = tile / tiles_per_slice;
    const int t0 = (tile % tiles_per_slice) * kTile;
    const int nv = min(kTile, T - t0);
    const bool valid = vec < nv;
    const size_t row0 = (size_t)slice * cap + dst_offset + t0;

    uint32_t w[C / 2];
    {
      const uint32_t* rw = reinterpret_cast<const uint32_t*>(raw);
      const uint4* xm4 = reinterpret_cast<const uint4*>(&s_xm[part * (C / 2)]);
#pragma unroll
      for (int i = 0; i < C / 8; ++i) {
        const uint4 m = xm4[i];
        w[4 * i] = rw[4 * i] ^ m.x;
        w[4 * i + 1] = rw[4 * i + 1] ^ m.y;
        w[4 * i + 2] = rw[4 * i + 2] ^ m.z;
        w[4 * i + 3] = rw[4 * i + 3] ^ m.w;
      }
    }
    // the next tile's inputs stay in flight while this one is computed
    load_tile(tile + gridDim.x, raw);

    // ---- phase A: sign flip, norm (float64), Walsh-Hadamard ----------------------------
    W xv[C];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < C / 2; ++i) {
      const float a = in_to_f32<DT>(w[i] & 0xFFFFu);
      const float b = in_to_f32<DT>(w[i] >> 16);
      ss = fma((double)a, (double)a, ss);
      ss = fma((double)b, (double)b, ss);
      xv[2 * i] = (W)a;
      xv[2 * i + 1] = (W)b;
    }
#pragma unroll
    for (int h = 1; h < C; h <<= 1) {
#pragma unroll
      for (int e = 0; e < C; ++e) {
        if ((e & h) == 0) {
          const W a = xv[e], b = xv[e + h];
          xv[e] = a + b;
          xv[e + h] = a - b;
        }
      }
    }
    // butterflies across the P lanes of the vector (stride C m <-> lane xor m): the upper
    // lane of each pair keeps partner - own, the lower own + partner
#define TQ_XSTAGE(M)                                              \
    if constexpr (P > M) {                                        \
      const W sg = (part & M) ? W(-1) : W(1);                     \
      _Pragma("unroll") for (int e = 0; e < C; ++e) {             \
        const W o = xor_lanes<M>(xv[e]);                          \
        xv[e] = fma(xv[e], sg, o);                                \
      }                                                           \
    }
    TQ_XSTAGE(1)
    TQ_XSTAGE(2)
    TQ_XSTAGE(4)
    TQ_XSTAGE(8)
#undef TQ_XSTAGE
    ss = group_sum_dpp<P>(ss);
    const double n = sqrt(ss);
    const double scale64 = (n > 0.0) ? kPre / (sqrt((double)D) * n) : 0.0;
    const W scale = (W)scale64;

    // ---- Lloyd-Max decision, packed codes, residual -----------------------------------
    uint32_t cw[LW + 1];                // the lane's C codes as a KB-bit stream
#pragma unroll
    for (int i = 0; i <= LW; ++i) cw[i] = 0u;
    double gg = 0.0;
    // eight coordinates at a time (keeps the centroid reads and residuals of one chunk
    // in registers); keys write each chunk's residual halves to LDS:
    // hi = fp16(r) and lo = fp16(r - hi), both rounded toward zero -- the pair carries 21+
    // significant bits and every product of halves is exact in float32
#pragma unroll
    for (int c = 0; c < C / 8; ++c) {
      float rf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int e = 8 * c + k;
        const W y = xv[e] * scale;
        // idx = #{i : t_i < y} = L/2 + cnt for y > 0 and L/2 - 1 - cnt otherwise, with cnt
        // the number of positive thresholds below |y| (L/2 + cnt = cnt ^ L/2 and
        // L/2 - 1 - cnt = cnt ^ (L/2 - 1) for cnt < L/2); float32 |y| changes a decision
        // only where y lies within one float32 ulp of a threshold
        const float yf = (float)y;
        const uint32_t cnt = magnitude_cell<KB>(fabsf(yf), thp);
        const uint32_t idx = cnt ^ ((yf > 0.f) ? (uint32_t)(L / 2) : (uint32_t)(L / 2 - 1));
        const int bit = KB * e;
        cw[bit >> 5] |= idx << (bit & 31);
        if ((bit & 31) + KB > 32) cw[(bit >> 5) + 1] |= idx >> (32 - (bit & 31));
        if constexpr (QJL) {
          const double r = (double)y - s_cent[idx];
          gg = fma(r, r, gg);
          rf[k] = (float)r;
        }
      }
      if constexpr (QJL) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const auto h = __builtin_amdgcn_cvt_pkrtz(rf[2 * q], rf[2 * q + 1]);
          const auto l = __builtin_amdgcn_cvt_pkrtz(rf[2 * q] - (float)h[0], rf[2 * q + 1] - (float)h[1]);
          hw[q] = __builtin_bit_cast(uint32_t, h);
          lw[q] = __builtin_bit_cast(uint32_t, l);
        }
        *reinterpret_cast<uint4*>(&s_rhi[vec * RH + C * part + 8 * c]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&s_rlo[vec * RH + C * part + 8 * c]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (KB != 3) {
      // whole words: 16 / 8 codes per word, C codes per lane
      if (valid) {
        uint32_t* crow = codes_out + (row0 + vec) * WK + LW * part;
        if constexpr (LW == 1) {
          crow[0] = cw[0];
        } else if constexpr (LW == 2) {
          *reinterpret_cast<uint2*>(crow) = make_uint2(cw[0], cw[1]);
        } else {
          *reinterpret_cast<uint4*>(crow) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
        }
      }
    } else {
      // the lane's stream is C * 3 bits; append the next lane's first word behind it (the
      // last lane of a vector appends zeros), then word kw0 + j starts at bit b0 + 30 j
      const uint32_t nx0 = next_lane_u32(cw[0]);
      const uint32_t nx = (part == P - 1) ? 0u : nx0;
      constexpr int NS = LW + (LSH ? 2 : 1);
      uint32_t st[NS + 1];
#pragma unroll
      for (int i = 0; i < LW; ++i) st[i] = cw[i];
      if constexpr (LSH) {
        st[LW] = cw[LW] | (nx << LSH);
        st[LW + 1] = nx >> (32 - LSH);
      } else {
        st[LW] = nx;
      }
      st[NS] = 0u;
      constexpr int NJ = (C + PER - 1) / PER + 1;   // most words starting in a lane's range
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        // bit bb of the stream lies in stream word j (j = 0 always) or j - 1
        const int bb = b0 + 30 * j;
        const bool up = j == 0 || (bb >> 5) == j;
        const uint32_t lo = up ? st[j < NS ? j : NS] : st[j - 1];
        const uint32_t hi = up ? st[j + 1 <= NS ? j + 1 : NS] : st[j < NS ? j : NS];
        const uint32_t word = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(bb & 31)) & 0x3FFFFFFFu;
        if (valid && kw0 + j <= kw1) codes_out[(row0 + vec) * WK + kw0 + j] = word;
      }
    }
    if constexpr (QJL) {
      gg = group_sum_dpp<P>(gg);
      if (valid && part == 0)
        aux_out[row0 + vec] = f64_to_f16_rne(n) | (f64_to_f16_rne(sqrt(gg) * (1.0 / kKeyScale)) << 16);
    } else {
      if (valid && part == 0) aux_out[row0 + vec] = __float_as_uint((float)n);
    }

    // ---- phase B: QJL projection on the matrix cores, sign bits packed per lane --------
    // Z^T = S R^T for the wave's 32 outputs x 32 tokens: A = rows of S, B = residual rows.
    if constexpr (QJL) {
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        const int mb = mb0 + m;
        floatx16 acc = {};
        const _Float16* ah = &s_rhi[(32 * mb + (lane & 31)) * RH + 8 * (lane >> 5)];
        const _Float16* al = &s_rlo[(32 * mb + (lane & 31)) * RH + 8 * (lane >> 5)];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const half8 r_h = *reinterpret_cast<const half8*>(ah + 16 * kb);
          const half8 r_l = *reinterpret_cast<const half8*>(al + 16 * kb);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sop[kb], r_h, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sop[kb], r_l, acc, 0, 0, 0);
        }
        // acc register r of lane l: token 32 mb + l % 32, projection output
        // 32 nb + 8 (r / 4) + 4 (l / 32) + r % 4.  Stored bit = (z >= 0), from the sign bit.
        uint32_t neg = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) neg |= (__float_as_uint(acc[r]) >> 31) << (8 * (r >> 2) + (r & 3));
        const uint32_t half_bits = (~neg & 0x0F0F0F0Fu) << (4 * (lane >> 5));
        const uint32_t word = half_bits | (uint32_t)__shfl_xor((int)half_bits, 32);
        const int t = 32 * mb + lane;
        if (lane < 32 && t < nv) signs_out[(row0 + t) * SW + nb] = word;
      }
      __syncthreads();   // the residual tile is overwritten by the next tile
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
  static_assert(QB == 8 || QB == 4 || QB == 2, "8-bit keys, 2/4-bit values");
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
        if constexpr (QB == 8) words[e >> 2] |= (uint32_t)qf << (8 * (e & 3));
        else words[0] |= (uint32_t)qf << (QB * e);
      }
      if (p < parts) {
        const size_t row = row_s + t;
        if constexpr (QB == 8) {
          *reinterpret_cast<uint2*>(codes_out + row * (D / 4) + 8 * g + 2 * sub) = make_uint2(words[0], words[1]);
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, encode_lm_kernel<D, KB, DT, QJL>, 64 * D / lm_coords<D>(), 0) !=
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
  const int tps = ceil_div(T, kTile);
  const int n_tiles = slices * tps;
  // persistent: as many groups as fit on the device at once; each loads its rows of S
  // (keys) once and walks the tiles with a stride of the grid size
  const int grid = std::min(n_tiles, device_cus() * lm_blocks_per_cu<D, KB, DT, QJL>());
  if (values) {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(64 * D / lm_coords<D>()), 0, st,
                       (const uint16_t*)x, T, tps, n_tiles, dst, C.capacity, S.v_centroids, S.v_thresholds,
                       S.v_signs, (const uint16_t*)nullptr, (uint32_t*)C.v_codes, (uint32_t*)nullptr,
                       (uint32_t*)C.v_aux);
  } else {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(64 * D / lm_coords<D>()), 0, st,
                       (const uint16_t*)x, T, tps, n_tiles, dst, C.capacity, S.k_centroids, S.k_thresholds,
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

template <int D, int DT>
hipError_t run_affine(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                      hipStream_t st) {
  const int slices = batch * Lay.n_kv_heads;
  hipLaunchKernelGGL((encode_affine8_kernel<D, DT>), group_grid(slices, T, D), dim3(256), 0, st,
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
  const bool d_ok = L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256;
  const bool dt_ok = L.in_dtype == TQ_F16 || L.in_dtype == TQ_BF16;
  if (L.k_kind == TQ_K_LM_QJL || L.k_kind == TQ_K_LM_MSE) return d_ok && dt_ok && L.k_bits >= 2 && L.k_bits <= 4;
  if (L.k_kind == TQ_K_AFFINE8) return d_ok && dt_ok && L.k_bits == 8;
  if (L.k_kind == TQ_K_F16) return d_ok && dt_ok && L.k_bits == 16;
  return false;
}

bool encode_v_compiled(const tq_layout& L) {
  const bool d_ok = L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256;
  const bool dt_ok = L.in_dtype == TQ_F16 || L.in_dtype == TQ_BF16;
  if (L.v_kind == TQ_V_GROUP_SYM || L.v_kind == TQ_V_GROUP_ASYM) return d_ok && dt_ok && (L.v_bits == 2 || L.v_bits == 4);
  if (L.v_kind == TQ_V_LM_ROT) return d_ok && dt_ok && L.v_bits >= 2 && L.v_bits <= 4;
  return false;
}

hipError_t launch_encode_k(const tq_layout& L, const tq_state& S, const void* k, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st) {
  hipError_t err = hipErrorInvalidValue;
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
    TQ_D_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        err = (run_affine<DD, DTT>(L, k, batch, n_tokens, dst_offset, C, st));))
  }
  return err;
}

hipError_t launch_encode_v(const tq_layout& L, const tq_state& S, const void* v, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st) {
  hipError_t err = hipErrorInvalidValue;
  if (L.v_kind == TQ_V_GROUP_SYM) {
    TQ_D_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        if (L.v_bits == 2) err = (run_group<DD, 2, DTT>(L, v, batch, n_tokens, dst_offset, C, st));
        else err = (run_group<DD, 4, DTT>(L, v, batch, n_tokens, dst_offset, C, st));))
  } else if (L.v_kind == TQ_V_GROUP_ASYM) {
    TQ_D_SWITCH(L.head_dim, TQ_DT_SWITCH(L.in_dtype,
        if (L.v_bits == 2) err = (run_minmax_v<DD, 2, DTT>(L, v, batch, n_tokens, dst_offset, C, st));
        else err = (run_minmax_v<DD, 4, DTT>(L, v, batch, n_tokens, dst_offset, C, st));))
  } else {
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.v_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, false>(L, S, v, batch, n_tokens, dst_offset, C, st, true));)))
  }
  return err;
}

}  // namespace tq

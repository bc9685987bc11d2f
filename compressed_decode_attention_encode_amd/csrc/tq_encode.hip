// TurboQuant encode kernels for gfx950.
//
// Rotated Lloyd-Max encode (keys with the QJL sketch; rotated-LM values):
//   TurboQuant vLLM guide (kwkr.cn), section 2, steps 1-3 and 5; TurboQuant-MLX page
//   (pomoai.com), core technique items 1-3.
// Group-32 symmetric values: TurboQuant vLLM guide, section 2, step 4.
// Per-block affine 8-bit keys: vllm-metal TurboQuant guide (wmrh.cn), quantisation
//   principle table (per-block scale, no rotation).
//
// Work decomposition (rotated-LM kernel): a work-group owns a tile of 64 consecutive
// tokens of one (batch, kv-head) slice.  Each vector is handled by P = d/32 consecutive
// lanes, each holding 32 coordinates in float64: the first five butterfly stages of the
// Walsh-Hadamard transform stay inside a lane, the remaining log2(P) stages go across
// lanes with xor shuffles.  Norm, rotation, Lloyd-Max decision and residual are float64,
// so every decision matches a float64 evaluation up to the last bits.
// The QJL projection Z = R S^T (64 x d times d x d) is a dense contraction and runs on
// the matrix cores with v_mfma_f32_32x32x2f32: each of the d/32 waves keeps its 32 rows
// of S resident in VGPRs for the whole (persistent) kernel and streams the residual
// tile from LDS; the sign bits fall out of one ballot per accumulator register.
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------------
// Rotated Lloyd-Max encode.  QJL = true: keys (codes + QJL signs + fp16 (n, gamma));
// QJL = false: rotated values (codes + fp32 n).
// ---------------------------------------------------------------------------------
template <int D, int KB, int DT, bool QJL>
__global__ void __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
encode_lm_kernel(const uint16_t* __restrict__ x, int T, int tiles_per_slice, int n_tiles,
                 int dst_offset, int cap,
                 const float* __restrict__ cent, const float* __restrict__ thr,
                 const uint32_t* __restrict__ sign_mask, const float* __restrict__ S,
                 uint32_t* __restrict__ codes_out, uint32_t* __restrict__ signs_out,
                 uint32_t* __restrict__ aux_out) {
  constexpr int P = D / 32;            // lanes per vector
  constexpr int L = 1 << KB;
  constexpr int PER = (KB == 3) ? 10 : 32 / KB;   // codes per word
  constexpr int WK = (D + PER - 1) / PER;          // words per row
  constexpr int RS = D + 4;                        // LDS row stride of the residual tile (floats)
  constexpr int SW = D / 32;                       // sign words per row

  __shared__ double s_cent[16];
  __shared__ __attribute__((aligned(16))) uint32_t s_code[kTile * D / 4];   // code bytes
  __shared__ __attribute__((aligned(16))) float s_res[QJL ? kTile * RS : 4];
  __shared__ uint32_t s_sgn[QJL ? kTile * SW : 1];
  __shared__ uint32_t s_aux[kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int vec = tid / P;     // vector within the tile
  const int part = tid % P;    // which 32 coordinates

  if (tid < L) s_cent[tid] = (double)cent[tid];
  // symmetric codebook: t[L/2-1] = 0 and t[L/2-1+i] = -t[L/2-1-i]; only the positive
  // thresholds are compared, against |y|
  double thp[L / 2 - 1];
#pragma unroll
  for (int i = 0; i < L / 2 - 1; ++i) thp[i] = (double)thr[L / 2 + i];
  const uint32_t smask = sign_mask[part];

  // Rows of S this wave keeps for the whole kernel: lane holds S[32*wave + lane%32][2kk + lane/32].
  float sb[QJL ? D / 2 : 1];
  if constexpr (QJL) {
    const float* srow = S + (size_t)(32 * wave + (lane & 31)) * D + (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) sb[kk] = srow[2 * kk];
  }
  __syncthreads();

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int slice = tile / tiles_per_slice;
    const int t0 = (tile % tiles_per_slice) * kTile;
    const int nv = min(kTile, T - t0);
    const bool valid = vec < nv;

    // ---- phase A: load 32 coordinates, sign flip, Walsh-Hadamard in float64 -------------
    double xv[32];
    {
      uint4 raw[4] = {};
      if (valid) {
        const uint4* src = reinterpret_cast<const uint4*>(x + ((size_t)slice * T + t0 + vec) * D + 32 * part);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = src[i];
      }
      const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        uint32_t b = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        b ^= ((smask >> e) & 1u) << 15;   // s_j = -1 flips the sign bit
        xv[e] = (double)in_to_f32<DT>(b);
      }
    }
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) ss = fma(xv[e], xv[e], ss);
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        if ((e & h) == 0) {
          const double a = xv[e], b = xv[e + h];
          xv[e] = a + b;
          xv[e + h] = a - b;
        }
      }
    }
    // butterflies across the P lanes of the vector (stride 32*m <-> lane xor m)
#define TQ_XSTAGE(M)                                              \
    if constexpr (P > M) {                                        \
      const bool hi = (part & M) != 0;                            \
      _Pragma("unroll") for (int e = 0; e < 32; ++e) {            \
        const double o = xor_lanes<M>(xv[e]);                     \
        xv[e] = hi ? (o - xv[e]) : (xv[e] + o);                   \
      }                                                           \
    }
    TQ_XSTAGE(1)
    TQ_XSTAGE(2)
    TQ_XSTAGE(4)
    TQ_XSTAGE(8)
#undef TQ_XSTAGE
    ss = group_sum_dpp<P>(ss);
    const double n = sqrt(ss);
    const double scale = (n > 0.0) ? 1.0 / (sqrt((double)D) * n) : 0.0;

    // ---- Lloyd-Max decision and residual --------------------------------------------
    uint32_t packed[8];
    double gg = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const double y = xv[e] * scale;
      // idx = #{i : t_i < y}: with cnt = #{positive t_i < |y|} (sign bit of t_i - |y|) this is
      // L/2 + cnt for y > 0 and L/2 - 1 - cnt otherwise (equal except when |y| == t_i exactly)
      const double ay = fabs(y);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < L / 2 - 1; ++i) cnt += (uint32_t)((uint64_t)__double_as_longlong(thp[i] - ay) >> 63);
      const uint32_t pos = (uint32_t)((uint64_t)__double_as_longlong(0.0 - y) >> 63);   // y > 0
      const int idx = pos ? (int)(L / 2 + cnt) : (int)(L / 2 - 1 - cnt);
      if ((e & 3) == 0) packed[e >> 2] = 0;
      packed[e >> 2] |= (uint32_t)idx << (8 * (e & 3));
      if constexpr (QJL) {
        const double r = y - s_cent[idx];
        gg = fma(r, r, gg);
        xv[e] = r;
      }
    }
    {
      uint4* dst = reinterpret_cast<uint4*>(&s_code[(vec * D + 32 * part) / 4]);
      dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    }
    if constexpr (QJL) {
      gg = group_sum_dpp<P>(gg);
      float4* dst = reinterpret_cast<float4*>(&s_res[vec * RS + 32 * part]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[i] = make_float4((float)xv[4 * i], (float)xv[4 * i + 1], (float)xv[4 * i + 2], (float)xv[4 * i + 3]);
      if (part == 0) s_aux[vec] = f64_to_f16_rne(n) | (f64_to_f16_rne(sqrt(gg)) << 16);
    } else {
      if (part == 0) s_aux[vec] = __float_as_uint((float)n);
    }
    __syncthreads();

    // ---- phase B: QJL projection on the matrix cores, sign bits by ballot ----------------
    if constexpr (QJL) {
      floatx16 acc0 = {}, acc1 = {};
      const float* a0 = &s_res[(lane & 31) * RS + (lane >> 5)];
      const float* a1 = a0 + 32 * RS;
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[2 * kk], sb[kk], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[2 * kk], sb[kk], acc1, 0, 0, 0);
      }
      // acc register r of lane l holds row 8(r/4) + 4(l/32) + r%4, column l%32.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + (r & 3);
        const uint64_t b0 = __ballot(acc0[r] >= 0.0f);
        const uint64_t b1 = __ballot(acc1[r] >= 0.0f);
        if (lane == 0) {
          s_sgn[row * SW + wave] = (uint32_t)b0;
          s_sgn[(row + 4) * SW + wave] = (uint32_t)(b0 >> 32);
          s_sgn[(32 + row) * SW + wave] = (uint32_t)b1;
          s_sgn[(36 + row) * SW + wave] = (uint32_t)(b1 >> 32);
        }
      }
      __syncthreads();
    }

    // ---- phase C: pack and store the tile's rows (contiguous in every plane) -------------
    const size_t row0 = (size_t)slice * cap + dst_offset + t0;
    const uint8_t* cb = reinterpret_cast<const uint8_t*>(s_code);
    for (int q = tid; q < nv * WK; q += 2 * D) {
      const int v = q / WK, kw = q % WK;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = kw * PER + i;
        if (j < D) word |= (uint32_t)cb[v * D + j] << (KB * i);
      }
      codes_out[row0 * WK + q] = word;
    }
    if constexpr (QJL) {
      for (int q = tid; q < nv * SW; q += 2 * D) signs_out[row0 * SW + q] = s_sgn[q];
    }
    for (int q = tid; q < nv; q += 2 * D) aux_out[row0 + q] = s_aux[q];
    __syncthreads();
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

template <int D, int VB, int DT>
__global__ void __launch_bounds__(256)
encode_group_kernel(const uint16_t* __restrict__ x, int T, long n_parts, int dst_offset, int cap,
                    uint32_t* __restrict__ codes_out, uint16_t* __restrict__ scale_out) {
  constexpr int G = D / 32;
  constexpr int L = 1 << VB;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  // n_parts is a multiple of 4 and the grid a multiple of 64: whole quads are in or out
  const bool live = gid < n_parts;
  const long gq = live ? gid : n_parts - 4 + (gid & 3);
  const int sub = (int)(gq & 3);                 // which 8 elements of the group
  const int g = (int)((gq >> 2) % G);
  const long vt = (gq >> 2) / G;                 // slice * T + t
  const long slice = vt / T, t = vt % T;

  float v[8];
  load8<DT>(x + vt * D + 32 * g + 8 * sub, v);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = quad_max(amax);
  // Delta = fp16(2 amax / (L-1)): amax is an fp16/bf16 value, so the exact quotient has a
  // repeating binary fraction (k/3 or k/15) that stays >= 1/30 of an fp16 ulp away from a
  // rounding tie; the float32 product with the rounded reciprocal (error ~1e-7 relative)
  // therefore rounds to the same fp16 value as the exact quotient.
  const uint32_t dbits = __builtin_bit_cast(uint16_t, (_Float16)(2.0f * amax * (1.0f / (float)(L - 1))));
  const float delta = f16_to_f32(dbits);
  const float inv = (delta > 0.f) ? 1.0f / delta : 0.f;
  const float off = 0.5f * (float)(L - 1);
  uint32_t code = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int k;
    if (delta > 0.f) {
      k = (int)rintf(fmaf(v[e], inv, off));
      k = min(max(k, 0), L - 1);
      if (k > 0 && !passes(v[e], delta * (float)(k - L / 2), k)) {
        k -= 1;
      } else if (k < L - 1 && passes(v[e], delta * (float)(k + 1 - L / 2), k + 1)) {
        k += 1;
      }
    } else {
      k = (v[e] > 0.f) ? L - 1 : ((v[e] < 0.f) ? 0 : L / 2);
    }
    code |= (uint32_t)k << (VB * e);
  }
  if (!live) return;
  const size_t row = (size_t)slice * cap + dst_offset + t;
  constexpr int WV = D * VB / 32;
  if constexpr (VB == 4) {
    codes_out[row * WV + g * 4 + sub] = code;                     // 8 codes = one word
  } else {
    reinterpret_cast<uint16_t*>(codes_out + row * WV + g * 2)[sub] = (uint16_t)code;   // half a word
  }
  if (sub == 0) scale_out[row * G + g] = (uint16_t)dbits;
}

// Per-block affine 8-bit keys.  Boundaries m + a (q -+ 1/2) are exact in float64 for fp16
// a and m, so a float32 estimate of rne((k - m)/a) is corrected by two exact float64
// comparisons (ties to even).
__device__ __forceinline__ bool passes64(double v, double tau, int k) {
  return (k & 1) ? (v > tau) : (v >= tau);
}

template <int D, int DT>
__global__ void __launch_bounds__(256)
encode_affine8_kernel(const uint16_t* __restrict__ x, int T, long n_parts, int dst_offset, int cap,
                      uint32_t* __restrict__ codes_out, uint32_t* __restrict__ aux_out) {
  constexpr int G = D / 32;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = gid < n_parts;
  const long gq = live ? gid : n_parts - 4 + (gid & 3);
  const int sub = (int)(gq & 3);
  const int g = (int)((gq >> 2) % G);
  const long vt = (gq >> 2) / G;
  const long slice = vt / T, t = vt % T;

  float v[8];
  load8<DT>(x + vt * D + 32 * g + 8 * sub, v);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) { lo = fminf(lo, v[e]); hi = fmaxf(hi, v[e]); }
  lo = quad_min(lo);
  hi = quad_max(hi);
  // a = fp16((hi - lo)/255): the difference is exact in float64; the quotient's binary
  // fraction repeats with period 8 (1/255), far from an fp16 rounding tie, so rounding the
  // float64 product to float32 and then to fp16 gives the exactly rounded result.
  const uint32_t abits =
      __builtin_bit_cast(uint16_t, (_Float16)(float)(((double)hi - (double)lo) * (1.0 / 255.0)));
  const uint32_t mbits = __builtin_bit_cast(uint16_t, (_Float16)lo);
  const double a = (double)f16_to_f32(abits);
  const double m = (double)f16_to_f32(mbits);
  const float inva = (a > 0.0) ? (float)(1.0 / a) : 0.f;
  uint32_t words[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int q = 0;
    if (a > 0.0) {
      const double ve = (double)v[e];
      q = (int)rintf((float)(ve - m) * inva);
      q = min(max(q, 0), 255);
      if (q > 0 && !passes64(ve, fma(a, (double)q - 0.5, m), q)) {
        q -= 1;
      } else if (q < 255 && passes64(ve, fma(a, (double)q + 0.5, m), q + 1)) {
        q += 1;
      }
    }
    words[e >> 2] |= (uint32_t)q << (8 * (e & 3));
  }
  if (!live) return;
  const size_t row = (size_t)slice * cap + dst_offset + t;
  *reinterpret_cast<uint2*>(codes_out + row * (D / 4) + 8 * g + 2 * sub) = make_uint2(words[0], words[1]);
  if (sub == 0) aux_out[row * G + g] = abits | (mbits << 16);
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
hipError_t run_lm(const tq_layout& Lay, const tq_state& S, const void* x, int batch, int T, int dst,
                  const tq_cache& C, hipStream_t st, bool values) {
  const int slices = batch * Lay.n_kv_heads;
  const int tps = ceil_div(T, kTile);
  const int n_tiles = slices * tps;
  // persistent: enough groups for every CU, each keeps its rows of S in registers
  const int per_cu = (D <= 64) ? 6 : (D <= 128 ? 3 : 1);
  const int grid = std::min(n_tiles, device_cus() * per_cu);
  if (values) {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(2 * D), 0, st,
                       (const uint16_t*)x, T, tps, n_tiles, dst, C.capacity, S.v_centroids, S.v_thresholds,
                       S.v_signs, (const float*)nullptr, (uint32_t*)C.v_codes, (uint32_t*)nullptr,
                       (uint32_t*)C.v_aux);
  } else {
    hipLaunchKernelGGL((encode_lm_kernel<D, KB, DT, QJL>), dim3(grid), dim3(2 * D), 0, st,
                       (const uint16_t*)x, T, tps, n_tiles, dst, C.capacity, S.k_centroids, S.k_thresholds,
                       S.k_signs, S.qjl, (uint32_t*)C.k_codes, (uint32_t*)C.k_signs, (uint32_t*)C.k_aux);
  }
  return hipGetLastError();
}

template <int D, int VB, int DT>
hipError_t run_group(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                     hipStream_t st) {
  const long n = (long)batch * Lay.n_kv_heads * T * (D / 8);   // 4 lanes per 32-group
  hipLaunchKernelGGL((encode_group_kernel<D, VB, DT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, T, n, dst, C.capacity, (uint32_t*)C.v_codes, (uint16_t*)C.v_aux);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t run_affine(const tq_layout& Lay, const void* x, int batch, int T, int dst, const tq_cache& C,
                      hipStream_t st) {
  const long n = (long)batch * Lay.n_kv_heads * T * (D / 8);
  hipLaunchKernelGGL((encode_affine8_kernel<D, DT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, T, n, dst, C.capacity, (uint32_t*)C.k_codes, (uint32_t*)C.k_aux);
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
  if (L.k_kind == TQ_K_LM_QJL) return d_ok && dt_ok && L.k_bits >= 2 && L.k_bits <= 4;
  if (L.k_kind == TQ_K_AFFINE8) return d_ok && dt_ok && L.k_bits == 8;
  return false;
}

bool encode_v_compiled(const tq_layout& L) {
  const bool d_ok = L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256;
  const bool dt_ok = L.in_dtype == TQ_F16 || L.in_dtype == TQ_BF16;
  if (L.v_kind == TQ_V_GROUP_SYM) return d_ok && dt_ok && (L.v_bits == 2 || L.v_bits == 4);
  if (L.v_kind == TQ_V_LM_ROT) return d_ok && dt_ok && L.v_bits >= 2 && L.v_bits <= 4;
  return false;
}

hipError_t launch_encode_k(const tq_layout& L, const tq_state& S, const void* k, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st) {
  hipError_t err = hipErrorInvalidValue;
  if (L.k_kind == TQ_K_LM_QJL) {
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.k_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, true>(L, S, k, batch, n_tokens, dst_offset, C, st, false));)))
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
  } else {
    TQ_D_SWITCH(L.head_dim, TQ_B_SWITCH(L.v_bits, TQ_DT_SWITCH(L.in_dtype,
        err = (run_lm<DD, BB, DTT, false>(L, S, v, batch, n_tokens, dst_offset, C, st, true));)))
  }
  return err;
}

}  // namespace tq

// Materialisation: packed cache rows -> natural-domain fp16 / bf16 rows, the dequantise
// step ahead of a dense prefill (vllm-metal guide, prefill section: long prefills
// materialise the compressed history and run ordinary attention on it; vLLM guide,
// section 7: the hybrid path dequantises the whole history).  Per row, exactly the
// decoded vectors the decode attention uses:
//
//   affine-8 keys      k_j = m + a q_j                        (per 32-block a, m)
//   group values       v_j = Delta (idx_j - (L-1)/2)          (per 32-group Delta)
//   rotated LM values  v = n Pi^T c[idx]                      (vllm-metal guide, principle
//                                                              table; MLX page, core technique)
//   LM + QJL keys      k = n Pi^T (c[idx] + gamma sqrt(pi/2)/d S^T sigma)
//                                                             (vLLM guide, section 2)
//
// with Pi^T x = diag(s) H x / sqrt(d) (Sylvester Hadamard H, sign vector s).
//
// Affine keys and group values are elementwise: one thread per 8 dimensions of a row
// (one 16-byte store).  The LM kinds run per tile of 8192/d tokens (256 threads): the
// tile's codes are unpacked into bytes in LDS; for QJL keys the sign bits become fp16
// +-1 values in LDS and the tile's S^T sigma is a dense contraction (d x d by d x tile)
// on the fp16 matrix cores -- sigma and S are exact in fp16, the products exact in fp32
// -- with each wave's 32 columns of S^T held in VGPRs for the whole kernel; then every
// thread takes 32 coordinates of one token: centroids (+ the QJL term), the butterflies
// of H (5 stages inside the thread, the rest across the d/32 threads of the token by DPP
// exchanges), the scale n/sqrt(d), the sign flips, one rounding to the output type and
// four 16-byte stores.
#include <algorithm>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// (kernels outside an anonymous namespace, so that profiles name them)
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr float kSqrtHalfPiM = 1.2533141373155003f;   // sqrt(pi/2)

// float -> output storage bits, round to nearest even (NaN stays NaN).
template <int OUT>
__device__ __forceinline__ uint32_t to_out(float x) {
  if constexpr (OUT == TQ_F16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  } else {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
}

// ---------------------------------------------------------------------------------
// Elementwise kinds: thread = (row, 8-dimension octet).
//   KIND 0: affine-8 keys (codes: bytes; aux: fp16 (a, m) per 32-block)
//   KIND 1: group values  (codes: VB-bit; aux: fp16 Delta per 32-group)
//   KIND 2: 16-bit keys   (codes: the stored row, dtype VB = TQ_F16 / TQ_BF16; no aux)
//   KIND 3: min/max values (codes: VB-bit; aux: fp16 (a, m) per 32-group; v = m + a c)
// ---------------------------------------------------------------------------------
template <int D, int KIND, int VB, int OUT>
__global__ void __launch_bounds__(256) materialize_elem_kernel(const uint32_t* __restrict__ codes,
                                                               const uint32_t* __restrict__ aux, int slices,
                                                               int cap, int t0, int n, uint16_t* __restrict__ out) {
  constexpr int OCT = D / 8;
  const long item = (long)blockIdx.x * 256 + threadIdx.x;
  if (item >= (long)slices * n * OCT) return;
  const int o = (int)(item % OCT);
  const long rt = item / OCT;                // slice * n + token
  const int t = (int)(rt % n);
  const long slice = rt / n;
  const long row = slice * cap + t0 + t;
  const int g = o / 4;                       // 32-block / 32-group of the octet
  float v[8];
  if constexpr (KIND == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(codes + row * (D / 2) + 4 * o);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = in_to_f32<VB>(ww[e] & 0xFFFFu);
      v[2 * e + 1] = in_to_f32<VB>(ww[e] >> 16);
    }
  } else if constexpr (KIND == 0) {
    const uint2 w = *reinterpret_cast<const uint2*>(codes + row * (D / 4) + 2 * o);
    const uint32_t am = aux[row * (D / 32) + g];
    const float a = f16_to_f32(am & 0xFFFFu), m = f16_to_f32(am >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = fmaf(a, (float)((w.x >> (8 * e)) & 0xFFu), m);
      v[4 + e] = fmaf(a, (float)((w.y >> (8 * e)) & 0xFFu), m);
    }
  } else if constexpr (KIND == 4) {
    // 5-bit affine keys: low nibbles (D/8 words), then the fifth bits (D/32 words)
    constexpr int W5 = D / 8 + D / 32;
    const uint32_t w = codes[row * W5 + o];
    const uint32_t hb = codes[row * W5 + D / 8 + g] >> (8 * (o & 3));
    const uint32_t am = aux[row * (D / 32) + g];
    const float a = f16_to_f32(am & 0xFFFFu), m = f16_to_f32(am >> 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaf(a, (float)(((w >> (4 * e)) & 15u) | (((hb >> e) & 1u) << 4)), m);
  } else if constexpr (KIND == 3) {
    constexpr int L = 1 << VB;
    constexpr int WR = D * VB / 32;
    const int bit0 = 8 * VB * o;
    const uint32_t w = codes[row * WR + (bit0 >> 5)] >> (bit0 & 31);
    const uint32_t am = aux[row * (D / 32) + g];
    const float a = f16_to_f32(am & 0xFFFFu), m = f16_to_f32(am >> 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaf(a, (float)((w >> (VB * e)) & (L - 1)), m);
  } else {
    constexpr int L = 1 << VB;
    constexpr int WR = D * VB / 32;          // code words per row
    const int bit0 = 8 * VB * o;
    const uint32_t w = codes[row * WR + (bit0 >> 5)] >> (bit0 & 31);
    const uint32_t dw = aux[row * (D / 64) + (g >> 1)];
    const float dl = f16_to_f32((dw >> (16 * (g & 1))) & 0xFFFFu);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = dl * ((float)((w >> (VB * e)) & (L - 1)) - 0.5f * (float)(L - 1));
  }
  uint4 r;
  r.x = to_out<OUT>(v[0]) | (to_out<OUT>(v[1]) << 16);
  r.y = to_out<OUT>(v[2]) | (to_out<OUT>(v[3]) << 16);
  r.z = to_out<OUT>(v[4]) | (to_out<OUT>(v[5]) << 16);
  r.w = to_out<OUT>(v[6]) | (to_out<OUT>(v[7]) << 16);
  *reinterpret_cast<uint4*>(out + rt * D + 8 * o) = r;
}

// ---------------------------------------------------------------------------------
// LM kinds: per tile of T = 8192/d tokens, 256 threads, persistent over the tiles.
// ---------------------------------------------------------------------------------
struct LmArgs {
  const uint32_t* codes;     // LM code plane
  const uint32_t* signs;     // QJL sign plane (QJL keys)
  const uint32_t* aux;       // keys: fp16 (n, gamma); values: fp32 n
  const float* cent;         // codebook
  const uint32_t* rsign;     // rotation sign vector, d/32 words
  const uint16_t* S;         // QJL matrix, fp16, row-major (QJL keys)
  uint16_t* out;             // [slices][n][d]
  int slices, cap, t0, n, tiles_per_slice;
};

template <int D, int KB, bool QJL, int OUT>
__global__ void __launch_bounds__(256) materialize_lm_kernel(const LmArgs A) {
  constexpr int T = 8192 / D;                // tokens per tile (P threads each)
  constexpr int P = D / 32;                  // threads per token, 32 coordinates each
  constexpr int KPER = (KB == 3) ? 10 : 32 / KB;
  constexpr int WC = (D + KPER - 1) / KPER;  // code words per row
  constexpr int WS = D / 32;                 // sign words per row
  constexpr int SZ = D + 4;                  // LDS row stride of Z (floats)
  constexpr int SSG = D + 8;                 // LDS row stride of the +-1 signs (halves)
  constexpr int NJ = D / 32;                 // 32-column blocks of S^T
  constexpr int NM = T / 32;                 // 32-token blocks of the tile
  constexpr int PAIRS = NJ * NM / 4;         // (column block, token block) pairs per wave
  constexpr int NKB = D / 16;                // k-blocks of 16
  static_assert(T * P == 256, "one token part per thread");
  static_assert(NJ * NM % 4 == 0, "whole (column, token) block pairs per wave");
  __shared__ __attribute__((aligned(16))) uint8_t s_idx[T * D];
  __shared__ uint32_t s_aux[T];
  __shared__ float s_cent[16];
  __shared__ __attribute__((aligned(16))) _Float16 s_sg[QJL ? T * SSG : 8];
  __shared__ __attribute__((aligned(16))) float s_z[QJL ? T * SZ : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < (1 << KB)) s_cent[tid] = A.cent[tid];

  // The wave's column blocks of S^T as MFMA A operands, for the whole kernel: block jb,
  // k-block kb, lane l holds S^T[32 jb + l % 32][16 kb + 8 (l / 32) + i]
  //                           = S[16 kb + 8 (l / 32) + i][32 jb + l % 32], i = 0..7.
  // column blocks (wave + 4 pi) % NJ of a wave's pairs: one block unless NJ = 8
  constexpr int NJW = (QJL && NJ > 4) ? PAIRS : 1;
  half8 sop[NJW][QJL ? NKB : 1];
  if constexpr (QJL) {
#pragma unroll
    for (int u = 0; u < NJW; ++u) {
      const int jb = (wave + 4 * u) % NJ;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint16_t* col = A.S + (size_t)(16 * kb + 8 * (lane >> 5)) * D + 32 * jb + (lane & 31);
        half8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = __builtin_bit_cast(_Float16, col[(size_t)i * D]);
        sop[u][kb] = h;
      }
    }
  }
  // this thread's rotation signs for its 32 coordinates
  const int tl = tid / P, part = tid % P;
  const uint32_t rs = A.rsign[part];

  const int n_tiles = A.slices * A.tiles_per_slice;
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int slice = tile / A.tiles_per_slice;
    const int tb = A.t0 + (tile % A.tiles_per_slice) * T;
    const int nv = min(T, A.t0 + A.n - tb);
    const size_t row0 = (size_t)slice * A.cap + tb;
    // ---- stage: codes unpacked to bytes, aux, QJL signs as fp16 +-1 ------------------
    for (int i = tid; i < nv * WC; i += 256) {
      const int t = i / WC, w = i % WC;
      const uint32_t cw = A.codes[row0 * WC + i];
#pragma unroll
      for (int e = 0; e < KPER; ++e) {
        const int j = w * KPER + e;
        if (j < D) s_idx[t * D + j] = (uint8_t)((cw >> (KB * e)) & ((1u << KB) - 1u));
      }
    }
    for (int i = tid; i < nv; i += 256) s_aux[i] = A.aux[row0 + i];
    if constexpr (QJL) {
      for (int i = tid; i < T * WS; i += 256) {
        const int t = i / WS, w = i % WS;
        const uint32_t sw = (t < nv) ? A.signs[row0 * WS + i] : 0u;
        uint4* dst = reinterpret_cast<uint4*>(&s_sg[t * SSG + 32 * w]);
        // stored bit 1 <=> sigma = +1: fp16 -1 = 0xBC00, clearing bit 15 gives +1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t d4[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t x = sw >> (8 * q + 2 * k);
            d4[k] = 0xBC00BC00u ^ ((x & 1u) << 15) ^ (((x >> 1) & 1u) << 31);
          }
          dst[q] = make_uint4(d4[0], d4[1], d4[2], d4[3]);
        }
      }
    }
    __syncthreads();
    // ---- QJL term on the matrix cores: Z^T = S^T sigma^T per (column, token) block ----
    if constexpr (QJL) {
#pragma unroll
      for (int pi = 0; pi < PAIRS; ++pi) {
        const int pr = wave + 4 * pi;
        const int jb = pr % NJ, mb = pr / NJ;
        const int u = (NJW == 1) ? 0 : pi;
        floatx16 acc = {};
        const _Float16* bsrc = &s_sg[(32 * mb + (lane & 31)) * SSG + 8 * (lane >> 5)];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const half8 sg = *reinterpret_cast<const half8*>(bsrc + 16 * kb);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sop[u][kb], sg, acc, 0, 0, 0);
        }
        // acc register r of lane l: column 32 jb + 8 (r/4) + 4 (l/32) + r%4, token 32 mb + l%32
        float* zrow = &s_z[(32 * mb + (lane & 31)) * SZ + 32 * jb + 4 * (lane >> 5)];
#pragma unroll
        for (int r = 0; r < 16; ++r) zrow[8 * (r >> 2) + (r & 3)] = acc[r];
      }
      __syncthreads();
    }
    // ---- per thread: 32 coordinates of token tl, butterflies, scale, store -------------
    {
      const uint32_t ax = s_aux[tl];
      float scale, qc = 0.f;
      if constexpr (QJL) {
        scale = f16_to_f32(ax & 0xFFFFu);
        qc = f16_to_f32(ax >> 16) * (kSqrtHalfPiM / (float)D);
      } else {
        scale = __uint_as_float(ax);
      }
      scale *= rsqrtf((float)D);
      const uint4* ip = reinterpret_cast<const uint4*>(&s_idx[tl * D + 32 * part]);
      uint32_t cw[8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = ip[q];
        cw[4 * q] = v.x; cw[4 * q + 1] = v.y; cw[4 * q + 2] = v.z; cw[4 * q + 3] = v.w;
      }
      float x[32];
#pragma unroll
      // (masked: rows past the tile's last token hold stale bytes and are not stored)
      for (int c = 0; c < 32; ++c) x[c] = s_cent[(cw[c >> 2] >> (8 * (c & 3))) & ((1u << KB) - 1u)];
      if constexpr (QJL) {
        const float4* zp = reinterpret_cast<const float4*>(&s_z[tl * SZ + 32 * part]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 z = zp[q];
          x[4 * q] = fmaf(qc, z.x, x[4 * q]);
          x[4 * q + 1] = fmaf(qc, z.y, x[4 * q + 1]);
          x[4 * q + 2] = fmaf(qc, z.z, x[4 * q + 2]);
          x[4 * q + 3] = fmaf(qc, z.w, x[4 * q + 3]);
        }
      }
      // H x: strides 1..16 inside the thread, 32 m across the token's threads (lane ^ m)
#pragma unroll
      for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          if ((c & hs) == 0) {
            const float a = x[c], b = x[c + hs];
            x[c] = a + b;
            x[c + hs] = a - b;
          }
        }
      }
#pragma unroll
      for (int m = 1; m < P; m <<= 1) {
        const bool up = (part & m) != 0;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          float o;
          if constexpr (P >= 2) {
            if (m == 1) o = xor_lanes<1>(x[c]);
            else if (m == 2) o = xor_lanes<2>(x[c]);
            else o = xor_lanes<4>(x[c]);
          }
          x[c] = up ? (o - x[c]) : (x[c] + o);
        }
      }
      if (tl < nv) {
        uint32_t pk[16];
#pragma unroll
        for (int c = 0; c < 32; c += 2) {
          float a = x[c] * scale, b = x[c + 1] * scale;
          if ((rs >> c) & 1u) a = -a;
          if ((rs >> (c + 1)) & 1u) b = -b;
          pk[c >> 1] = to_out<OUT>(a) | (to_out<OUT>(b) << 16);
        }
        uint4* dst = reinterpret_cast<uint4*>(A.out + ((size_t)slice * A.n + (tb - A.t0) + tl) * D + 32 * part);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
      }
    }
    __syncthreads();   // the next tile overwrites the LDS tile
  }
}

namespace {

template <int D, int KB, bool QJL, int OUT>
hipError_t run_lm(const LmArgs& A, hipStream_t st) {
  static int blocks = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, materialize_lm_kernel<D, KB, QJL, OUT>, 256, 0) !=
            hipSuccess || b <= 0)
      b = 1;
    return b;
  }();
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  const long tiles = (long)A.slices * A.tiles_per_slice;
  const long grid = std::min<long>(tiles, (long)cus * blocks);
  hipLaunchKernelGGL((materialize_lm_kernel<D, KB, QJL, OUT>), dim3((unsigned)grid), dim3(256), 0, st, A);
  return hipGetLastError();
}

template <int D, int OUT>
hipError_t run_lm_bits(const LmArgs& A, int bits, bool qjl, hipStream_t st) {
  if (qjl) {
    switch (bits) {
      case 2: return run_lm<D, 2, true, OUT>(A, st);
      case 3: return run_lm<D, 3, true, OUT>(A, st);
      case 4: return run_lm<D, 4, true, OUT>(A, st);
    }
  } else {
    switch (bits) {
      case 2: return run_lm<D, 2, false, OUT>(A, st);
      case 3: return run_lm<D, 3, false, OUT>(A, st);
      case 4: return run_lm<D, 4, false, OUT>(A, st);
    }
  }
  return hipErrorInvalidValue;
}

template <int OUT>
hipError_t run_lm_any(const LmArgs& A, int d, int bits, bool qjl, hipStream_t st) {
  switch (d) {
    case 64: return run_lm_bits<64, OUT>(A, bits, qjl, st);
    case 128: return run_lm_bits<128, OUT>(A, bits, qjl, st);
    case 256: return run_lm_bits<256, OUT>(A, bits, qjl, st);
  }
  return hipErrorInvalidValue;
}

template <int D, int KIND, int VB, int OUT>
hipError_t run_elem(const uint32_t* codes, const uint32_t* aux, int slices, int cap, int t0, int n, uint16_t* out,
                    hipStream_t st) {
  const long items = (long)slices * n * (D / 8);
  const long grid = (items + 255) / 256;
  hipLaunchKernelGGL((materialize_elem_kernel<D, KIND, VB, OUT>), dim3((unsigned)grid), dim3(256), 0, st, codes, aux,
                     slices, cap, t0, n, out);
  return hipGetLastError();
}

template <int KIND, int VB, int OUT>
hipError_t run_elem_d(int d, const uint32_t* codes, const uint32_t* aux, int slices, int cap, int t0, int n,
                      uint16_t* out, hipStream_t st) {
  switch (d) {
    case 64: return run_elem<64, KIND, VB, OUT>(codes, aux, slices, cap, t0, n, out, st);
    case 128: return run_elem<128, KIND, VB, OUT>(codes, aux, slices, cap, t0, n, out, st);
    case 256: return run_elem<256, KIND, VB, OUT>(codes, aux, slices, cap, t0, n, out, st);
    case 512: return run_elem<512, KIND, VB, OUT>(codes, aux, slices, cap, t0, n, out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool materialize_compiled(const tq_layout& L) {
  return L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256 || L.head_dim == 512;
}

hipError_t launch_materialize_k(const tq_layout& L, const tq_state& S, const tq_cache& C, int t0, int n,
                                void* out, int out_dtype, hipStream_t st) {
  const int slices = C.batch * L.n_kv_heads;
  uint16_t* o = static_cast<uint16_t*>(out);
  if (L.k_kind == TQ_K_F16) {
    const uint32_t* codes = static_cast<const uint32_t*>(C.k_codes);
    if (L.in_dtype == TQ_BF16)
      return (out_dtype == TQ_BF16) ? run_elem_d<2, TQ_BF16, TQ_BF16>(L.head_dim, codes, nullptr, slices, C.capacity, t0, n, o, st)
                                    : run_elem_d<2, TQ_BF16, TQ_F16>(L.head_dim, codes, nullptr, slices, C.capacity, t0, n, o, st);
    return (out_dtype == TQ_BF16) ? run_elem_d<2, TQ_F16, TQ_BF16>(L.head_dim, codes, nullptr, slices, C.capacity, t0, n, o, st)
                                  : run_elem_d<2, TQ_F16, TQ_F16>(L.head_dim, codes, nullptr, slices, C.capacity, t0, n, o, st);
  }
  if (L.k_kind == TQ_K_AFFINE8) {
    // m + a q per element: bytes (kind 0), nibble + fifth-bit planes (kind 4), 4/2-bit words (kind 3,
    // the min/max value layout)
    const uint32_t* codes = static_cast<const uint32_t*>(C.k_codes);
    const uint32_t* aux = static_cast<const uint32_t*>(C.k_aux);
    const bool bf = out_dtype == TQ_BF16;
    switch (L.k_bits) {
      case 8: return bf ? run_elem_d<0, 8, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                        : run_elem_d<0, 8, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
      case 5: return bf ? run_elem_d<4, 5, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                        : run_elem_d<4, 5, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
      case 4: return bf ? run_elem_d<3, 4, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                        : run_elem_d<3, 4, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
      case 2: return bf ? run_elem_d<3, 2, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                        : run_elem_d<3, 2, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
      default: return hipErrorInvalidValue;
    }
  }
  const bool qjl = L.k_kind == TQ_K_LM_QJL;   // MSE-only keys: centroids and fp32 n alone
  if (L.head_dim == 512)
    return launch_materialize_lm512(static_cast<const uint32_t*>(C.k_codes),
                                    qjl ? static_cast<const uint32_t*>(C.k_signs) : nullptr,
                                    static_cast<const uint32_t*>(C.k_aux), S.k_centroids, S.k_signs,
                                    qjl ? S.qjl : nullptr, L.k_bits, qjl, slices, n, C.capacity, t0, o, out_dtype, st);
  LmArgs A{};
  A.codes = static_cast<const uint32_t*>(C.k_codes);
  A.signs = qjl ? static_cast<const uint32_t*>(C.k_signs) : nullptr;
  A.aux = static_cast<const uint32_t*>(C.k_aux);
  A.cent = S.k_centroids;
  A.rsign = S.k_signs;
  A.S = qjl ? S.qjl : nullptr;
  A.out = o;
  A.slices = slices;
  A.cap = C.capacity;
  A.t0 = t0;
  A.n = n;
  A.tiles_per_slice = ceil_div(n, 8192 / L.head_dim);
  return (out_dtype == TQ_BF16) ? run_lm_any<TQ_BF16>(A, L.head_dim, L.k_bits, qjl, st)
                                : run_lm_any<TQ_F16>(A, L.head_dim, L.k_bits, qjl, st);
}

hipError_t launch_materialize_v(const tq_layout& L, const tq_state& S, const tq_cache& C, int t0, int n,
                                void* out, int out_dtype, hipStream_t st) {
  const int slices = C.batch * L.n_kv_heads;
  uint16_t* o = static_cast<uint16_t*>(out);
  const uint32_t* codes = static_cast<const uint32_t*>(C.v_codes);
  const uint32_t* aux = static_cast<const uint32_t*>(C.v_aux);
  if (L.v_kind == TQ_V_GROUP_ASYM) {
    if (L.v_bits == 2)
      return (out_dtype == TQ_BF16) ? run_elem_d<3, 2, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                                    : run_elem_d<3, 2, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
    return (out_dtype == TQ_BF16) ? run_elem_d<3, 4, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                                  : run_elem_d<3, 4, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
  }
  if (L.v_kind == TQ_V_GROUP_SYM) {
    if (L.v_bits == 2)
      return (out_dtype == TQ_BF16) ? run_elem_d<1, 2, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                                    : run_elem_d<1, 2, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
    return (out_dtype == TQ_BF16) ? run_elem_d<1, 4, TQ_BF16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st)
                                  : run_elem_d<1, 4, TQ_F16>(L.head_dim, codes, aux, slices, C.capacity, t0, n, o, st);
  }
  if (L.head_dim == 512)
    return launch_materialize_lm512(codes, nullptr, aux, S.v_centroids, S.v_signs, nullptr, L.v_bits, false, slices, n,
                                    C.capacity, t0, o, out_dtype, st);
  LmArgs A{};
  A.codes = codes;
  A.signs = nullptr;
  A.aux = aux;
  A.cent = S.v_centroids;
  A.rsign = S.v_signs;
  A.S = nullptr;
  A.out = o;
  A.slices = slices;
  A.cap = C.capacity;
  A.t0 = t0;
  A.n = n;
  A.tiles_per_slice = ceil_div(n, 8192 / L.head_dim);
  return (out_dtype == TQ_BF16) ? run_lm_any<TQ_BF16>(A, L.head_dim, L.v_bits, false, st)
                                : run_lm_any<TQ_F16>(A, L.head_dim, L.v_bits, false, st);
}

}  // namespace tq

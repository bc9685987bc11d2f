// head_dim 512 (vllm-metal guide, support limits: the rotation kernel takes head dimensions
// 64, 128, 256 and 512).  The matrix-core encoder and the decode kernels hold a token's
// operands in registers and stage S in LDS, sized for d <= 256; at d = 512 (S alone is
// 512 KB) the work runs on plain vector-ALU kernels with one wavefront per token: lane l
// holds dimensions 8 l .. 8 l + 7, the Walsh-Hadamard transform takes three butterfly
// stages inside the lane and six across lanes, and a dot product over the head dimension is
// a lane sum followed by a wave reduction.  They are the correctness path for this geometry
// (no benchmark workload uses it), not a tuned one:
//   encode_lm512_kernel        rotated Lloyd-Max keys (+ QJL signs) and values
//                              (TurboQuant vLLM guide, section 2, steps 1-3 and 5)
//   decode512_kernel           split decode of every key / value kind on the packed cache;
//                              partials in the format of the other split kernels, so the
//                              same merge finishes them
//   materialize_lm512_kernel   k = n Pi^T (c[idx] + gamma sqrt(pi/2)/d S^T sigma), v = n Pi^T c[idx]
// The group / affine encoders and the elementwise materialiser are the generic templates.
#include <algorithm>

#include "tq_decode_main.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int kD5 = 512;
constexpr int kMaxRep512 = 8;

// Walsh-Hadamard transform (unnormalised, Sylvester order) of the 512 values a wave holds,
// lane l holding dimension 8 l + i in x[i].
__device__ __forceinline__ void wht512(float (&x)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = __shfl_xor(x[e], m);
      x[e] = (lane & m) ? o - x[e] : x[e] + o;
    }
  }
}

template <typename T>
__device__ __forceinline__ T wave_total(T v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Code words per row of 512 codes of b bits: ten 3-bit codes per word, bytes for 8 bits,
// a nibble plane plus a fifth-bit plane for 5 bits, 32/b codes per word otherwise.
template <int B>
constexpr int row_words() { return B == 3 ? (kD5 + 9) / 10 : kD5 * B / 32; }

// The 8 codes of dimensions 8 l .. 8 l + 7 from a packed row of 512 b-bit codes.
template <int B>
__device__ __forceinline__ void codes8(const uint32_t* __restrict__ row, int lane, uint32_t (&c)[8]) {
  if constexpr (B == 3) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * lane + i;
      c[i] = (row[j / 10] >> (3 * (j % 10))) & 7u;
    }
  } else if constexpr (B == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 2 * lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = (w.x >> (8 * i)) & 0xFFu;
      c[4 + i] = (w.y >> (8 * i)) & 0xFFu;
    }
  } else if constexpr (B == 4 || B == 5) {
    const uint32_t w = row[lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (w >> (4 * i)) & 15u;
    if constexpr (B == 5) {
      const uint32_t hb = row[kD5 / 8 + lane / 4] >> (8 * (lane & 3));
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] |= ((hb >> i) & 1u) << 4;
    }
  } else {
    const uint32_t w = row[lane >> 1] >> (16 * (lane & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (w >> (2 * i)) & 3u;
  }
}

// float -> fp16 / bf16 storage bits, round to nearest even (NaN stays NaN).
template <int OUT>
__device__ __forceinline__ uint32_t out16(float x) {
  if constexpr (OUT == TQ_F16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  } else {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
}

__device__ __forceinline__ void unpack8(const uint4& w, int bf16, float (&x)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bits16_to_f32(a[i] & 0xFFFFu, bf16);
    x[2 * i + 1] = bits16_to_f32(a[i] >> 16, bf16);
  }
}

// In-wave hand-off through LDS (lanes read what other lanes of the same wave wrote).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

// (kernels outside the anonymous namespace, so that profiles name them)

// ---------------------------------------------------------------------------------
// encode: one wave per token, 4 waves per work-group, persistent over the tokens
// ---------------------------------------------------------------------------------
// x: [slices][T][512] tokens (fp16 / bf16); token v = slice * T + t goes to row
// slice * cap + dst_offset + t of each plane.  Keys with QJL: codes, signs, aux = fp16
// (n, gamma); otherwise aux = fp32 n.
template <int KB, int DT, bool QJL>
__global__ void __launch_bounds__(256) encode_lm512_kernel(const uint16_t* __restrict__ x, int T, long n_vec,
                                                           int dst_offset, int cap, const float* __restrict__ cent,
                                                           const float* __restrict__ thr,
                                                           const uint32_t* __restrict__ sign_mask,
                                                           const uint16_t* __restrict__ S,
                                                           uint32_t* __restrict__ codes_out,
                                                           uint32_t* __restrict__ signs_out,
                                                           uint32_t* __restrict__ aux_out) {
  constexpr int L = 1 << KB;
  constexpr int WK = row_words<KB>();
  __shared__ __attribute__((aligned(16))) float s_r[4][kD5];   // a wave's residual (the QJL input)
  __shared__ uint32_t s_c[4][kD5];                             // a wave's codes (3-bit packing)
  __shared__ float s_cent[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < L) s_cent[threadIdx.x] = cent[threadIdx.x];
  float th[L - 1];
#pragma unroll
  for (int i = 0; i < L - 1; ++i) th[i] = thr[i];
  const uint32_t sm = (sign_mask[lane >> 2] >> (8 * (lane & 3))) & 0xFFu;
  __syncthreads();

  for (long v = (long)blockIdx.x * 4 + wave; v < n_vec; v += (long)gridDim.x * 4) {
    const long slice = v / T;
    const int t = (int)(v % T);
    const size_t row = (size_t)slice * cap + dst_offset + t;
    const uint4 raw = *reinterpret_cast<const uint4*>(x + (size_t)v * kD5 + 8 * lane);
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    float xv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[2 * i] = in_to_f32<DT>(rw[i] & 0xFFFFu);
      xv[2 * i + 1] = in_to_f32<DT>(rw[i] >> 16);
    }
    // n: float64 sum of the exact squares
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fma((double)xv[i], (double)xv[i], ss);
    ss = wave_total(ss);
    const double n = sqrt(ss);
    // a power of two keeps the float32 transform of large (bf16) or tiny tokens in range
    const float p2 = (n > 0x1p64) ? 0x1p-64f : ((n > 0.0 && n < 0x1p-64) ? 0x1p64f : 1.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xv[i] *= p2;
      if ((sm >> i) & 1u) xv[i] = -xv[i];
    }
    wht512(xv, lane);
    // y = Pi x / n = H diag(s) x / (sqrt(d) n)
    const float scale = (n > 0.0) ? (float)(1.0 / (sqrt((double)kD5) * n * (double)p2)) : 0.f;
    uint32_t idx[8];
    float gg = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = xv[i] * scale;
      uint32_t k = 0;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) k += (th[j] < y) ? 1u : 0u;   // idx = #{i : t_i < y}
      idx[i] = k;
      if constexpr (QJL) {
        const float r = y - s_cent[k];
        gg = fmaf(r, r, gg);
        s_r[wave][8 * lane + i] = r;
      }
    }
    if constexpr (KB == 4) {
      uint32_t w = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= idx[i] << (4 * i);
      codes_out[row * WK + lane] = w;
    } else if constexpr (KB == 2) {
      uint32_t w = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= idx[i] << (2 * i);
      const uint32_t o = (uint32_t)__shfl_xor((int)w, 1);
      if ((lane & 1) == 0) codes_out[row * WK + lane / 2] = w | (o << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_c[wave][8 * lane + i] = idx[i];
    }
    wave_sync();
    if constexpr (KB == 3) {
      if (lane < WK) {
        uint32_t w = 0u;
#pragma unroll
        for (int i = 0; i < 10; ++i) {
          const int j = 10 * lane + i;
          if (j < kD5) w |= s_c[wave][j] << (3 * i);
        }
        codes_out[row * WK + lane] = w;
      }
    }
    if constexpr (QJL) {
      // z_o = sum_j S[o][j] r_j for the lane's outputs o = 8 l + i; sign bit = (z_o >= 0)
      float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < kD5; j0 += 8) {
        const float4 ra = *reinterpret_cast<const float4*>(&s_r[wave][j0]);
        const float4 rb = *reinterpret_cast<const float4*>(&s_r[wave][j0 + 4]);
        const float r8[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 sw = *reinterpret_cast<const uint4*>(S + (size_t)(8 * lane + i) * kD5 + j0);
          const uint32_t s4[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            z[i] = fmaf(f16_to_f32(s4[k] & 0xFFFFu), r8[2 * k], z[i]);
            z[i] = fmaf(f16_to_f32(s4[k] >> 16), r8[2 * k + 1], z[i]);
          }
        }
      }
      uint32_t b = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) b |= (z[i] >= 0.f ? 1u : 0u) << i;
      b <<= 8 * (lane & 3);
      b |= (uint32_t)__shfl_xor((int)b, 1);
      b |= (uint32_t)__shfl_xor((int)b, 2);
      if ((lane & 3) == 0) signs_out[row * (kD5 / 32) + lane / 4] = b;
      const float g = sqrtf(wave_total(gg));
      if (lane == 0) {
        const uint32_t nb = f64_to_f16_rne(n);
        const uint32_t gb = __builtin_bit_cast(uint16_t, (_Float16)g);
        aux_out[row] = nb | (gb << 16);
      }
    } else {
      if (lane == 0) aux_out[row] = __float_as_uint((float)n);
    }
    wave_sync();   // the LDS rows are rewritten by the wave's next token
  }
}

// ---------------------------------------------------------------------------------
// decode: work-groups as in the other split kernels (compressed splits of A.chunk tokens,
// then one recent-buffer group per (batch, kv-head)); a wave takes one token per step and
// scores it against the n_rep <= 8 query heads of its kv-head
// ---------------------------------------------------------------------------------
template <int KK, int KB, int VK, int VB>
__global__ void __launch_bounds__(256) decode512_kernel(const DecodeArgs A) {
  constexpr int D = kD5;
  constexpr bool ROTK = KK == TQ_K_LM_QJL || KK == TQ_K_LM_MSE;
  constexpr bool QJL = KK == TQ_K_LM_QJL;
  __shared__ __attribute__((aligned(16))) float s_qa[kMaxRep512][D];   // queries for the scores
  __shared__ __attribute__((aligned(16))) float s_qb[kMaxRep512][D];   // projected queries (QJL)
  __shared__ __attribute__((aligned(16))) float s_acc[4][D];           // merge of the waves' sums
  __shared__ float s_kc[16], s_vc[16];
  __shared__ float s_ml[4][2][kMaxRep512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrep = A.Hq / A.Hkv;
  const int n_comp = A.nsplit * A.Hkv * A.batch;
  const bool recent = (int)blockIdx.x >= n_comp;
  int b, g, split;
  if (recent) {
    const int u = blockIdx.x - n_comp;
    b = u / A.Hkv;
    g = u % A.Hkv;
    split = A.nsplit;
  } else {
    split = blockIdx.x % A.nsplit;
    g = (blockIdx.x / A.nsplit) % A.Hkv;
    b = blockIdx.x / (A.nsplit * A.Hkv);
  }
  const size_t slice = (size_t)b * A.Hkv + g;
  const float sc = kLog2e * rsqrtf((float)D);   // scores in the log2 domain
  const bool rot = ROTK && !recent;
  if (tid < 16) {
    s_kc[tid] = (ROTK && tid < (1 << KB)) ? A.kcent[tid] : 0.f;
    s_vc[tid] = (VK == TQ_V_LM_ROT && tid < (1 << VB)) ? A.vcent[tid] : 0.f;
  }
  for (int i = tid; i < nrep * D; i += 256) {
    const int h = i / D, j = i % D;
    float q = bits16_to_f32(A.q[((size_t)b * A.Hq + g * nrep + h) * D + j], A.q_bf16);
    if (rot && ((A.ksign[j >> 5] >> (j & 31)) & 1u)) q = -q;
    s_qa[h][j] = rot ? q : q * sc;
  }
  __syncthreads();
  if (rot) {
    // q_r = Pi q = H diag(s) q / sqrt(d), times the score scale
    for (int hs = 1; hs < D; hs <<= 1) {
      for (int i = tid; i < nrep * (D / 2); i += 256) {
        const int h = i / (D / 2), p = i % (D / 2);
        const int lo = (p / hs) * 2 * hs + (p % hs);
        const float u = s_qa[h][lo], w = s_qa[h][lo + hs];
        s_qa[h][lo] = u + w;
        s_qa[h][lo + hs] = u - w;
      }
      __syncthreads();
    }
    for (int i = tid; i < nrep * D; i += 256) s_qa[i / D][i % D] *= rsqrtf((float)D) * sc;
    __syncthreads();
    if constexpr (QJL) {
      // q_s = S q_r, times sqrt(pi/2)/d (the estimator's scale)
      for (int o = tid; o < D; o += 256) {
        float acc[kMaxRep512];
#pragma unroll
        for (int h = 0; h < kMaxRep512; ++h) acc[h] = 0.f;
        const uint4* srow = reinterpret_cast<const uint4*>(A.S + (size_t)o * D);
        for (int j8 = 0; j8 < D / 8; ++j8) {
          const uint4 w = srow[j8];
          const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
          float sv[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            sv[2 * k] = f16_to_f32(w4[k] & 0xFFFFu);
            sv[2 * k + 1] = f16_to_f32(w4[k] >> 16);
          }
#pragma unroll
          for (int h = 0; h < kMaxRep512; ++h) {
            if (h < nrep) {
#pragma unroll
              for (int k = 0; k < 8; ++k) acc[h] = fmaf(sv[k], s_qa[h][8 * j8 + k], acc[h]);
            }
          }
        }
#pragma unroll
        for (int h = 0; h < kMaxRep512; ++h)
          if (h < nrep) s_qb[h][o] = acc[h] * (kSqrtHalfPi / (float)D);
      }
      __syncthreads();
    }
  }

  float m[kMaxRep512], l[kMaxRep512], acc[kMaxRep512][8];
#pragma unroll
  for (int h = 0; h < kMaxRep512; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }
  const int tb = recent ? 0 : split * A.chunk;
  const int te = recent ? A.n_recent : min(A.n_c, tb + A.chunk);
  const int grp = lane / 4;   // the lane's 32-dimension block
  for (int t = tb + wave; t < te; t += 4) {
    float kv[8], vv[8];
    float kn = 1.f, kg = 0.f;
    uint32_t sg = 0u;
    if (recent) {
      const size_t r = (slice * A.recent_cap + t) * D + 8 * lane;
      unpack8(*reinterpret_cast<const uint4*>(A.rk + r), A.recent_bf16, kv);
      unpack8(*reinterpret_cast<const uint4*>(A.rv + r), A.recent_bf16, vv);
    } else {
      const size_t row = slice * A.cap + t;
      if constexpr (KK == TQ_K_F16) {
        unpack8(*reinterpret_cast<const uint4*>(A.kc + row * (D / 2) + 4 * lane), A.q_bf16, kv);
      } else if constexpr (KK == TQ_K_AFFINE8) {
        uint32_t c[8];
        codes8<KB>(A.kc + row * row_words<KB>(), lane, c);
        const uint32_t am = A.ka[row * (D / 32) + grp];
        const float a = f16_to_f32(am & 0xFFFFu), mm = f16_to_f32(am >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[i] = fmaf(a, (float)c[i], mm);
      } else {
        uint32_t c[8];
        codes8<KB>(A.kc + row * row_words<KB>(), lane, c);
#pragma unroll
        for (int i = 0; i < 8; ++i) kv[i] = s_kc[c[i]];
        const uint32_t ax = A.ka[row];
        if constexpr (QJL) {
          kn = f16_to_f32(ax & 0xFFFFu);
          kg = f16_to_f32(ax >> 16);
          sg = (A.ks[row * (D / 32) + lane / 4] >> (8 * (lane & 3))) & 0xFFu;
        } else {
          kn = __uint_as_float(ax);
        }
      }
      uint32_t c[8];
      codes8<VB>(A.vc + row * row_words<VB>(), lane, c);
      if constexpr (VK == TQ_V_GROUP_SYM) {
        const float dl = f16_to_f32(reinterpret_cast<const uint16_t*>(A.va)[row * (D / 32) + grp]);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = dl * ((float)c[i] - 0.5f * (float)((1 << VB) - 1));
      } else if constexpr (VK == TQ_V_GROUP_ASYM) {
        const uint32_t am = A.va[row * (D / 32) + grp];
        const float a = f16_to_f32(am & 0xFFFFu), mm = f16_to_f32(am >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = fmaf(a, (float)c[i], mm);
      } else {
        const float vn = __uint_as_float(A.va[row]);   // rotated domain: n c[idx]
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = vn * s_vc[c[i]];
      }
    }
    // scores of the n_rep heads, online softmax, value sums
#pragma unroll
    for (int h = 0; h < kMaxRep512; ++h) {
      if (h < nrep) {
        const float4 qa0 = *reinterpret_cast<const float4*>(&s_qa[h][8 * lane]);
        const float4 qa1 = *reinterpret_cast<const float4*>(&s_qa[h][8 * lane + 4]);
        const float qa[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qa[i], kv[i], s);
        if (QJL && !recent) {
          const float4 qb0 = *reinterpret_cast<const float4*>(&s_qb[h][8 * lane]);
          const float4 qb1 = *reinterpret_cast<const float4*>(&s_qb[h][8 * lane + 4]);
          const float qb[8] = {qb0.x, qb0.y, qb0.z, qb0.w, qb1.x, qb1.y, qb1.z, qb1.w};
          float u = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) u += ((sg >> i) & 1u) ? qb[i] : -qb[i];
          s = fmaf(kg, u, s);
        }
        s = wave_total(s);
        if (rot) s *= kn;
        const float mn = fmaxf(m[h], s);
        const float al = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - mn);
        const float p = exp2f(s - mn);
        l[h] = fmaf(l[h], al, p);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(acc[h][i], al, p * vv[i]);
        m[h] = mn;
      }
    }
  }

  // merge the four waves: one partial (m, l, pad, pad, acc[d]) per head
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kMaxRep512; ++h) {
      s_ml[wave][0][h] = m[h];
      s_ml[wave][1][h] = l[h];
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < kMaxRep512; ++h) {
    if (h < nrep) {
      float mx = s_ml[0][0][h];
#pragma unroll
      for (int w = 1; w < 4; ++w) mx = fmaxf(mx, s_ml[w][0][h]);
      const float wsc = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - mx);
#pragma unroll
      for (int i = 0; i < 8; ++i) s_acc[wave][8 * lane + i] = acc[h][i] * wsc;
      __syncthreads();
      float* dst = partial_ptr<D>(A, b, g * nrep + h, split);
      for (int j = tid; j < D; j += 256) dst[4 + j] = s_acc[0][j] + s_acc[1][j] + s_acc[2][j] + s_acc[3][j];
      if (tid == 0) {
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mw = s_ml[w][0][h];
          lt += (mw == -INFINITY) ? 0.f : s_ml[w][1][h] * exp2f(mw - mx);
        }
        dst[0] = mx;
        dst[1] = lt;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// materialise (rotated kinds): one wave per token
// ---------------------------------------------------------------------------------
template <int KB, bool QJL, int OUT>
__global__ void __launch_bounds__(256) materialize_lm512_kernel(const uint32_t* __restrict__ codes,
                                                                const uint32_t* __restrict__ signs,
                                                                const uint32_t* __restrict__ aux,
                                                                const float* __restrict__ cent,
                                                                const uint32_t* __restrict__ rsign,
                                                                const uint16_t* __restrict__ S, long n_vec, int n,
                                                                int cap, int t0, uint16_t* __restrict__ out) {
  __shared__ float s_c[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < (1 << KB)) s_c[threadIdx.x] = cent[threadIdx.x];
  const uint32_t rs = (rsign[lane >> 2] >> (8 * (lane & 3))) & 0xFFu;
  __syncthreads();
  for (long v = (long)blockIdx.x * 4 + wave; v < n_vec; v += (long)gridDim.x * 4) {
    const long slice = v / n;
    const int t = (int)(v % n);
    const size_t row = (size_t)slice * cap + t0 + t;
    uint32_t c[8];
    codes8<KB>(codes + row * row_words<KB>(), lane, c);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = s_c[c[i]];
    float nrm;
    if constexpr (QJL) {
      const uint32_t ax = aux[row];
      nrm = f16_to_f32(ax & 0xFFFFu);
      const float gm = f16_to_f32(ax >> 16) * (kSqrtHalfPi / (float)kD5);
      // (S^T sigma)_j for the lane's j = 8 l + i: sum over the rows o of S[o][j] sigma_o
      float st[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < kD5 / 32; ++w) {
        const uint32_t sw = signs[row * (kD5 / 32) + w];
        for (int k = 0; k < 32; ++k) {
          const float sgn = ((sw >> k) & 1u) ? 1.f : -1.f;
          const uint4 s4 = *reinterpret_cast<const uint4*>(S + (size_t)(32 * w + k) * kD5 + 8 * lane);
          const uint32_t sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            st[2 * q] = fmaf(sgn, f16_to_f32(sv[q] & 0xFFFFu), st[2 * q]);
            st[2 * q + 1] = fmaf(sgn, f16_to_f32(sv[q] >> 16), st[2 * q + 1]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fmaf(gm, st[i], y[i]);
    } else {
      nrm = __uint_as_float(aux[row]);
    }
    // n Pi^T y = n diag(s) H y / sqrt(d)
    wht512(y, lane);
    const float f = nrm * rsqrtf((float)kD5);
    uint32_t o4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a = y[2 * q] * f, b2 = y[2 * q + 1] * f;
      if ((rs >> (2 * q)) & 1u) a = -a;
      if ((rs >> (2 * q + 1)) & 1u) b2 = -b2;
      o4[q] = out16<OUT>(a) | (out16<OUT>(b2) << 16);
    }
    *reinterpret_cast<uint4*>(out + (size_t)v * kD5 + 8 * lane) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
}

namespace {

int grid_for(long n_vec, int blocks_per_cu) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  const long want = (n_vec + 3) / 4;
  return (int)std::max<long>(1, std::min<long>(want, (long)cus * blocks_per_cu));
}

template <int KK, int KB, int VK, int VB>
hipError_t decode512_launch(dim3 grid, hipStream_t st, const DecodeArgs& A) {
  hipLaunchKernelGGL((decode512_kernel<KK, KB, VK, VB>), grid, dim3(256), 0, st, A);
  return hipGetLastError();
}

template <int KK, int KB, int VK, int VB>
int decode512_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode512_kernel<KK, KB, VK, VB>, 256, 0) != hipSuccess ||
        b <= 0)
      b = 1;
    return b;
  }();
  return n;
}

template <int KK, int KB, int VK, int VB>
MainKernel k512() {
  return MainKernel{&decode512_launch<KK, KB, VK, VB>, &decode512_blocks_per_cu<KK, KB, VK, VB>};
}

template <int KK, int KB>
MainKernel pick_v(int vk, int vb) {
  if (vk == TQ_V_GROUP_SYM) {
    if (vb == 2) return k512<KK, KB, TQ_V_GROUP_SYM, 2>();
    if (vb == 4) return k512<KK, KB, TQ_V_GROUP_SYM, 4>();
  } else if (vk == TQ_V_GROUP_ASYM) {
    if (vb == 2) return k512<KK, KB, TQ_V_GROUP_ASYM, 2>();
    if (vb == 4) return k512<KK, KB, TQ_V_GROUP_ASYM, 4>();
  } else if (vk == TQ_V_LM_ROT) {
    if (vb == 2) return k512<KK, KB, TQ_V_LM_ROT, 2>();
    if (vb == 3) return k512<KK, KB, TQ_V_LM_ROT, 3>();
    if (vb == 4) return k512<KK, KB, TQ_V_LM_ROT, 4>();
  }
  return MainKernel{nullptr, nullptr};
}

}  // namespace

// ---------------------------------------------------------------------------------
// entry points of the encode / decode / materialise dispatch
// ---------------------------------------------------------------------------------
hipError_t launch_encode_lm512(const tq_layout& L, const tq_state& S, const void* x, int batch, int T, int dst,
                               const tq_cache& C, hipStream_t st, bool values) {
  const long n_vec = (long)batch * L.n_kv_heads * T;
  if (n_vec <= 0) return hipSuccess;
  const int grid = grid_for(n_vec, 2);
  const bool qjl = !values && L.k_kind == TQ_K_LM_QJL;
  const int bits = values ? L.v_bits : L.k_bits;
  const float* cent = values ? S.v_centroids : S.k_centroids;
  const float* thr = values ? S.v_thresholds : S.k_thresholds;
  const uint32_t* sgn = values ? S.v_signs : S.k_signs;
  uint32_t* codes = static_cast<uint32_t*>(values ? C.v_codes : C.k_codes);
  uint32_t* aux = static_cast<uint32_t*>(values ? C.v_aux : C.k_aux);
  uint32_t* signs = qjl ? static_cast<uint32_t*>(C.k_signs) : nullptr;
  const uint16_t* qm = qjl ? S.qjl : nullptr;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const bool bf = L.in_dtype == TQ_BF16;
#define TQ_E512(KBV, Q)                                                                                          \
  do {                                                                                                           \
    if (bf)                                                                                                      \
      hipLaunchKernelGGL((encode_lm512_kernel<KBV, TQ_BF16, Q>), dim3(grid), dim3(256), 0, st, xs, T, n_vec, dst, \
                         C.capacity, cent, thr, sgn, qm, codes, signs, aux);                                     \
    else                                                                                                         \
      hipLaunchKernelGGL((encode_lm512_kernel<KBV, TQ_F16, Q>), dim3(grid), dim3(256), 0, st, xs, T, n_vec, dst,  \
                         C.capacity, cent, thr, sgn, qm, codes, signs, aux);                                     \
  } while (0)
  switch (bits) {
    case 2: if (qjl) TQ_E512(2, true); else TQ_E512(2, false); break;
    case 3: if (qjl) TQ_E512(3, true); else TQ_E512(3, false); break;
    case 4: if (qjl) TQ_E512(4, true); else TQ_E512(4, false); break;
    default: return hipErrorInvalidValue;
  }
#undef TQ_E512
  return hipGetLastError();
}

MainKernel find_main_d512(const tq_layout& L) {
  const int vk = L.v_kind, vb = L.v_bits;
  if (L.n_kv_heads <= 0 || L.n_q_heads % L.n_kv_heads || L.n_q_heads / L.n_kv_heads > kMaxRep512)
    return MainKernel{nullptr, nullptr};
  switch (L.k_kind) {
    case TQ_K_LM_QJL:
      if (L.k_bits == 2) return pick_v<TQ_K_LM_QJL, 2>(vk, vb);
      if (L.k_bits == 3) return pick_v<TQ_K_LM_QJL, 3>(vk, vb);
      if (L.k_bits == 4) return pick_v<TQ_K_LM_QJL, 4>(vk, vb);
      break;
    case TQ_K_LM_MSE:
      if (L.k_bits == 2) return pick_v<TQ_K_LM_MSE, 2>(vk, vb);
      if (L.k_bits == 3) return pick_v<TQ_K_LM_MSE, 3>(vk, vb);
      if (L.k_bits == 4) return pick_v<TQ_K_LM_MSE, 4>(vk, vb);
      break;
    case TQ_K_AFFINE8:
      if (L.k_bits == 8) return pick_v<TQ_K_AFFINE8, 8>(vk, vb);
      if (L.k_bits == 5) return pick_v<TQ_K_AFFINE8, 5>(vk, vb);
      if (L.k_bits == 4) return pick_v<TQ_K_AFFINE8, 4>(vk, vb);
      if (L.k_bits == 2) return pick_v<TQ_K_AFFINE8, 2>(vk, vb);
      break;
    case TQ_K_F16:
      if (L.k_bits == 16) return pick_v<TQ_K_F16, 16>(vk, vb);
      break;
    default:
      break;
  }
  return MainKernel{nullptr, nullptr};
}

hipError_t launch_materialize_lm512(const uint32_t* codes, const uint32_t* signs, const uint32_t* aux,
                                    const float* cent, const uint32_t* rsign, const uint16_t* S, int bits, bool qjl,
                                    long slices, int n, int cap, int t0, uint16_t* out, int out_dtype,
                                    hipStream_t st) {
  const long n_vec = slices * n;
  if (n_vec <= 0) return hipSuccess;
  const int grid = grid_for(n_vec, 2);
  const bool bf = out_dtype == TQ_BF16;
#define TQ_M512(KBV, Q)                                                                                             \
  do {                                                                                                              \
    if (bf)                                                                                                         \
      hipLaunchKernelGGL((materialize_lm512_kernel<KBV, Q, TQ_BF16>), dim3(grid), dim3(256), 0, st, codes, signs,   \
                         aux, cent, rsign, S, n_vec, n, cap, t0, out);                                              \
    else                                                                                                            \
      hipLaunchKernelGGL((materialize_lm512_kernel<KBV, Q, TQ_F16>), dim3(grid), dim3(256), 0, st, codes, signs,    \
                         aux, cent, rsign, S, n_vec, n, cap, t0, out);                                              \
  } while (0)
  switch (bits) {
    case 2: if (qjl) TQ_M512(2, true); else TQ_M512(2, false); break;
    case 3: if (qjl) TQ_M512(3, true); else TQ_M512(3, false); break;
    case 4: if (qjl) TQ_M512(4, true); else TQ_M512(4, false); break;
    default: return hipErrorInvalidValue;
  }
#undef TQ_M512
  return hipGetLastError();
}

}  // namespace tq

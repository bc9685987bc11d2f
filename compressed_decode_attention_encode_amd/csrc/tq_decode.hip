// Decode attention: query preparation, split combination (+ exact recent buffer and the
// single inverse butterfly), the split plan and the launch sequence.
//
//   prep     (TurboQuant-MLX page, GPU kernel optimisation section, pre-rotated query):
//            once per (batch, q-head): q_r = Pi q and q_s = S q_r for LM + QJL keys, or
//            32-block sums of q for affine keys; scales 1/sqrt(d), log2(e) and the QJL
//            factor sqrt(pi/2)/d are folded in here.
//   main     tq_decode_main.h
//   combine  log-sum-exp merge of the splits (news page, oMLX section: a two-pass flash
//            decode); the exact recent tokens (TurboQuant vLLM guide, section 5; benchmark
//            page, buffering strategy) join under the same normaliser; rotated-domain value
//            sums are rotated back once (TurboQuant-MLX page, butterfly pulled out).
#include "tq_decode_main.h"

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------
// prep: qa (scores against codes), qb (QJL), qn (natural domain, recent tokens), G (affine)
// ---------------------------------------------------------------------------------
template <int D, int KK, int DT>
__global__ void __launch_bounds__(256)
decode_prep_kernel(const uint16_t* __restrict__ q, const uint32_t* __restrict__ sign_mask,
                   const float* __restrict__ S, float* __restrict__ qprep, int Hq) {
  constexpr int QF = 4 * D;
  __shared__ float s_x[D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int j = threadIdx.x;
  const float scale = kLog2e * rsqrtf((float)D);
  float* out = qprep + (size_t)(b * Hq + h) * QF;
  float qj = 0.f;
  if (j < D) {
    qj = in_to_f32<DT>(q[(size_t)(b * Hq + h) * D + j]);
    out[2 * D + j] = qj * scale;   // qn
  }
  if constexpr (KK == TQ_K_LM_QJL) {
    if (j < D) s_x[j] = ((sign_mask[j >> 5] >> (j & 31)) & 1u) ? -qj : qj;
    __syncthreads();
    // in-place fast Walsh-Hadamard transform, one butterfly per thread per stage
    for (int hs = 1; hs < D; hs <<= 1) {
      float a = 0.f, c = 0.f;
      int lo = 0;
      if (j < D / 2) {
        lo = (j / hs) * 2 * hs + (j % hs);
        a = s_x[lo];
        c = s_x[lo + hs];
      }
      __syncthreads();
      if (j < D / 2) {
        s_x[lo] = a + c;
        s_x[lo + hs] = a - c;
      }
      __syncthreads();
    }
    const float rs = rsqrtf((float)D);
    if (j < D) out[j] = s_x[j] * rs * scale;   // qa = Pi q
    // q_s = S q_r; thread i takes row i of S
    if (j < D) {
      const float* srow = S + (size_t)j * D;
      float acc = 0.f;
      for (int k = 0; k < D; ++k) acc = fmaf(srow[k], s_x[k], acc);
      const float qjl = 1.2533141373155003f / (float)D;   // sqrt(pi/2)/d
      out[D + j] = acc * rs * scale * qjl;
    }
  } else {
    if (j < D) out[j] = qj * scale;
    if (j < D) s_x[j] = qj * scale;
    __syncthreads();
    if (j < D / 32) {
      float gsum = 0.f;
      for (int k = 0; k < 32; ++k) gsum += s_x[32 * j + k];
      out[3 * D + j] = gsum;
    }
  }
}

// ---------------------------------------------------------------------------------
// combine: merge splits, fold in the recent tokens, inverse rotation, normalise
// ---------------------------------------------------------------------------------
template <int D, int VK, int RDT>
__global__ void __launch_bounds__(256)
decode_combine_kernel(const float* __restrict__ part, int nsplit, const float* __restrict__ qprep,
                      const uint16_t* __restrict__ rk, const uint16_t* __restrict__ rv, int n_recent,
                      int recent_cap, const uint32_t* __restrict__ vsign_mask, float* __restrict__ out,
                      int Hq, int Hkv) {
  constexpr int QF = 4 * D;
  constexpr int PS = D + 4;
  __shared__ float s_red[256];
  __shared__ float s_w[256];          // split weights, then recent weights
  __shared__ float s_qn[D];
  __shared__ float s_acc[D];
  __shared__ float s_pr[kMaxRecent];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int g = h / (Hq / Hkv);
  const float* qp = qprep + (size_t)(b * Hq + h) * QF;
  const float* pp = part + (size_t)(b * Hq + h) * nsplit * PS;
  if (tid < D) s_qn[tid] = qp[2 * D + tid];

  // max over split maxima
  float mloc = -INFINITY;
  for (int s = tid; s < nsplit; s += blockDim.x) mloc = fmaxf(mloc, pp[(size_t)s * PS]);
  // recent scores
  __syncthreads();
  const size_t rbase = ((size_t)b * Hkv + g) * recent_cap;
  float sr = -INFINITY;
  if (tid < n_recent) {
    const uint16_t* kr = rk + (rbase + tid) * D;
    float a = 0.f;
    for (int k = 0; k < D; ++k) a = fmaf(s_qn[k], in_to_f32<RDT>(kr[k]), a);
    sr = a;
    mloc = fmaxf(mloc, a);
  }
  s_red[tid] = mloc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
    __syncthreads();
  }
  const float M = s_red[0];
  __syncthreads();

  // normaliser
  float lloc = 0.f;
  for (int s = tid; s < nsplit; s += blockDim.x) {
    const float m = pp[(size_t)s * PS];
    lloc += (m == -INFINITY) ? 0.f : pp[(size_t)s * PS + 1] * exp2f(m - M);
  }
  if (tid < n_recent) {
    const float pr = exp2f(sr - M);
    s_pr[tid] = pr;
    lloc += pr;
  }
  s_red[tid] = lloc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] += s_red[tid + w];
    __syncthreads();
  }
  const float l = s_red[0];

  // value sums: compressed part (rotated domain for LM values), recent part (natural)
  float main_j = 0.f, rec_j = 0.f;
  if (tid < D) {
    for (int s = 0; s < nsplit; ++s) {
      const float m = pp[(size_t)s * PS];
      if (m != -INFINITY) main_j = fmaf(pp[(size_t)s * PS + 4 + tid], exp2f(m - M), main_j);
    }
    const uint16_t* vr = rv + rbase * D + tid;
    for (int r = 0; r < n_recent; ++r) rec_j = fmaf(s_pr[r], in_to_f32<RDT>(vr[(size_t)r * D]), rec_j);
  }
  if constexpr (VK == TQ_V_LM_ROT) {
    // Pi^T acc = diag(s) H acc / sqrt(d): one fast transform of the summed vector
    if (tid < D) s_acc[tid] = main_j;
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
      float a = 0.f, c = 0.f;
      int lo = 0;
      if (tid < D / 2) {
        lo = (tid / hs) * 2 * hs + (tid % hs);
        a = s_acc[lo];
        c = s_acc[lo + hs];
      }
      __syncthreads();
      if (tid < D / 2) {
        s_acc[lo] = a + c;
        s_acc[lo + hs] = a - c;
      }
      __syncthreads();
    }
    if (tid < D) {
      const float hv = s_acc[tid] * rsqrtf((float)D);
      main_j = ((vsign_mask[tid >> 5] >> (tid & 31)) & 1u) ? -hv : hv;
    }
  }
  if (tid < D) out[(size_t)(b * Hq + h) * D + tid] = (main_j + rec_j) / l;
}

// ---------------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------------
DecodePlan plan_decode(const tq_layout& L, int batch, int n_c) {
  DecodePlan p{};
  const int d = L.head_dim;
  const long units = (long)batch * L.n_kv_heads;
  const int tiles = ceil_div(n_c, kTile);
  if (n_c <= 0) {
    p.n_splits = 0;
    p.chunk = 0;
  } else {
    int want = ceil_div(kTargetDecodeGroups, units);
    want = std::max(1, std::min(want, ceil_div(tiles, 4)));   // >= 4 tiles (one per wave) per split
    const int tiles_per = ceil_div(tiles, want);
    p.chunk = tiles_per * kTile;
    p.n_splits = ceil_div(tiles, tiles_per);
  }
  p.q_floats = 4 * (size_t)d;
  p.part_stride = (size_t)d + 4;
  p.ws_bytes = sizeof(float) * ((size_t)batch * L.n_q_heads * p.q_floats +
                                (size_t)batch * L.n_q_heads * p.n_splits * p.part_stride);
  return p;
}

size_t decode_ws_bound(const tq_layout& L, int batch, int max_c) {
  // n_splits of any n_c <= max_c is at most min(ceil(target/units), tiles(max_c))
  const long units = (long)batch * L.n_kv_heads;
  const int max_splits = std::max(0, std::min(ceil_div(kTargetDecodeGroups, units), ceil_div(std::max(max_c, 0), kTile)));
  const size_t d = L.head_dim;
  return sizeof(float) * ((size_t)batch * L.n_q_heads * 4 * d + (size_t)batch * L.n_q_heads * max_splits * (d + 4));
}

namespace {

MainLaunch find_main(const tq_layout& L) {
  const int nrep = L.n_q_heads / L.n_kv_heads;
  const int d = L.head_dim, vk = L.v_kind, vb = L.v_bits;
#define TQ_BY_D(name)                                                   \
  switch (d) {                                                          \
    case 64: return name##_d64(nrep, vk, vb);                           \
    case 128: return name##_d128(nrep, vk, vb);                         \
    case 256: return name##_d256(nrep, vk, vb);                         \
    default: return nullptr;                                            \
  }
  if (L.k_kind == TQ_K_LM_QJL) {
    switch (L.k_bits) {
      case 2: TQ_BY_D(find_main_lm2)
      case 3: TQ_BY_D(find_main_lm3)
      case 4: TQ_BY_D(find_main_lm4)
      default: return nullptr;
    }
  }
  if (L.k_kind == TQ_K_AFFINE8 && L.k_bits == 8) { TQ_BY_D(find_main_aff8) }
#undef TQ_BY_D
  return nullptr;
}

template <int D, int KK>
hipError_t run_prep(const tq_layout& L, const tq_state& S, const void* q, float* qprep, int batch, hipStream_t st) {
  if (L.in_dtype == TQ_F16)
    hipLaunchKernelGGL((decode_prep_kernel<D, KK, TQ_F16>), dim3(L.n_q_heads, batch), dim3(256), 0, st,
                       (const uint16_t*)q, S.k_signs, S.qjl, qprep, L.n_q_heads);
  else
    hipLaunchKernelGGL((decode_prep_kernel<D, KK, TQ_BF16>), dim3(L.n_q_heads, batch), dim3(256), 0, st,
                       (const uint16_t*)q, S.k_signs, S.qjl, qprep, L.n_q_heads);
  return hipGetLastError();
}

template <int D, int VK>
hipError_t run_combine(const tq_layout& L, const tq_state& S, const float* part, int nsplit, const float* qprep,
                       const void* rk, const void* rv, int n_recent, int rcap, float* out, int batch,
                       hipStream_t st) {
  if (L.recent_dtype == TQ_F16)
    hipLaunchKernelGGL((decode_combine_kernel<D, VK, TQ_F16>), dim3(L.n_q_heads, batch), dim3(256), 0, st, part,
                       nsplit, qprep, (const uint16_t*)rk, (const uint16_t*)rv, n_recent, rcap, S.v_signs, out,
                       L.n_q_heads, L.n_kv_heads);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, VK, TQ_BF16>), dim3(L.n_q_heads, batch), dim3(256), 0, st, part,
                       nsplit, qprep, (const uint16_t*)rk, (const uint16_t*)rv, n_recent, rcap, S.v_signs, out,
                       L.n_q_heads, L.n_kv_heads);
  return hipGetLastError();
}

template <int D>
hipError_t run_decode_d(const tq_layout& L, const tq_state& S, const void* q, const tq_cache& C, int n_c,
                        const void* rk, const void* rv, int n_recent, int rcap, float* out, void* ws,
                        const DecodePlan& plan, hipStream_t st) {
  const int batch = C.batch;
  float* qprep = (float*)ws;
  float* part = qprep + (size_t)batch * L.n_q_heads * plan.q_floats;
  hipError_t e = (L.k_kind == TQ_K_LM_QJL) ? run_prep<D, TQ_K_LM_QJL>(L, S, q, qprep, batch, st)
                                           : run_prep<D, TQ_K_AFFINE8>(L, S, q, qprep, batch, st);
  if (e != hipSuccess) return e;
  if (n_c > 0) {
    MainLaunch fn = find_main(L);
    if (!fn) return hipErrorInvalidDeviceFunction;
    e = fn(dim3(plan.n_splits, L.n_kv_heads, batch), st, C, S, qprep, part, L.n_kv_heads, n_c, plan.chunk,
           plan.n_splits);
    if (e != hipSuccess) return e;
  }
  return (L.v_kind == TQ_V_GROUP_SYM)
             ? run_combine<D, TQ_V_GROUP_SYM>(L, S, part, plan.n_splits, qprep, rk, rv, n_recent, rcap, out, batch, st)
             : run_combine<D, TQ_V_LM_ROT>(L, S, part, plan.n_splits, qprep, rk, rv, n_recent, rcap, out, batch, st);
}

}  // namespace

bool decode_compiled(const tq_layout& L) {
  if (!(L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256)) return false;
  if (L.n_kv_heads <= 0 || L.n_q_heads % L.n_kv_heads) return false;
  return find_main(L) != nullptr;
}

hipError_t launch_decode(const tq_layout& L, const tq_state& S, const void* q, const tq_cache& C, int n_c,
                         const void* rk, const void* rv, int n_recent, int rcap, float* out, void* ws,
                         const DecodePlan& plan, hipStream_t st) {
  switch (L.head_dim) {
    case 64: return run_decode_d<64>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st);
    case 128: return run_decode_d<128>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st);
    case 256: return run_decode_d<256>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq

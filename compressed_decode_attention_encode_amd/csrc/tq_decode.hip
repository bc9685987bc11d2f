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
                   const uint16_t* __restrict__ S, float* __restrict__ qprep, int Hq) {
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
    // q_s = S q_r; thread i takes row i of S (fp16) with independent 16-byte loads
    if (j < D) {
      const uint4* srow = reinterpret_cast<const uint4*>(S + (size_t)j * D);
      float acc = 0.f;
#pragma unroll 4
      for (int k = 0; k < D / 8; ++k) {
        const uint4 sv = srow[k];
        const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(f16_to_f32(w[i] & 0xFFFFu), s_x[8 * k + 2 * i], acc);
          acc = fmaf(f16_to_f32(w[i] >> 16), s_x[8 * k + 2 * i + 1], acc);
        }
      }
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
// finish: merge the splits of one (query head, batch), with the recent buffer and the
// inverse rotation (also the whole decode when nothing is compressed: zero splits).
// ---------------------------------------------------------------------------------
template <int D, int VK>
__global__ void __launch_bounds__(256) decode_finish_kernel(const DecodeArgs A, int nrep) {
  __shared__ float sm[finish_floats<D, 1>()];
  const int h = blockIdx.x;
  finish_group<D, 1, VK>(A, blockIdx.y, h / nrep, h, sm);
}

// ---------------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------------
// Workspace: prepared queries [B][Hq][4d] | split partials [B][Hq][n_splits][d+4].
static size_t ws_layout_bytes(const tq_layout& L, int batch, int n_splits) {
  const size_t d = L.head_dim;
  return sizeof(float) *
         ((size_t)batch * L.n_q_heads * 4 * d + (size_t)batch * L.n_q_heads * n_splits * (d + 4));
}

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
    want = std::min(want, kMaxFinishSplits);   // the finishing merge stages every split in LDS
    want = std::max(1, std::min(want, ceil_div(tiles, kMinTilesPerSplit)));
    const int tiles_per = ceil_div(tiles, want);
    p.chunk = tiles_per * kTile;
    p.n_splits = ceil_div(tiles, tiles_per);
  }
  p.q_floats = 4 * (size_t)d;
  p.part_stride = (size_t)d + 4;
  p.ws_bytes = ws_layout_bytes(L, batch, p.n_splits);
  return p;
}

size_t decode_ws_bound(const tq_layout& L, int batch, int max_c) {
  // n_splits of any n_c <= max_c is at most min(ceil(target/units), tiles(max_c))
  const long units = (long)batch * L.n_kv_heads;
  const int max_splits =
      std::max(0, std::min(ceil_div(kTargetDecodeGroups, units), ceil_div(std::max(max_c, 0), kTile)));
  return ws_layout_bytes(L, batch, max_splits);
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
hipError_t run_finish(const DecodeArgs& A, int nrep, int batch, hipStream_t st) {
  hipLaunchKernelGGL((decode_finish_kernel<D, VK>), dim3(A.Hq, batch), dim3(256), 0, st, A, nrep);
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
  DecodeArgs A{};
  A.kc = (const uint32_t*)C.k_codes;
  A.ks = (const uint32_t*)C.k_signs;
  A.ka = (const uint32_t*)C.k_aux;
  A.vc = (const uint32_t*)C.v_codes;
  A.va = (const uint32_t*)C.v_aux;
  A.kcent = S.k_centroids;
  A.vcent = S.v_centroids;
  A.vsign = S.v_signs;
  A.qprep = qprep;
  A.part = part;
  A.rk = (const uint16_t*)rk;
  A.rv = (const uint16_t*)rv;
  A.out = out;
  A.Hq = L.n_q_heads;
  A.Hkv = L.n_kv_heads;
  A.cap = C.capacity;
  A.n_c = n_c;
  A.chunk = plan.chunk;
  A.nsplit = plan.n_splits;
  A.n_recent = n_recent;
  A.recent_cap = rcap;
  A.recent_bf16 = (L.recent_dtype == TQ_BF16) ? 1 : 0;
  if (n_c > 0) {
    MainLaunch fn = find_main(L);
    if (!fn) return hipErrorInvalidDeviceFunction;
    e = fn(dim3(plan.n_splits, L.n_kv_heads, batch), st, A);
    if (e != hipSuccess) return e;
  }
  const int nrep = L.n_q_heads / L.n_kv_heads;
  return (L.v_kind == TQ_V_GROUP_SYM) ? run_finish<D, TQ_V_GROUP_SYM>(A, nrep, batch, st)
                                      : run_finish<D, TQ_V_LM_ROT>(A, nrep, batch, st);
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

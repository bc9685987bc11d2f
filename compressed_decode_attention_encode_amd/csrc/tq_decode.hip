// Decode attention: the split merge (one inverse butterfly for rotated-domain value
// sums), the split plan and the launch sequence.
//
//   main     tq_decode_main.h: per (split, kv-head, batch) the query preparation
//            (TurboQuant-MLX page, GPU kernel optimisation section, pre-rotated query),
//            scoring on the packed cache, online softmax and value sums; one extra split
//            per (batch, kv-head) takes the exact recent tokens (TurboQuant vLLM guide,
//            section 5; benchmark page, buffering strategy).
//   finish   log-sum-exp merge of the partials of one query head (news page, oMLX
//            section: a two-pass flash decode), rotated-domain value sums rotated back
//            once (TurboQuant-MLX page, butterfly pulled out of the loop), plus the
//            recent buffer's natural-domain sum under the same normaliser.
#include <algorithm>

#include "tq_decode_main.h"

namespace tq {

// Partials merged by one finish work-group (staged in LDS).
constexpr int kMaxParts = 512;

// ---------------------------------------------------------------------------------
// finish: grid (n_q_heads, batch)
// ---------------------------------------------------------------------------------
// One work-group per (query head, batch): the log-sum-exp merge of the compressed
// splits' partials and the recent buffer's partial (slot nsplit, natural domain) under
// one normaliser.  Every read is issued on entry, 16 bytes at a time, so the kernel waits
// on one round of reads before its arithmetic.
template <int D, int VK>
__global__ void __launch_bounds__(256) decode_finish_kernel(const DecodeArgs A) {
  static_assert(kMaxParts <= 2 * 256, "two split (m, l) pairs per thread");
  constexpr int SG = 1024 / D;           // split groups: thread = (4-dimension quad, split group)
  constexpr int PF = 8;                  // partial quads held per thread and pass
  __shared__ float s_w[kMaxParts];       // split weights
  __shared__ float s_red[8];
  __shared__ __attribute__((aligned(16))) float s_rot[SG][D];   // per split group sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x, b = blockIdx.y;
  const int ns = A.nsplit, np = A.n_part;   // np = ns + 1 with a recent partial
  const float* pp = A.part + (size_t)(b * A.Hq + head) * np * (D + 4);
  // Reads past the last split are clamped to it (never out of bounds, never a branch
  // around a load: that would make the compiler wait on each load in turn) and their
  // values are not used.
  // thread s (and s + 256): split s's maximum and normaliser
  float2 ml[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) ml[k] = *reinterpret_cast<const float2*>(pp + (size_t)min(tid + 256 * k, np - 1) * (D + 4));
  // the recent partial's values, 4 dimensions per thread
  float4 nat = make_float4(0.f, 0.f, 0.f, 0.f);
  if (np > ns && tid < D / 4) nat = *reinterpret_cast<const float4*>(pp + (size_t)ns * (D + 4) + 4 + 4 * tid);
  // thread (quad dq, split group sg): splits sg, sg + SG, ..., dimensions 4dq..4dq+3
  const int dq = tid % (D / 4), sg = tid / (D / 4);
  float4 pv[PF];
  if (ns > 0) {
#pragma unroll
    for (int i = 0; i < PF; ++i)
      pv[i] = *reinterpret_cast<const float4*>(pp + (size_t)min(sg + SG * i, ns - 1) * (D + 4) + 4 + 4 * dq);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (tid + 256 * k < np) mx = fmaxf(mx, ml[k].x);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (tid + 256 * k < np) {
      const float m = ml[k].x;
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - mx);
      s_w[tid + 256 * k] = w;
      l = fmaf(ml[k].y, w, l);
    }
  }
  l = wave_sum(l);
  if (lane == 0) s_red[4 + wave] = l;
  __syncthreads();
  const float L = s_red[4] + s_red[5] + s_red[6] + s_red[7];
  {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < ns; s0 += SG * PF) {
      if (s0 > 0) {
#pragma unroll
        for (int i = 0; i < PF; ++i)
          pv[i] = *reinterpret_cast<const float4*>(pp + (size_t)min(s0 + sg + SG * i, ns - 1) * (D + 4) + 4 + 4 * dq);
      }
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int s = s0 + sg + SG * i;
        if (s < ns) {
          const float w = s_w[s];
          a.x = fmaf(pv[i].x, w, a.x); a.y = fmaf(pv[i].y, w, a.y);
          a.z = fmaf(pv[i].z, w, a.z); a.w = fmaf(pv[i].w, w, a.w);
        }
      }
    }
    *reinterpret_cast<float4*>(&s_rot[sg][4 * dq]) = a;
  }
  // the recent partial under the common normaliser, kept in registers of threads < D/4
  if (np > ns && tid < D / 4) {
    const float w = s_w[ns];
    nat.x *= w; nat.y *= w; nat.z *= w; nat.w *= w;
  }
  __syncthreads();
  if constexpr (VK == TQ_V_LM_ROT) {
    for (int j = tid; j < D; j += 256) {
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < SG; ++q) a += s_rot[q][j];
      s_rot[0][j] = a;
    }
    __syncthreads();
    // Pi^T acc = diag(s) H acc / sqrt(d): butterflies in LDS
    float* x = s_rot[0];
    for (int hs = 1; hs < D; hs <<= 1) {
      if (tid < D / 2) {
        const int lo = (tid / hs) * 2 * hs + (tid % hs);
        const float u = x[lo], v = x[lo + hs];
        x[lo] = u + v;
        x[lo + hs] = u - v;
      }
      __syncthreads();
    }
  }
  if (tid < D / 4) {
    float4 mv;
    if constexpr (VK == TQ_V_LM_ROT) {
      const float r = rsqrtf((float)D);
      float e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int jj = 4 * tid + k;
        e[k] = s_rot[0][jj] * r;
        if ((A.vsign[jj >> 5] >> (jj & 31)) & 1u) e[k] = -e[k];
      }
      mv = make_float4(e[0], e[1], e[2], e[3]);
    } else {
      mv = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < SG; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&s_rot[q][4 * tid]);
        mv.x += v.x; mv.y += v.y; mv.z += v.z; mv.w += v.w;
      }
    }
    const float il = 1.f / L;
    *reinterpret_cast<float4*>(A.out + (size_t)(b * A.Hq + head) * D + 4 * tid) =
        make_float4((mv.x + nat.x) * il, (mv.y + nat.y) * il, (mv.z + nat.z) * il, (mv.w + nat.w) * il);
  }
}

// ---------------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------------
// Workspace: partials [B][Hq][n_splits + 1][d + 4] floats (the last slot: recent buffer).
static size_t ws_layout_bytes(const tq_layout& L, int batch, int n_splits) {
  return sizeof(float) * (size_t)batch * L.n_q_heads * (n_splits + 1) * (L.head_dim + 4);
}

// Most splits a launch may use: every split gets >= kMinTilesPerSplit tiles, all
// (batch, kv-head) units together stay within two rounds of kTargetDecodeGroups, and the
// merge stages every partial in LDS.
static int max_splits(const tq_layout& L, int batch, int n_c) {
  if (n_c <= 0) return 0;
  const long units = (long)batch * L.n_kv_heads;
  int s = ceil_div(n_c, kTile * kMinTilesPerSplit);
  s = std::min(s, ceil_div(2L * kTargetDecodeGroups, units));
  return std::max(1, std::min(s, kMaxParts - 1));
}

DecodePlan plan_decode(const tq_layout& L, int batch, int n_c) {
  DecodePlan p{};
  p.n_splits = max_splits(L, batch, n_c);
  p.chunk = 0;
  p.q_floats = 0;
  p.part_stride = (size_t)L.head_dim + 4;
  p.ws_bytes = ws_layout_bytes(L, batch, p.n_splits);
  return p;
}

size_t decode_ws_bound(const tq_layout& L, int batch, int max_c) {
  // max_splits is nondecreasing in n_c
  return ws_layout_bytes(L, batch, max_splits(L, batch, std::max(max_c, 0)));
}

// Multi-query decode: the splits are planned over the (batch, kv-head) units as for one
// query; the partials hold one row per (batch, query, q-head).
size_t decode_multi_ws_bound(const tq_layout& L, int batch, int n_query, int max_c) {
  return ws_layout_bytes(L, batch * n_query, max_splits(L, batch, std::max(max_c, 0)));
}

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

MainKernel find_main(const tq_layout& L) {
  const int nrep = L.n_q_heads / L.n_kv_heads;
  const int d = L.head_dim, vk = L.v_kind, vb = L.v_bits;
  if (d == 512) return find_main_d512(L);
#define TQ_BY_D(name)                                                   \
  switch (d) {                                                          \
    case 64: return name##_d64(nrep, vk, vb);                           \
    case 128: return name##_d128(nrep, vk, vb);                         \
    case 256: return name##_d256(nrep, vk, vb);                         \
    default: return MainKernel{nullptr, nullptr};                       \
  }
  if (L.k_kind == TQ_K_LM_QJL) {
    switch (L.k_bits) {
      case 2: TQ_BY_D(find_main_lm2)
      case 3: TQ_BY_D(find_main_lm3)
      case 4: TQ_BY_D(find_main_lm4)
      default: return MainKernel{nullptr, nullptr};
    }
  }
  if (L.k_kind == TQ_K_LM_MSE) {
    switch (L.k_bits) {
      case 2: TQ_BY_D(find_main_lmm2)
      case 3: TQ_BY_D(find_main_lmm3)
      case 4: TQ_BY_D(find_main_lmm4)
      default: return MainKernel{nullptr, nullptr};
    }
  }
  if (L.k_kind == TQ_K_AFFINE8 && L.k_bits == 8) { TQ_BY_D(find_main_aff8) }
  if (L.k_kind == TQ_K_AFFINE8 && (d == 64 || d == 128)) {   // 5/4/2-bit affine keys
    const bool d64 = d == 64;
    switch (L.k_bits) {
      case 5: return d64 ? find_main_aff5_d64(nrep, vk, vb) : find_main_aff5_d128(nrep, vk, vb);
      case 4: return d64 ? find_main_aff4_d64(nrep, vk, vb) : find_main_aff4_d128(nrep, vk, vb);
      case 2: return d64 ? find_main_aff2_d64(nrep, vk, vb) : find_main_aff2_d128(nrep, vk, vb);
      default: return MainKernel{nullptr, nullptr};
    }
  }
  // 16-bit keys: d = 64 and 128; d = 256 on the matrix cores with 32-token tiles (either storage)
  if (L.k_kind == TQ_K_F16 && L.k_bits == 16) {
    // fp16-stored keys are exact matrix-core operands; bf16 ones stay on the vector ALUs
    if (d == 64 && L.in_dtype == TQ_F16 && nrep >= 3) {
      const MainKernel mk = find_mma_f16_d64(nrep, vk, vb);
      if (mk.launch) return mk;
    }
    if (d == 64) return find_main_f16_d64(nrep, vk, vb);
    if (d == 128) return find_main_f16_d128(nrep, vk, vb);
    if (d == 256) return find_mma_f16_d256(nrep, vk, vb);          // fp16 or bf16 storage
    return MainKernel{nullptr, nullptr};
  }
#undef TQ_BY_D
  return MainKernel{nullptr, nullptr};
}

template <int D, int VK>
hipError_t run_finish(const DecodeArgs& A, int batch, hipStream_t st) {
  hipLaunchKernelGGL((decode_finish_kernel<D, VK>), dim3(A.Hq, batch), dim3(256), 0, st, A);
  return hipGetLastError();
}

// Multi-query instantiations (LM + QJL keys, group values): n_rep query heads, nq queries.
MainKernel find_multi(const tq_layout& L, int nq) {
  const int nrep = L.n_q_heads / L.n_kv_heads;
  if (L.k_kind != TQ_K_LM_QJL || L.v_kind != TQ_V_GROUP_SYM) return MainKernel{nullptr, nullptr};
  if (L.head_dim == 64 && L.k_bits == 3) return find_multi_lm3_d64(nrep, nq, L.v_bits);
  if (L.head_dim == 64 && L.k_bits == 4) return find_multi_lm4_d64(nrep, nq, L.v_bits);
  if (L.head_dim == 128 && L.k_bits == 3) return find_multi_lm3_d128(nrep, nq, L.v_bits);
  if (L.head_dim == 128 && L.k_bits == 4) return find_multi_lm4_d128(nrep, nq, L.v_bits);
  return MainKernel{nullptr, nullptr};
}

// One decode launch sequence: the split kernel `mk` over (split, kv-head, batch) groups, then
// the merge over (q-head, batch x nq) rows.
template <int D>
hipError_t run_decode_d(const tq_layout& L, const tq_state& S, const void* q, const tq_cache& C, int n_c,
                        const void* rk, const void* rv, int n_recent, int rcap, float* out, void* ws,
                        const DecodePlan& plan, hipStream_t st, const MainKernel& mk, int nq) {
  const int batch = C.batch;
  if (!mk.launch) return hipErrorInvalidDeviceFunction;
  // splits: one round of resident work-groups over all (batch, kv-head) units, within the
  // planned maximum; every split a whole number of tiles
  int nsplit = 0, chunk = 0;
  if (n_c > 0) {
    const long units = (long)batch * L.n_kv_heads;
    const long resident = (long)device_cus() * mk.blocks_per_cu();
    const int tiles = ceil_div(n_c, kTile);
    const int want = std::max(1, std::min(plan.n_splits, ceil_div(resident, units)));
    int tiles_per = ceil_div(tiles, want);
    if (tiles_per > 4) tiles_per = (tiles_per + 3) & ~3;   // whole rounds of the 4 waves
    chunk = tiles_per * kTile;
    nsplit = ceil_div(tiles, tiles_per);
  }
  DecodeArgs A{};
  A.q = (const uint16_t*)q;
  A.kc = (const uint32_t*)C.k_codes;
  A.ks = (const uint32_t*)C.k_signs;
  A.ka = (const uint32_t*)C.k_aux;
  A.vc = (const uint32_t*)C.v_codes;
  A.va = (const uint32_t*)C.v_aux;
  A.kcent = S.k_centroids;
  A.vcent = S.v_centroids;
  A.ksign = S.k_signs;
  A.vsign = S.v_signs;
  A.S = S.qjl;
  A.part = (float*)ws;
  A.rk = (const uint16_t*)rk;
  A.rv = (const uint16_t*)rv;
  A.out = out;
  A.Hq = L.n_q_heads;
  A.Hkv = L.n_kv_heads;
  A.batch = batch;
  A.cap = C.capacity;
  A.n_c = n_c;
  A.chunk = chunk;
  A.nsplit = nsplit;
  A.n_part = nsplit + (n_recent > 0 ? 1 : 0);
  A.n_recent = n_recent;
  A.recent_cap = rcap;
  A.recent_bf16 = (L.recent_dtype == TQ_BF16) ? 1 : 0;
  A.q_bf16 = (L.in_dtype == TQ_BF16) ? 1 : 0;
  const long groups = (long)A.n_part * L.n_kv_heads * batch;
  if (groups > 0x7FFFFFFFL) return hipErrorInvalidConfiguration;
  if (groups > 0) {
    const hipError_t e = mk.launch(dim3((unsigned)groups), st, A);
    if (e != hipSuccess) return e;
  }
  // natural-domain value sums (symmetric and min/max groups) merge alike; rotated ones are
  // rotated back once after the merge
  return (L.v_kind == TQ_V_LM_ROT) ? run_finish<D, TQ_V_LM_ROT>(A, batch * nq, st)
                                   : run_finish<D, TQ_V_GROUP_SYM>(A, batch * nq, st);
}

}  // namespace

bool decode_compiled(const tq_layout& L) {
  if (!(L.head_dim == 64 || L.head_dim == 128 || L.head_dim == 256 || L.head_dim == 512)) return false;
  if (L.n_kv_heads <= 0 || L.n_q_heads % L.n_kv_heads) return false;
  return find_main(L).launch != nullptr;
}

hipError_t launch_decode(const tq_layout& L, const tq_state& S, const void* q, const tq_cache& C, int n_c,
                         const void* rk, const void* rv, int n_recent, int rcap, float* out, void* ws,
                         const DecodePlan& plan, hipStream_t st) {
  const MainKernel mk = find_main(L);
  switch (L.head_dim) {
    case 64: return run_decode_d<64>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, 1);
    case 128: return run_decode_d<128>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, 1);
    case 256: return run_decode_d<256>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, 1);
    case 512: return run_decode_d<512>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, 1);
    default: return hipErrorInvalidValue;
  }
}

bool decode_multi_compiled(const tq_layout& L, int n_query) {
  if (L.n_kv_heads <= 0 || L.n_q_heads % L.n_kv_heads) return false;
  return find_multi(L, n_query).launch != nullptr;
}

hipError_t launch_decode_multi(const tq_layout& L, const tq_state& S, const void* q, int n_query, const tq_cache& C,
                               int n_c, const void* rk, const void* rv, int n_recent, int rcap, float* out, void* ws,
                               const DecodePlan& plan, hipStream_t st) {
  const MainKernel mk = find_multi(L, n_query);
  switch (L.head_dim) {
    case 64: return run_decode_d<64>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, n_query);
    case 128: return run_decode_d<128>(L, S, q, C, n_c, rk, rv, n_recent, rcap, out, ws, plan, st, mk, n_query);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq

// Fused split-K decode attention over the packed cache (gfx950, vector ALUs).
//
// Method sources: news page "vLLM, llama.cpp, MLX all follow up" (digipub.cc), oMLX
// section: attention computed straight from the packed indices, no fp16 intermediate;
// TurboQuant-MLX page (pomoai.com), GPU kernel optimisation section: query rotated once
// before scoring, weighted value sum accumulated in the rotated domain with a single
// butterfly afterwards, wave-level reductions, GQA n_rep handled without repeating KV;
// TurboQuant vLLM guide (kwkr.cn), section 2: the unbiased LM + QJL inner product.
//
// One work-group = one (batch, kv-head, split) and 4 independent waves.  A wave takes
// 64-token tiles of the split in turn:
//   1. stage the tile's packed rows (every plane) from HBM into its own LDS area with
//      coalesced loads (rows padded to an odd word stride: conflict-free row reads);
//   2. scores, one token per lane, for all n_rep query heads of the group at once: the
//      codes are unpacked once and the prepared query (uniform across the wave) comes in
//      through scalar registers, so each code element costs one FMA per head;
//   3. online softmax in the log2 domain (scores carry log2(e)/sqrt(d) from the prep);
//   4. weighted value sum, 8 dimensions per lane: each decoded value element is used by
//      all n_rep heads; group-scaled values fold the scale into the weight and the
//      (L-1)/2 offset into one per-group running sum.
// The four waves then merge (m, l, acc) through LDS and write one partial per head; a
// second kernel (one work-group per (batch, kv-head)) merges the splits: the kernel
// boundary makes every partial visible without device-wide cache flushes.
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

template <int D, int NREP, int KK, int KB, int VK, int VB>
struct DecodeGeom {
  static constexpr int KPER = (KB == 3) ? 10 : (KK == TQ_K_AFFINE8 ? 4 : 32 / KB);
  static constexpr int WK = (KK == TQ_K_AFFINE8) ? D / 4 : (D + KPER - 1) / KPER;
  static constexpr int WS = (KK == TQ_K_LM_QJL) ? D / 32 : 0;
  static constexpr int WAK = (KK == TQ_K_LM_QJL) ? 1 : D / 32;
  static constexpr int VPER = (VB == 3) ? 10 : 32 / VB;
  static constexpr int WV = (D + VPER - 1) / VPER;
  static constexpr int WAV = (VK == TQ_V_GROUP_SYM) ? D / 64 : 1;
  // odd LDS strides
  static constexpr int odd(int w) { return w == 0 ? 0 : (w | 1); }
  static constexpr int SK = odd(WK), SS = odd(WS), SAK = odd(WAK), SV = odd(WV), SAV = odd(WAV);
  static constexpr int STAGE = kTile * (SK + SS + SAK + SV + SAV);   // words per wave
  static constexpr int LPT = D / 8;                                 // value lanes per token
  static constexpr int SLOTS = kWave / LPT;                         // tokens per value step
  static constexpr int QF = 4 * D;                                  // prepared-query floats per head
  static constexpr int PS = D + 4;                                  // partial stride (floats)
};

// Register double-buffer for one plane of a 64-token tile: load() issues the global
// reads of the next tile (they stay in flight while the current tile is computed),
// store() later writes them into the wave's LDS area with row stride LS.  Reads never
// go past the last valid row; rows beyond it are zero-filled.
template <int W, int LS>
struct RowLoader {
  static constexpr int N = kTile * W;               // words per tile
  static constexpr int NV = (N + 4 * kWave - 1) / (4 * kWave);
  static constexpr int NR = (W == 0) ? 1 : 4 * NV;  // registers per lane
  uint32_t r[NR];
  bool vec;
  __device__ __forceinline__ void load(const uint32_t* __restrict__ g, int rows, int lane) {
    if constexpr (W == 0) return;
    const int nvalid = rows * W;
    vec = (reinterpret_cast<uintptr_t>(g) & 15) == 0;
    if (vec) {
      const uint4* g4 = reinterpret_cast<const uint4*>(g);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int q = 4 * (i * kWave + lane);
        if (q + 4 <= nvalid) {
          const uint4 v = g4[q / 4];
          r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) r[4 * i + k] = (q + k < nvalid) ? g[q + k] : 0u;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int q = i * kWave + lane;
        r[i] = (q < nvalid) ? g[q] : 0u;
      }
    }
  }
  __device__ __forceinline__ void store(uint32_t* __restrict__ lds, int lane) const {
    if constexpr (W == 0) return;
    if (vec) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = 4 * (i * kWave + lane) + k;
          if (q < N) lds[(q / W) * LS + (q % W)] = r[4 * i + k];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int q = i * kWave + lane;
        if (q < N) lds[(q / W) * LS + (q % W)] = r[i];
      }
    }
  }
};

// Everything the decode kernels need, passed by value.
struct DecodeArgs {
  const uint32_t *kc, *ks, *ka, *vc, *va;   // packed planes
  const float *kcent, *vcent;                 // codebooks (LM keys / rotated LM values)
  const uint32_t* vsign;                      // value rotation signs (rotated LM values)
  const float* qprep;                         // prepared queries [B][Hq][QF]
  float* part;                                // split partials [B][Hq][nsplit][PS]
  const uint16_t *rk, *rv;                    // recent buffer [B][Hkv][recent_cap][d]
  float* out;                                 // [B][Hq][d]
  int Hq, Hkv, cap, n_c, chunk, nsplit, n_recent, recent_cap, recent_bf16;
};

__device__ __forceinline__ float recent_to_f32(uint32_t bits, int bf16) {
  return bf16 ? __uint_as_float(bits << 16) : f16_to_f32(bits);
}

// Merge the n_split partials of NREP consecutive query heads h0.. of kv-head g (batch b),
// fold in the
// exact recent tokens under the same normaliser, rotate rotated-domain value sums back
// with one inverse Walsh-Hadamard transform, normalise and write the output.
// Uses all 256 threads.  Every global load is independent of the others: split maxima,
// normalisers and queries are staged in LDS first, weights are computed once per head,
// and each (head, dimension) sum is spread over 256/(n_rep d) threads.
// Needs NREP * nsplit <= kMaxFinishSplits; `sm` holds finish_floats<D, NREP>() floats.
constexpr int kMaxFinishSplits = 512;

template <int D, int NREP>
constexpr int finish_floats() {
  constexpr int items = NREP * D;
  return items + 2 * kMaxFinishSplits + NREP * kMaxRecent + 2 * NREP + 2 * (items > 256 ? items : 256);
}

template <int D, int NREP, int VK>
__device__ void finish_group(const DecodeArgs& A, int b, int g, int h0, float* sm) {
  constexpr int QF = 4 * D, PS = D + 4;
  constexpr int ITEMS = NREP * D;
  constexpr int NG = (ITEMS >= 256) ? 1 : 256 / ITEMS;   // threads per (head, dimension) item
  constexpr int PART = (ITEMS > 256 ? ITEMS : 256);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = A.Hq;
  const int R = A.n_recent, ns = A.nsplit;
  float* s_qn = sm;                         // [NREP][D]
  float* s_w = s_qn + ITEMS;                // [NREP][ns] split maxima -> weights
  float* s_l = s_w + kMaxFinishSplits;      // [NREP][ns] split normalisers
  float* s_sr = s_l + kMaxFinishSplits;     // [NREP][kMaxRecent] recent scores -> weights
  float* s_M = s_sr + NREP * kMaxRecent;    // [NREP]
  float* s_L = s_M + NREP;                  // [NREP]
  float* s_pa = s_L + NREP;                 // [NG][ITEMS] partial sums (compressed part)
  float* s_pr = s_pa + PART;                // [NG][ITEMS] partial sums (recent part)
  const size_t rbase = ((size_t)b * A.Hkv + g) * A.recent_cap;
  const float* pp0 = A.part + (size_t)(b * Hq + h0) * ns * PS;
  const float* qn0 = A.qprep + (size_t)(b * Hq + h0) * QF + 2 * D;
  for (int i = tid; i < ITEMS; i += 256) s_qn[i] = qn0[(size_t)(i / D) * QF + (i % D)];
  for (int i = tid; i < NREP * ns; i += 256) {
    const float* pp = pp0 + (size_t)i * PS;    // head i / ns, split i % ns
    s_w[i] = pp[0];
    s_l[i] = pp[1];
  }
  __syncthreads();
  // recent-token scores, one (head, token) pair per thread
  for (int i = tid; i < NREP * R; i += 256) {
    const int h = i / R, r = i % R;
    const uint4* kr = reinterpret_cast<const uint4*>(A.rk + (rbase + r) * D);
    const float* qn = s_qn + h * D;
    float a = 0.f;
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
      const uint4 u = kr[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a = fmaf(qn[8 * c + 2 * k], recent_to_f32(w[k] & 0xFFFFu, A.recent_bf16), a);
        a = fmaf(qn[8 * c + 2 * k + 1], recent_to_f32(w[k] >> 16, A.recent_bf16), a);
      }
    }
    s_sr[h * kMaxRecent + r] = a;
  }
  __syncthreads();
  // per head: max, weights, normaliser (one wave per head, heads strided over 4 waves)
  for (int h = wave; h < NREP; h += 4) {
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, s_w[h * ns + s]);
    for (int r = lane; r < R; r += 64) mx = fmaxf(mx, s_sr[h * kMaxRecent + r]);
    mx = wave_max(mx);
    float l = 0.f;
    for (int s = lane; s < ns; s += 64) {
      const float m = s_w[h * ns + s];
      const float w = (m == -INFINITY) ? 0.f : exp2f(m - mx);
      s_w[h * ns + s] = w;
      l = fmaf(s_l[h * ns + s], w, l);
    }
    for (int r = lane; r < R; r += 64) {
      const float p = exp2f(s_sr[h * kMaxRecent + r] - mx);
      s_sr[h * kMaxRecent + r] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { s_M[h] = mx; s_L[h] = l; }
  }
  __syncthreads();
  // (head, dimension) sums: thread group `grp` takes splits / recent tokens grp, grp+NG, ...
  for (int it = tid; it < ITEMS * NG; it += 256) {
    const int item = it % ITEMS, grp = it / ITEMS;
    const int h = item / D, j = item % D;
    const float* pp = pp0 + (size_t)h * ns * PS + 4 + j;
    const float* w = s_w + h * ns;
    float a = 0.f;
#pragma unroll 8
    for (int s = grp; s < ns; s += NG) a = fmaf(pp[(size_t)s * PS], w[s], a);
    const uint16_t* vr = A.rv + rbase * D + j;
    const float* pr = s_sr + h * kMaxRecent;
    float rs = 0.f;
#pragma unroll 8
    for (int r = grp; r < R; r += NG) rs = fmaf(pr[r], recent_to_f32(vr[(size_t)r * D], A.recent_bf16), rs);
    s_pa[grp * ITEMS + item] = a;
    s_pr[grp * ITEMS + item] = rs;
  }
  __syncthreads();
  if constexpr (NG > 1) {
    for (int i = tid; i < ITEMS; i += 256) {
      float a = 0.f, rs = 0.f;
#pragma unroll
      for (int q = 0; q < NG; ++q) { a += s_pa[q * ITEMS + i]; rs += s_pr[q * ITEMS + i]; }
      s_pa[i] = a;
      s_pr[i] = rs;
    }
    __syncthreads();
  }
  if constexpr (VK == TQ_V_LM_ROT) {
    // Pi^T acc = diag(s) H acc / sqrt(d) for every head: butterflies in LDS
    for (int hs = 1; hs < D; hs <<= 1) {
      for (int i = tid; i < ITEMS / 2; i += 256) {
        const int h = i / (D / 2), t = i % (D / 2);
        const int lo = h * D + (t / hs) * 2 * hs + (t % hs);
        const float x = s_pa[lo], y = s_pa[lo + hs];
        s_pa[lo] = x + y;
        s_pa[lo + hs] = x - y;
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < ITEMS; i += 256) {
    const int h = i / D, j = i % D;
    float mv = s_pa[i];
    if constexpr (VK == TQ_V_LM_ROT) {
      mv *= rsqrtf((float)D);
      if ((A.vsign[j >> 5] >> (j & 31)) & 1u) mv = -mv;
    }
    A.out[(size_t)(b * Hq + h0 + h) * D + j] = (mv + s_pr[i]) / s_L[h];
  }
}

template <int D, int NREP, int KK, int KB, int VK, int VB>
__global__ void __launch_bounds__(256)
decode_main_kernel(const DecodeArgs A) {
  using G = DecodeGeom<D, NREP, KK, KB, VK, VB>;
  constexpr int LK = 1 << KB;
  constexpr int LV = 1 << VB;

  __shared__ __attribute__((aligned(16))) uint32_t s_stage[4 * G::STAGE];
  __shared__ float s_p[4][NREP * kWave];
  __shared__ float s_kcent[16], s_vcent[16];
  __shared__ float s_mrg_m[4][NREP], s_mrg_l[4][NREP];
  // the four waves' value sums reuse the staging area once the tile loop is done
  static_assert(4 * G::STAGE >= 4 * NREP * D, "merge buffer does not fit in the staging area");
  float(*s_mrg_acc)[NREP * D] = reinterpret_cast<float(*)[NREP * D]>(s_stage);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int Hkv = A.Hkv, cap = A.cap, n_c = A.n_c, chunk = A.chunk, nsplit = A.nsplit;
  const uint32_t* __restrict__ kc = A.kc;
  const uint32_t* __restrict__ ks = A.ks;
  const uint32_t* __restrict__ ka = A.ka;
  const uint32_t* __restrict__ vc = A.vc;
  const uint32_t* __restrict__ va = A.va;
  const int Hq = Hkv * NREP;

  if (threadIdx.x < 16) {
    if constexpr (KK == TQ_K_LM_QJL) s_kcent[threadIdx.x] = (threadIdx.x < LK) ? A.kcent[threadIdx.x] : 0.f;
    if constexpr (VK == TQ_V_LM_ROT) s_vcent[threadIdx.x] = (threadIdx.x < LV) ? A.vcent[threadIdx.x] : 0.f;
  }
  __syncthreads();

  const float* __restrict__ qp = A.qprep + (size_t)(b * Hq + g * NREP) * G::QF;
  const size_t slice = (size_t)b * Hkv + g;
  const int tb = split * chunk;
  const int te = min(n_c, tb + chunk);

  uint32_t* st_k = s_stage + wave * G::STAGE;
  uint32_t* st_s = st_k + kTile * G::SK;
  uint32_t* st_ak = st_s + kTile * G::SS;
  uint32_t* st_v = st_ak + kTile * G::SAK;
  uint32_t* st_av = st_v + kTile * G::SV;
  float* sp = s_p[wave];

  float m_run[NREP], l_run[NREP], off[NREP];
  float acc[NREP][8];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
    off[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const int slot = lane / G::LPT;
  const int prt = lane % G::LPT;

  RowLoader<G::WK, G::SK> ld_k;
  RowLoader<G::WS, G::SS> ld_s;
  RowLoader<G::WAK, G::SAK> ld_ak;
  RowLoader<G::WV, G::SV> ld_v;
  RowLoader<G::WAV, G::SAV> ld_av;
  auto issue = [&](int t0) {
    const int nv = min(kTile, te - t0);
    const size_t row0 = slice * cap + t0;
    ld_k.load(kc + row0 * G::WK, nv, lane);
    ld_s.load(ks + row0 * G::WS, nv, lane);
    ld_ak.load(ka + row0 * G::WAK, nv, lane);
    ld_v.load(vc + row0 * G::WV, nv, lane);
    ld_av.load(va + row0 * G::WAV, nv, lane);
  };
  if (tb + wave * kTile < te) issue(tb + wave * kTile);

  for (int t0 = tb + wave * kTile; t0 < te; t0 += 4 * kTile) {
    const int nv = min(kTile, te - t0);
    // ---- 1. stage this tile from registers into LDS, then start loading the next one ------
    ld_k.store(st_k, lane);
    ld_s.store(st_s, lane);
    ld_ak.store(st_ak, lane);
    ld_v.store(st_v, lane);
    ld_av.store(st_av, lane);
    if (t0 + 4 * kTile < te) issue(t0 + 4 * kTile);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 2. scores: lane = token ----------------------------------------------------------
    // The query block is uniform across the wave and is read through scalar loads; the
    // outer loop walks CH dimensions at a time and is not unrolled, so only one chunk of
    // query values is live in scalar registers (a fully unrolled loop would hoist all of
    // them and spill).  Codes come from the lane's staged row in LDS.
    float s2[NREP];
    {
      constexpr int CH = (NREP <= 4) ? 8 : 4;
      const uint32_t* krow = st_k + lane * G::SK;
      if constexpr (KK == TQ_K_LM_QJL) {
        const uint32_t* srow = st_s + lane * G::SS;
        const uint32_t aux = st_ak[lane * G::SAK];
        float alm[NREP], aqj[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) { alm[h] = 0.f; aqj[h] = 0.f; }
#pragma unroll 1
        for (int j0 = 0; j0 < D; j0 += CH) {
          uint32_t x;   // code j0 + i at bits KB*i
          if constexpr (KB == 3) {
            const int w0 = j0 / 10, r0 = j0 % 10, k0 = 10 - r0;   // codes left in word w0
            const uint32_t lo = krow[w0] >> (3 * r0);
            x = (k0 >= CH) ? lo : ((lo & ((1u << (3 * k0)) - 1u)) | (krow[w0 + 1] << (3 * k0)));
          } else {
            constexpr int PER = 32 / KB;
            x = krow[j0 / PER] >> (KB * (j0 % PER));
          }
          const uint32_t nsw = ~(srow[j0 >> 5] >> (j0 & 31));   // inverted QJL bits, dim j0 at bit 0
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            const float c = s_kcent[(x >> (KB * i)) & (LK - 1)];
            // sigma = +1 where the stored bit is 1: +-1.0f from the inverted bit
            const float sg = __uint_as_float(((nsw << (31 - i)) & 0x80000000u) | 0x3F800000u);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              alm[h] = fmaf(qp[h * G::QF + j0 + i], c, alm[h]);
              aqj[h] = fmaf(qp[h * G::QF + D + j0 + i], sg, aqj[h]);
            }
          }
        }
        const float nn = f16_to_f32(aux & 0xFFFFu);
        const float gm = f16_to_f32(aux >> 16);
#pragma unroll
        for (int h = 0; h < NREP; ++h) s2[h] = nn * fmaf(gm, aqj[h], alm[h]);
      } else {
        float ag[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) { s2[h] = 0.f; ag[h] = 0.f; }
#pragma unroll 1
        for (int j0 = 0; j0 < D; j0 += CH) {
#pragma unroll
          for (int wi = 0; wi < CH / 4; ++wi) {
            const uint32_t word = krow[j0 / 4 + wi];
#pragma unroll
            for (int bsel = 0; bsel < 4; ++bsel) {
              const float q8 = (float)((word >> (8 * bsel)) & 0xFFu);
#pragma unroll
              for (int h = 0; h < NREP; ++h) ag[h] = fmaf(qp[h * G::QF + j0 + 4 * wi + bsel], q8, ag[h]);
            }
          }
          if (((j0 + CH) & 31) == 0) {   // end of a 32-block: fold in its scale and offset
            const int gi = j0 >> 5;
            const uint32_t aux = st_ak[lane * G::SAK + gi];
            const float a = f16_to_f32(aux & 0xFFFFu);
            const float m = f16_to_f32(aux >> 16);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              s2[h] = fmaf(a, ag[h], fmaf(m, qp[h * G::QF + 3 * D + gi], s2[h]));
              ag[h] = 0.f;
            }
          }
        }
      }
    }
    if (lane >= nv) {
#pragma unroll
      for (int h = 0; h < NREP; ++h) s2[h] = -INFINITY;
    }

    // ---- 3. online softmax -------------------------------------------------------------
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      const float mn = fmaxf(m_run[h], wave_max(s2[h]));
      const float alpha = exp2f(m_run[h] - mn);
      const float p = exp2f(s2[h] - mn);
      l_run[h] = fmaf(l_run[h], alpha, p);
      m_run[h] = mn;
      off[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      sp[h * kWave + lane] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 4. weighted values: lane = (token slot, 8 dimensions) ---------------------------
#pragma unroll 2
    for (int stp = 0; stp < kTile / G::SLOTS; ++stp) {
      const int t = stp * G::SLOTS + slot;
      float pw[NREP];
#pragma unroll
      for (int h = 0; h < NREP; ++h) pw[h] = sp[h * kWave + t];
      float cv[8];
      if constexpr (VK == TQ_V_GROUP_SYM) {
        // 8 codes of VB bits, all inside one word
        const int bit0 = 8 * prt * VB;
        const uint32_t w = st_v[t * G::SV + (bit0 >> 5)] >> (bit0 & 31);
#pragma unroll
        for (int e = 0; e < 8; ++e) cv[e] = (float)((w >> (VB * e)) & (LV - 1));
        const int gi = prt / 4;   // 32-group of these 8 dimensions
        const float dl = f16_to_f32((st_av[t * G::SAV + (gi >> 1)] >> (16 * (gi & 1))) & 0xFFFFu);
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float wgt = pw[h] * dl;
          off[h] += wgt;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wgt, cv[e], acc[h][e]);
        }
      } else {
        const float nv_t = __uint_as_float(st_av[t * G::SAV]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 8 * prt + e;
          const uint32_t code = (st_v[t * G::SV + j / G::VPER] >> (VB * (j % G::VPER))) & (LV - 1);
          cv[e] = s_vcent[code];
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          const float wgt = pw[h] * nv_t;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wgt, cv[e], acc[h][e]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- wave totals: l over tokens, acc over token slots ---------------------------------
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    l_run[h] = wave_sum(l_run[h]);
    if constexpr (VK == TQ_V_GROUP_SYM) {
      const float o = 0.5f * (float)(LV - 1) * off[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] -= o;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int m = G::LPT; m < kWave; m <<= 1) acc[h][e] += __shfl_xor(acc[h][e], m);
    }
  }
  __syncthreads();   // every wave is done with its staging area
  if (lane < G::LPT) {
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_mrg_acc[wave][h * D + 8 * lane + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      s_mrg_m[wave][h] = m_run[h];
      s_mrg_l[wave][h] = l_run[h];
    }
  }
  __syncthreads();

  // ---- merge the four waves, write one partial per head ----------------------------------
  for (int i = threadIdx.x; i < NREP * D; i += blockDim.x) {
    const int h = i / D, j = i % D;
    float mx = s_mrg_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, s_mrg_m[w][h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = (s_mrg_m[w][h] == -INFINITY) ? 0.f : exp2f(s_mrg_m[w][h] - mx);
      a = fmaf(s_mrg_acc[w][h * D + j], sc, a);
      l = fmaf(s_mrg_l[w][h], sc, l);
    }
    float* dst = A.part + ((size_t)(b * Hq + g * NREP + h) * nsplit + split) * G::PS;
    dst[4 + j] = a;
    if (j == 0) {
      dst[0] = mx;
      dst[1] = l;
    }
  }

}

using MainLaunch = hipError_t (*)(dim3 grid, hipStream_t st, const DecodeArgs& A);

template <int D, int NREP, int KK, int KB, int VK, int VB>
hipError_t main_launch(dim3 grid, hipStream_t st, const DecodeArgs& A) {
  hipLaunchKernelGGL((decode_main_kernel<D, NREP, KK, KB, VK, VB>), grid, dim3(256), 0, st, A);
  return hipGetLastError();
}

// Lookup of the compiled instantiations (one file per key kind and head_dim).
MainLaunch find_main_lm2_d64(int nrep, int vk, int vb);
MainLaunch find_main_lm3_d64(int nrep, int vk, int vb);
MainLaunch find_main_lm4_d64(int nrep, int vk, int vb);
MainLaunch find_main_aff8_d64(int nrep, int vk, int vb);
MainLaunch find_main_lm2_d128(int nrep, int vk, int vb);
MainLaunch find_main_lm3_d128(int nrep, int vk, int vb);
MainLaunch find_main_lm4_d128(int nrep, int vk, int vb);
MainLaunch find_main_aff8_d128(int nrep, int vk, int vb);
MainLaunch find_main_lm2_d256(int nrep, int vk, int vb);
MainLaunch find_main_lm3_d256(int nrep, int vk, int vb);
MainLaunch find_main_lm4_d256(int nrep, int vk, int vb);
MainLaunch find_main_aff8_d256(int nrep, int vk, int vb);

}  // namespace tq

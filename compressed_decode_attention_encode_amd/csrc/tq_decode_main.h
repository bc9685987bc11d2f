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
// The four waves then merge (m, l, acc) through LDS and write one partial per head.
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

// Copy `rows` (<= 64) rows of W words from global into LDS with row stride LS; rows
// beyond `rows` are zero-filled.  Global reads never go past the last valid row: a
// 16-byte load is used only when all four of its words are inside the valid rows.
template <int W, int LS>
__device__ __forceinline__ void stage_rows(uint32_t* __restrict__ lds, const uint32_t* __restrict__ g,
                                           int rows, int lane) {
  if constexpr (W == 0) return;
  constexpr int N = kTile * W;
  const int nvalid = rows * W;
  if ((reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    const uint4* g4 = reinterpret_cast<const uint4*>(g);
#pragma unroll
    for (int i = 0; i < (N + 4 * kWave - 1) / (4 * kWave); ++i) {
      const int q = 4 * (i * kWave + lane);
      if (q < N) {
        uint32_t vv[4] = {0u, 0u, 0u, 0u};
        if (q + 4 <= nvalid) {
          const uint4 v = g4[q / 4];
          vv[0] = v.x; vv[1] = v.y; vv[2] = v.z; vv[3] = v.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (q + k < nvalid) vv[k] = g[q + k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int qq = q + k;
          if (qq < N) lds[(qq / W) * LS + (qq % W)] = vv[k];
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < (N + kWave - 1) / kWave; ++i) {
      const int q = i * kWave + lane;
      if (q < N) lds[(q / W) * LS + (q % W)] = (q < nvalid) ? g[q] : 0u;
    }
  }
}

template <int D, int NREP, int KK, int KB, int VK, int VB>
__global__ void __launch_bounds__(256)
decode_main_kernel(const uint32_t* __restrict__ kc, const uint32_t* __restrict__ ks,
                   const uint32_t* __restrict__ ka, const uint32_t* __restrict__ vc,
                   const uint32_t* __restrict__ va, const float* __restrict__ kcent,
                   const float* __restrict__ vcent, const float* __restrict__ qprep,
                   float* __restrict__ part, int Hkv, int cap, int n_c, int chunk, int nsplit) {
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
  const int Hq = Hkv * NREP;

  if (threadIdx.x < 16) {
    if constexpr (KK == TQ_K_LM_QJL) s_kcent[threadIdx.x] = (threadIdx.x < LK) ? kcent[threadIdx.x] : 0.f;
    if constexpr (VK == TQ_V_LM_ROT) s_vcent[threadIdx.x] = (threadIdx.x < LV) ? vcent[threadIdx.x] : 0.f;
  }
  __syncthreads();

  const float* __restrict__ qp = qprep + (size_t)(b * Hq + g * NREP) * G::QF;
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

  for (int t0 = tb + wave * kTile; t0 < te; t0 += 4 * kTile) {
    const int nv = min(kTile, te - t0);
    const size_t row0 = slice * cap + t0;
    // ---- 1. stage ----------------------------------------------------------------------
    stage_rows<G::WK, G::SK>(st_k, kc + row0 * G::WK, nv, lane);
    stage_rows<G::WS, G::SS>(st_s, ks + row0 * G::WS, nv, lane);
    stage_rows<G::WAK, G::SAK>(st_ak, ka + row0 * G::WAK, nv, lane);
    stage_rows<G::WV, G::SV>(st_v, vc + row0 * G::WV, nv, lane);
    stage_rows<G::WAV, G::SAV>(st_av, va + row0 * G::WAV, nv, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 2. scores: lane = token ----------------------------------------------------------
    float s2[NREP];
    {
      uint32_t kw[G::WK];
#pragma unroll
      for (int i = 0; i < G::WK; ++i) kw[i] = st_k[lane * G::SK + i];
      if constexpr (KK == TQ_K_LM_QJL) {
        uint32_t nsw[G::WS];
#pragma unroll
        for (int i = 0; i < G::WS; ++i) nsw[i] = ~st_s[lane * G::SS + i];
        const uint32_t aux = st_ak[lane * G::SAK];
        float alm[NREP], aqj[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) { alm[h] = 0.f; aqj[h] = 0.f; }
#pragma unroll
        for (int j = 0; j < D; ++j) {
          const uint32_t idx = (kw[j / G::KPER] >> (KB * (j % G::KPER))) & (LK - 1);
          const float c = s_kcent[idx];
          // sigma_j = +1 where the stored bit is 1: build +-1.0f from the inverted bit
          const float sg = __uint_as_float(((nsw[j >> 5] << (31 - (j & 31))) & 0x80000000u) | 0x3F800000u);
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
            alm[h] = fmaf(qp[h * G::QF + j], c, alm[h]);
            aqj[h] = fmaf(qp[h * G::QF + D + j], sg, aqj[h]);
          }
        }
        const float nn = f16_to_f32(aux & 0xFFFFu);
        const float gm = f16_to_f32(aux >> 16);
#pragma unroll
        for (int h = 0; h < NREP; ++h) s2[h] = nn * fmaf(gm, aqj[h], alm[h]);
      } else {
#pragma unroll
        for (int h = 0; h < NREP; ++h) s2[h] = 0.f;
#pragma unroll
        for (int gi = 0; gi < D / 32; ++gi) {
          const uint32_t aux = st_ak[lane * G::SAK + gi];
          const float a = f16_to_f32(aux & 0xFFFFu);
          const float m = f16_to_f32(aux >> 16);
          float ag[NREP];
#pragma unroll
          for (int h = 0; h < NREP; ++h) ag[h] = 0.f;
#pragma unroll
          for (int j = 32 * gi; j < 32 * gi + 32; ++j) {
            const float q8 = (float)((kw[j >> 2] >> (8 * (j & 3))) & 0xFFu);
#pragma unroll
            for (int h = 0; h < NREP; ++h) ag[h] = fmaf(qp[h * G::QF + j], q8, ag[h]);
          }
#pragma unroll
          for (int h = 0; h < NREP; ++h) s2[h] = fmaf(a, ag[h], fmaf(m, qp[h * G::QF + 3 * D + gi], s2[h]));
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
    float* dst = part + ((size_t)(b * Hq + g * NREP + h) * nsplit + split) * G::PS;
    dst[4 + j] = a;
    if (j == 0) {
      dst[0] = mx;
      dst[1] = l;
    }
  }
}

using MainLaunch = hipError_t (*)(dim3 grid, hipStream_t st, const tq_cache& C, const tq_state& S,
                                  const float* qprep, float* part, int Hkv, int n_c, int chunk, int nsplit);

template <int D, int NREP, int KK, int KB, int VK, int VB>
hipError_t main_launch(dim3 grid, hipStream_t st, const tq_cache& C, const tq_state& S, const float* qprep,
                       float* part, int Hkv, int n_c, int chunk, int nsplit) {
  hipLaunchKernelGGL((decode_main_kernel<D, NREP, KK, KB, VK, VB>), grid, dim3(256), 0, st,
                     (const uint32_t*)C.k_codes, (const uint32_t*)C.k_signs, (const uint32_t*)C.k_aux,
                     (const uint32_t*)C.v_codes, (const uint32_t*)C.v_aux, S.k_centroids, S.v_centroids,
                     qprep, part, Hkv, C.capacity, n_c, chunk, nsplit);
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

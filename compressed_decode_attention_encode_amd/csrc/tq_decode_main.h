// Fused split-K decode attention over the packed cache (gfx950, vector ALUs).
//
// Method sources: news page "vLLM, llama.cpp, MLX all follow up" (digipub.cc), oMLX
// section: attention computed straight from the packed indices, no fp16 intermediate;
// TurboQuant-MLX page (pomoai.com), GPU kernel optimisation section: query rotated once
// before scoring, weighted value sum accumulated in the rotated domain with a single
// butterfly afterwards, wave-level reductions, GQA n_rep handled without repeating KV;
// TurboQuant vLLM guide (kwkr.cn), section 2: the unbiased LM + QJL inner product.
//
// One work-group = one (batch, kv-head, split), 4 waves.  It first prepares the n_rep
// queries of its kv-head in LDS (sign flip, Walsh-Hadamard, QJL projection S q, all
// scales folded in) and turns them into lookup tables:
// a QJL table: for every 4 consecutive dimensions and each of the 16 sign patterns, the
// signed sum of the projected query for all n_rep heads (padded to 1, 2, 4 or 8 floats,
// one LDS read) -- one read replaces 4 n_rep FMAs.  The 16 entries of a 4-dimension
// block span the LDS banks once, so random entries rarely collide.  (A table over pairs
// of 3-bit codes would replace more FMAs, but its 64 entries per pair collide in the
// banks and its size halves the resident work-groups: slower on this part.)
// Then every wave takes 64-token tiles of the split in turn:
//   1. stage the tile's packed rows (every plane) from HBM into its own LDS area with
//      coalesced loads (rows padded to an odd word stride: conflict-free row reads);
//   2. scores, one token per lane, for all n_rep query heads at once;
//   3. online softmax in the log2 domain (the scales carry log2(e)/sqrt(d));
//   4. weighted value sum, 8 dimensions per lane: each decoded value element is used by
//      all n_rep heads.  Group-scaled values fold the scale into the weight, rounded to
//      fp16, and take two tokens per dot instruction (fp16 operands, exact products, fp32
//      sums), the (L-1)/2 offset going into a per-group running sum of the same weights.
//      The weight rounding moves an output by a relative 2^-12 per token, with errors of
//      independent sign; scores stay in fp32 (fp16 queries or centroids cost too much of
//      the 2e-3 attention tolerance where keys carry outlier channels).
// The four waves merge (m, l, acc) through LDS and write one partial per head.  One more
// split per (batch, kv-head) scores the exact fp16 recent buffer.  A second kernel (one
// work-group per query head) merges the partials: the kernel boundary makes them visible
// without device-wide cache flushes.
#pragma once

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtHalfPi = 1.2533141373155003f;   // sqrt(pi/2)

template <int D, int NREP, int KK, int KB, int VK, int VB>
struct DecodeGeom {
  static constexpr int KPER = (KB == 3) ? 10 : (KK == TQ_K_AFFINE8 ? (KB == 8 ? 4 : 32 / KB) : 32 / KB);
  // affine keys: bytes (8 bits), low-nibble plane + fifth-bit plane (5 bits), words of 4/2-bit codes
  static constexpr int WK = (KK == TQ_K_AFFINE8) ? (KB == 8 ? D / 4 : (KB == 5 ? D / 8 + D / 32 : D * KB / 32))
                                                 : (D + KPER - 1) / KPER;
  static constexpr int WS = (KK == TQ_K_LM_QJL) ? D / 32 : 0;
  static constexpr int WAK = (KK == TQ_K_AFFINE8) ? D / 32 : (KK == TQ_K_F16 ? 0 : 1);
  static constexpr int VPER = (VB == 3) ? 10 : 32 / VB;
  static constexpr int WV = (D + VPER - 1) / VPER;
  static constexpr int WAV = (VK == TQ_V_GROUP_SYM) ? D / 64 : (VK == TQ_V_GROUP_ASYM ? D / 32 : 1);
  // odd LDS strides
  static constexpr int odd(int w) { return w == 0 ? 0 : (w | 1); }
  static constexpr int SK = odd(WK), SS = odd(WS), SAK = odd(WAK), SV = odd(WV), SAV = odd(WAV);
  static constexpr int STAGE = kTile * (SK + SS + SAK + SV + SAV);   // words per wave
  static constexpr int LPT = D / 8;                                 // value lanes per token
  static constexpr int SLOTS = kWave / LPT;                         // tokens per value step
  static constexpr int PS = D + 4;                                  // partial stride (floats)
  // lookup tables
  static constexpr int NE = NREP == 1 ? 1 : (NREP == 2 ? 2 : (NREP <= 4 ? 4 : 8));   // floats per entry
  static constexpr int LK = (KK == TQ_K_AFFINE8 || KK == TQ_K_F16) ? 1 : (1 << KB);
  static constexpr int TQ_FLOATS = (KK == TQ_K_LM_QJL) ? (D / 4) * 16 * NE : 0;
  // LDS carve-out (floats): queries, second query block (QJL projection / affine block
  // sums), QJL table, staging, softmax weights, codebooks, merge scalars
  static constexpr int OFF_QA = 0;
  static constexpr int OFF_QB = OFF_QA + NREP * D;
  static constexpr int OFF_TQ = OFF_QB + ((NREP * D + 3) & ~3);
  static constexpr int OFF_ST = OFF_TQ + TQ_FLOATS;
  // the staging area also holds the recent split's scratch and the waves' merge buffer
  static constexpr int RECENT_SCRATCH = NREP * kMaxRecent + 2 * NREP + (256 / D) * NREP * D;
  static constexpr int STAGE_ALL = (4 * STAGE > RECENT_SCRATCH) ? 4 * STAGE : RECENT_SCRATCH;
  static constexpr int OFF_P = OFF_ST + STAGE_ALL;
  static constexpr int OFF_CENT = OFF_P + 4 * NREP * kWave;
  static constexpr int OFF_MRG = OFF_CENT + 32;
  static constexpr int FLOATS = OFF_MRG + 8 * NREP + 16;
};

// Register double-buffer for one plane of a 64-token tile: load() issues the global
// reads of the next tile (they stay in flight while the current tile is computed),
// store() later writes them into the wave's LDS area with row stride LS.  Reads never
// go past the last valid row; rows beyond it are zero-filled.
//
// DW = true: one 4-byte read per register, the index clamped to the last valid word and the
// value selected away past it -- no branch and no alignment case, so no load ever waits for an
// earlier one (the two-path form makes the compiler wait on every load in flight where the
// paths join, which serialises the prefetch behind the tile in flight).
// Fourth word of a raw buffer resource on CDNA (gfx9 family): 32-bit data format, no swizzle.
constexpr int kBufferRsrcWord3 = 0x00020000;
// cache policy of the packed-cache tile loads: non-temporal (each tile is read once per decode
// step, so it is streamed rather than kept in the caches)
constexpr int kTileLoadPolicy = 2;

template <int W, int LS, int TR = kTile, bool DW = false>
struct RowLoader {
  static constexpr int N = TR * W;                  // words per tile (TR rows)
  static constexpr int NV = (N + 4 * kWave - 1) / (4 * kWave);
  static constexpr int NR = (W == 0) ? 1 : (DW ? (N + kWave - 1) / kWave : 4 * NV);  // registers per lane
  uint32_t r[NR];
  bool vec;
  __device__ __forceinline__ void load(const uint32_t* __restrict__ g, int rows, int lane) {
    if constexpr (W == 0) return;
    if constexpr (DW) {
      const int nvalid = rows * W;                  // >= 1: a tile has at least one row
      vec = false;
      // Raw buffer loads over exactly the tile's words: the base and range live in scalar
      // registers, each lane supplies a 32-bit byte offset, and words past the range read as
      // zero (the hardware's range check), so no clamp and no select.
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(g), (short)0, 4 * nvalid, kBufferRsrcWord3);
#pragma unroll
      for (int i = 0; i < NR; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (i * kWave + lane), 0, kTileLoadPolicy);
      return;
    }
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
  // Word w of row t goes to lds[w * LS + t] instead (token-major columns: the same word
  // of consecutive rows is contiguous).
  __device__ __forceinline__ void store_transposed(uint32_t* __restrict__ lds, int lane) const {
    if constexpr (W == 0) return;
    if constexpr (DW) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int q = i * kWave + lane;
        if (q < N) lds[(q % W) * LS + (q / W)] = r[i];   // past the tile's words: zero
      }
      return;
    }
    if (vec) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = 4 * (i * kWave + lane) + k;
          if (q < N) lds[(q % W) * LS + (q / W)] = r[4 * i + k];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int q = i * kWave + lane;
        if (q < N) lds[(q % W) * LS + (q / W)] = r[i];
      }
    }
  }
  __device__ __forceinline__ void store(uint32_t* __restrict__ lds, int lane) const {
    if constexpr (W == 0) return;
    if constexpr (DW) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int q = i * kWave + lane;
        if (q < N) lds[(q / W) * LS + (q % W)] = r[i];   // past the tile's words: zero
      }
      return;
    }
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
  const uint16_t* q;                          // queries [B][Hq][d], fp16 / bf16
  const uint32_t *kc, *ks, *ka, *vc, *va;     // packed planes
  const float *kcent, *vcent;                 // codebooks (LM keys / rotated LM values)
  const uint32_t *ksign, *vsign;              // rotation signs (keys / rotated LM values)
  const uint16_t* S;                          // QJL matrix, fp16 [d][d]
  float* part;                                // partials [B][Hq][n_part][PS]
  const uint16_t *rk, *rv;                    // recent buffer [B][Hkv][recent_cap][d]
  float* out;                                 // [B][Hq][d]
  int Hq, Hkv, batch, cap, n_c, chunk, nsplit, n_part, n_recent, recent_cap, recent_bf16, q_bf16;
};

__device__ __forceinline__ float bits16_to_f32(uint32_t bits, int bf16) {
  return bf16 ? __uint_as_float(bits << 16) : f16_to_f32(bits);
}

// Query rows of one (batch, kv-head) group: NR = NQ x n_rep rows, row r = query j = r / n_rep of
// the step's NQ consecutive queries, head g n_rep + r % n_rep.  Queries are [B][NQ][Hq][d]; with
// NQ = 1 this is [B][Hq][d].  Partials are indexed by (b NQ + j, head).
template <int D, int NR, int NQ>
__device__ __forceinline__ const uint16_t* query_row(const DecodeArgs& A, int b, int g, int r) {
  constexpr int NK = NR / NQ;
  return A.q + ((size_t)(b * NQ + r / NK) * A.Hq + g * NK + r % NK) * D;
}

// NE consecutive floats of a table entry (16-byte aligned for NE >= 4).
template <int NE>
__device__ __forceinline__ void read_entry(const float* p, float (&e)[NE]) {
  if constexpr (NE == 1) {
    e[0] = p[0];
  } else if constexpr (NE == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    e[0] = v.x; e[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NE / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      e[4 * i] = v.x; e[4 * i + 1] = v.y; e[4 * i + 2] = v.z; e[4 * i + 3] = v.w;
    }
  }
}

// Query preparation for the n_rep heads h0.. of one kv-head, into LDS (256 threads):
//   LM + QJL keys: qa = Pi q * log2(e)/sqrt(d), qb = S Pi q * log2(e)/sqrt(d) * sqrt(pi/2)/d,
//                  then the QJL table;
//   affine keys:   qa = q * log2(e)/sqrt(d), qb[h][blk] = sum of qa over the 32-block.
template <int D, int NREP, int KK, int KB, int VK, int VB, bool TABLE = true, int NQ = 1>
__device__ void prepare_queries(const DecodeArgs& A, int b, int g, float* sm) {
  using G = DecodeGeom<D, NREP, KK, KB, VK, VB>;
  constexpr int NE = G::NE;
  const int tid = threadIdx.x;
  float* qa = sm + G::OFF_QA;
  float* qb = sm + G::OFF_QB;
  const float scale = kLog2e * rsqrtf((float)D);
  if constexpr (KK == TQ_K_LM_QJL || KK == TQ_K_LM_MSE) {
    constexpr bool QJL = KK == TQ_K_LM_QJL;
    // this thread's slice of S (row i, columns part*KL ..): its first reads go out first
    constexpr int KS = (256 / D) > 0 ? 256 / D : 1;
    constexpr int KL = D / KS;
    constexpr int PRE = QJL ? ((KL / 8 < 8) ? KL / 8 : 8) : 1;   // 16-byte reads issued up front
    const int i = tid / KS, part = tid % KS;
    const uint4* srow = QJL ? reinterpret_cast<const uint4*>(A.S + (size_t)i * D + part * KL) : nullptr;
    uint4 spre[PRE];
    if constexpr (QJL) {
#pragma unroll
      for (int c = 0; c < PRE; ++c) spre[c] = srow[c];
    }
    // H (s * q) per head, one wave per head: lane holds E = d/64 consecutive coordinates;
    // strides below E inside the lane, the others across lanes (xor exchanges)
    {
      constexpr int E = D / 64;
      const int lane = tid & 63, wave = tid >> 6;
      for (int h = wave; h < NREP; h += 4) {
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = lane * E + e;
          const float v = bits16_to_f32(query_row<D, NREP, NQ>(A, b, g, h)[j], A.q_bf16);
          x[e] = ((A.ksign[j >> 5] >> (j & 31)) & 1u) ? -v : v;
        }
#pragma unroll
        for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if ((e & hs) == 0) {
              const float u = x[e], v = x[e + hs];
              x[e] = u + v;
              x[e + hs] = u - v;
            }
          }
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const bool up = (lane & m) != 0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float o = __shfl_xor(x[e], m);
            x[e] = up ? (o - x[e]) : (x[e] + o);
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) qa[h * D + lane * E + e] = x[e];
      }
    }
    __syncthreads();
    // qb = S (H s q): row i of S per group of KS threads, each a 1/KS slice of k
    if constexpr (QJL) {
    {
      float acc[NREP];
#pragma unroll
      for (int h = 0; h < NREP; ++h) acc[h] = 0.f;
      if (i < D) {
#pragma unroll 2
        for (int k8 = 0; k8 < KL / 8; ++k8) {
          uint4 sv;
          if (k8 < PRE) {
#pragma unroll
            for (int c = 0; c < PRE; ++c)
              if (c == k8) sv = spre[c];
          } else {
            sv = srow[k8];
          }
          const uint32_t w[4] = {sv.x, sv.y, sv.z, sv.w};
          float sf[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            sf[2 * t] = f16_to_f32(w[t] & 0xFFFFu);
            sf[2 * t + 1] = f16_to_f32(w[t] >> 16);
          }
          const int k0 = part * KL + 8 * k8;
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[h] = fmaf(sf[t], qa[h * D + k0 + t], acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        if constexpr (KS >= 2) acc[h] += xor_lanes<1>(acc[h]);
        if constexpr (KS >= 4) acc[h] += xor_lanes<2>(acc[h]);
      }
      const float sq = rsqrtf((float)D) * scale * (kSqrtHalfPi / (float)D);
      if (i < D && part == 0) {
#pragma unroll
        for (int h = 0; h < NREP; ++h) qb[h * D + i] = acc[h] * sq;
      }
    }
    }
    __syncthreads();
    for (int i = tid; i < NREP * D; i += 256) qa[i] *= rsqrtf((float)D) * scale;
    __syncthreads();
    // QJL table: entry (nib, v), head h = sum_t (bit t of v ? +1 : -1) qb[h][4 nib + t]
    float* tq = sm + G::OFF_TQ;
    for (int i = tid; QJL && TABLE && i < (D / 4) * 16; i += 256) {
      const int nib = i / 16, v = i % 16;
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        const float* qq = qb + h * D + 4 * nib;
        float a = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) a += ((v >> t) & 1) ? qq[t] : -qq[t];
        tq[i * NE + h] = a;
      }
    }
  } else {
    for (int i = tid; i < NREP * D; i += 256)
      qa[i] = bits16_to_f32(query_row<D, NREP, NQ>(A, b, g, i / D)[i % D], A.q_bf16) * scale;
    __syncthreads();
    for (int i = tid; KK == TQ_K_AFFINE8 && i < NREP * (D / 32); i += 256) {
      const int h = i / (D / 32), blk = i % (D / 32);
      float s = 0.f;
      for (int k = 0; k < 32; ++k) s += qa[h * D + 32 * blk + k];
      qb[i] = s;
    }
  }
  __syncthreads();
}

// Write (m, l, acc[d]) of head h0 + h (partial index `pi`) from LDS-merged values.
template <int D>
__device__ __forceinline__ float* partial_ptr(const DecodeArgs& A, int b, int head, int pi) {
  return A.part + ((size_t)(b * A.Hq + head) * A.n_part + pi) * (D + 4);
}

// The exact recent tokens of kv-head g (n_recent >= 1): scores with the natural-domain
// query, softmax, value sum (natural domain), one partial per head at index nsplit.  Every
// global read is issued on entry, before any is used: two threads per token row (half a
// row each) for the scores, and value columns as thread = (dimension, token subset), 32
// rows at a time.
//
// With NQ > 1 (multi-query groups, NREP = NQ x n_rep rows) the last NQ recent tokens are the
// queries' own, in order, and query j sees recent tokens 0 .. R - NQ + j (causal inside the
// suffix); R >= NQ is checked on the host, so every row sees at least one token.
// SCR: float offset of its scratch in the work-group's LDS (by default the staging area of
// the vector-ALU kernel; the matrix-core kernel places it right after the queries).
template <int D, int NREP, int KK, int KB, int VK, int VB, int NQ = 1, int SCR = -1>
__device__ void recent_split(const DecodeArgs& A, int b, int g, float* sm) {
  using G = DecodeGeom<D, NREP, KK, KB, VK, VB>;
  static_assert(kMaxRecent * 2 <= 256, "two threads per recent token");
  constexpr int NG = 256 / D;                 // threads per dimension in the value sums
  constexpr int VCH = 32;                     // value rows in flight per thread
  constexpr int HU = D / 16;                  // 16-byte reads per half row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = A.n_recent;
  const int bf = A.recent_bf16;
  float* qn = sm + G::OFF_QA;
  float* sr = sm + (SCR >= 0 ? SCR : G::OFF_ST);   // [NREP][kMaxRecent] scores -> weights
  float* sML = sr + NREP * kMaxRecent;        // [NREP] max, [NREP] normaliser
  float* sacc = sML + 2 * NREP;               // [NG][NREP][D] partial value sums
  static_assert(SCR >= 0 || G::STAGE_ALL >= NREP * kMaxRecent + 2 * NREP + NG * NREP * D,
                "recent scratch does not fit the staging area");
  const size_t rbase = ((size_t)b * A.Hkv + g) * A.recent_cap;
  // Reads past the last row are clamped to it (never out of bounds, never a branch
  // around a load: that would make the compiler wait on each load in turn) and their
  // values are not used.
  // key half rows
  const int r_k = tid >> 1, half = tid & 1;
  uint4 kr[HU];
  {
    const uint4* src = reinterpret_cast<const uint4*>(A.rk + (rbase + min(r_k, R - 1)) * D + half * (D / 2));
#pragma unroll
    for (int c = 0; c < HU; ++c) kr[c] = src[c];
  }
  // first block of value rows (fp16 / bf16 bits, one per register)
  const int j = tid % D, grp = tid / D;
  uint32_t vv[VCH];
#pragma unroll
  for (int i = 0; i < VCH; ++i) vv[i] = A.rv[(rbase + min(grp + NG * i, R - 1)) * D + j];
  const float scale = kLog2e * rsqrtf((float)D);
  for (int i = tid; i < NREP * D; i += 256)
    qn[i] = bits16_to_f32(query_row<D, NREP, NQ>(A, b, g, i / D)[i % D], A.q_bf16) * scale;
  __syncthreads();
  // scores: each thread dots its half row with every head, the pair adds its halves
#pragma unroll 1
  for (int h = 0; h < NREP; ++h) {
    const float* q = qn + h * D + half * (D / 2);
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < HU; ++c) {
      const uint32_t w[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a = fmaf(q[8 * c + 2 * k], bits16_to_f32(w[k] & 0xFFFFu, bf), a);
        a = fmaf(q[8 * c + 2 * k + 1], bits16_to_f32(w[k] >> 16, bf), a);
      }
    }
    a += xor_lanes<1>(a);
    if (half == 0 && r_k < R) sr[h * kMaxRecent + r_k] = (r_k <= R - NQ + h / (NREP / NQ)) ? a : -INFINITY;
  }
  __syncthreads();
  for (int h = wave; h < NREP; h += 4) {
    float mx = -INFINITY;
    for (int r = lane; r < R; r += 64) mx = fmaxf(mx, sr[h * kMaxRecent + r]);
    mx = wave_max(mx);
    float l = 0.f;
    for (int r = lane; r < R; r += 64) {
      const float p = exp2f(sr[h * kMaxRecent + r] - mx);
      sr[h * kMaxRecent + r] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { sML[h] = mx; sML[NREP + h] = l; }
  }
  __syncthreads();
  // value sums: thread (j, grp) over tokens grp, grp + NG, ... for every head
  float acc[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) acc[h] = 0.f;
  for (int r0 = 0; r0 < R; r0 += NG * VCH) {
    if (r0 > 0) {
#pragma unroll
      for (int i = 0; i < VCH; ++i) vv[i] = A.rv[(rbase + min(r0 + grp + NG * i, R - 1)) * D + j];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int r = r0 + grp + NG * i;   // uniform over a wave (grp is)
      if (r < R) {
        const float v = bits16_to_f32(vv[i], bf);
#pragma unroll
        for (int h = 0; h < NREP; ++h) acc[h] = fmaf(sr[h * kMaxRecent + r], v, acc[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NREP; ++h) sacc[(grp * NREP + h) * D + j] = acc[h];
  __syncthreads();
  for (int i = tid; i < NREP * D; i += 256) {
    const int h = i / D, jj = i % D;
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) a += sacc[(q * NREP + h) * D + jj];
    constexpr int NK = NREP / NQ;
    float* dst = partial_ptr<D>(A, b * NQ + h / NK, g * NK + h % NK, A.nsplit);
    dst[4 + jj] = a;
    if (jj == 0) { dst[0] = sML[h]; dst[1] = sML[NREP + h]; }
  }
}

template <int D, int NREP, int KK, int KB, int VK, int VB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_main_kernel(const DecodeArgs A) {
  using G = DecodeGeom<D, NREP, KK, KB, VK, VB>;
  constexpr int LK = 1 << KB;
  constexpr int LV = 1 << VB;
  constexpr int NE = G::NE;

  __shared__ __attribute__((aligned(16))) float sm[G::FLOATS];
  // the four waves' value sums reuse the staging area once the tile loop is done
  static_assert(G::STAGE_ALL >= 4 * NREP * D, "merge buffer does not fit in the staging area");
  static_assert(VK != TQ_V_GROUP_SYM || VB == 2 || VB == 4, "group-scaled values are 2 or 4 bits");
  static_assert((kTile / G::SLOTS) % 2 == 0, "value steps go in token pairs");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // 1-D grid: the n_splits x (batch, kv-head) compressed groups first, then one short
  // recent-buffer group per (batch, kv-head), dispatched last: they take the slots of the
  // first compressed groups to finish
  const int n_comp = A.nsplit * A.Hkv * A.batch;
  if ((int)blockIdx.x >= n_comp) {
    const int u = blockIdx.x - n_comp;
    recent_split<D, NREP, KK, KB, VK, VB>(A, u / A.Hkv, u % A.Hkv, sm);
    return;
  }
  const int split = blockIdx.x % A.nsplit;
  const int g = (blockIdx.x / A.nsplit) % A.Hkv;
  const int b = blockIdx.x / (A.nsplit * A.Hkv);

  float* s_kcent = sm + G::OFF_CENT;
  float* s_vcent = s_kcent + 16;
  if (threadIdx.x < 16) {
    if constexpr (KK == TQ_K_LM_QJL || KK == TQ_K_LM_MSE)
      s_kcent[threadIdx.x] = (threadIdx.x < LK) ? A.kcent[threadIdx.x] : 0.f;
    if constexpr (VK == TQ_V_LM_ROT) s_vcent[threadIdx.x] = (threadIdx.x < LV) ? A.vcent[threadIdx.x] : 0.f;
  }
  const float* qa = sm + G::OFF_QA;
  const float* qb = sm + G::OFF_QB;
  const float* tq = sm + G::OFF_TQ;
  const int Hkv = A.Hkv, cap = A.cap, n_c = A.n_c, chunk = A.chunk;
  const uint32_t* __restrict__ kc = A.kc;
  const uint32_t* __restrict__ ks = A.ks;
  const uint32_t* __restrict__ ka = A.ka;
  const uint32_t* __restrict__ vc = A.vc;
  const uint32_t* __restrict__ va = A.va;

  const size_t slice = (size_t)b * Hkv + g;
  const int tb = split * chunk;
  const int te = min(n_c, tb + chunk);

  uint32_t* stage = reinterpret_cast<uint32_t*>(sm + G::OFF_ST);
  uint32_t* st_k = stage + wave * G::STAGE;
  uint32_t* st_s = st_k + kTile * G::SK;
  uint32_t* st_ak = st_s + kTile * G::SS;
  uint32_t* st_v = st_ak + kTile * G::SAK;
  uint32_t* st_av = st_v + kTile * G::SV;
  float* sp = sm + G::OFF_P + wave * NREP * kWave;

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
  // the first tile's loads overlap the query preparation
  if (tb + wave * kTile < te) issue(tb + wave * kTile);
  prepare_queries<D, NREP, KK, KB, VK, VB>(A, b, g, sm);

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
    float s2[NREP];
    {
      const uint32_t* krow = st_k + lane * G::SK;
      if constexpr (KK == TQ_K_F16) {
        // 16-bit keys (V-only mode): <q, k> over the stored row, 8 dimensions (4 words)
        // per trip, keys in the query's storage type
#pragma unroll
        for (int h = 0; h < NREP; ++h) s2[h] = 0.f;
        auto score_rows = [&](auto bf) {
#pragma unroll 1
          for (int j0 = 0; j0 < D; j0 += 8) {
            const uint32_t w[4] = {krow[j0 / 2], krow[j0 / 2 + 1], krow[j0 / 2 + 2], krow[j0 / 2 + 3]};
            float kv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (decltype(bf)::value) {
                kv[2 * i] = __uint_as_float(w[i] << 16);
                kv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
              } else {
                kv[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
                kv[2 * i + 1] = f16_to_f32(w[i] >> 16);
              }
            }
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              const float4 q0 = *reinterpret_cast<const float4*>(qa + h * D + j0);
              const float4 q1 = *reinterpret_cast<const float4*>(qa + h * D + j0 + 4);
              float a = s2[h];
              a = fmaf(q0.x, kv[0], a); a = fmaf(q0.y, kv[1], a); a = fmaf(q0.z, kv[2], a); a = fmaf(q0.w, kv[3], a);
              a = fmaf(q1.x, kv[4], a); a = fmaf(q1.y, kv[5], a); a = fmaf(q1.z, kv[6], a); a = fmaf(q1.w, kv[7], a);
              s2[h] = a;
            }
          }
        };
        if (A.q_bf16) score_rows(std::true_type{});
        else score_rows(std::false_type{});
      } else if constexpr (KK != TQ_K_AFFINE8) {
        constexpr bool QJL = KK == TQ_K_LM_QJL;   // MSE-only keys: the codebook term alone
        const uint32_t aux = st_ak[lane * G::SAK];
        float alm[NREP], aqj[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) { alm[h] = 0.f; aqj[h] = 0.f; }
        // QJL term: one table entry per 4 dimensions (stored bit 1 <=> sigma = +1)
        if constexpr (NREP <= 4) {
          // QJL and codebook terms together, every LDS read issued one chunk (8 dimensions)
          // ahead of its use: the row's code and sign words first, then per chunk its 8
          // centroids, its 2 QJL entries and its query values.  With one token per lane
          // and two waves per SIMD, little else can hide the LDS latency.
          constexpr int CH = 8;
          constexpr int NCH = D / CH;
          const uint32_t* srow = st_s + lane * G::SS;
          uint32_t kw[G::WK], sw[QJL ? D / 32 : 1];
#pragma unroll
          for (int w = 0; w < G::WK; ++w) kw[w] = krow[w];
          if constexpr (QJL) {
#pragma unroll
            for (int w = 0; w < D / 32; ++w) sw[w] = srow[w];
          }
          float cb[2][CH], qj[2][2][NE];
          float4 qv[2][NREP][2];
          auto fetch = [&](int c, int buf) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
              const int j = c * CH + i;
              cb[buf][i] = s_kcent[(kw[j / G::KPER] >> (KB * (j % G::KPER))) & (LK - 1)];
            }
            if constexpr (QJL) {
#pragma unroll
              for (int n = 0; n < 2; ++n) {
                const int blk = 2 * c + n;
                const uint32_t v = (sw[blk / 8] >> (4 * (blk % 8))) & 15u;
                read_entry<NE>(tq + (blk * 16 + v) * NE, qj[buf][n]);
              }
            }
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              qv[buf][h][0] = *reinterpret_cast<const float4*>(qa + h * D + c * CH);
              qv[buf][h][1] = *reinterpret_cast<const float4*>(qa + h * D + c * CH + 4);
            }
          };
          fetch(0, 0);
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const int cur = c & 1;
            if (c + 1 < NCH) fetch(c + 1, cur ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              const float4 q0 = qv[cur][h][0], q1 = qv[cur][h][1];
              const float* cc = cb[cur];
              float a = alm[h];
              a = fmaf(q0.x, cc[0], a); a = fmaf(q0.y, cc[1], a); a = fmaf(q0.z, cc[2], a); a = fmaf(q0.w, cc[3], a);
              a = fmaf(q1.x, cc[4], a); a = fmaf(q1.y, cc[5], a); a = fmaf(q1.z, cc[6], a); a = fmaf(q1.w, cc[7], a);
              alm[h] = a;
              if constexpr (QJL) aqj[h] += qj[cur][0][h] + qj[cur][1][h];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (QJL) {
          // n_rep > 4: reads go out in batches into separate registers, the next batch
          // before the current one is added, so their LDS latencies overlap
          const uint32_t* srow = st_s + lane * G::SS;
          constexpr int NB = D / 4;                       // 4-dimension blocks
          constexpr int QB = 4;                           // entries per batch
          uint32_t sw[D / 32];
#pragma unroll
          for (int w = 0; w < D / 32; ++w) sw[w] = srow[w];
          float e[2][QB][NE];
          auto fetch = [&](int b0, float (&dst)[QB][NE]) {
#pragma unroll
            for (int k = 0; k < QB; ++k) {
              const int blk = b0 + k;
              const uint32_t v = (sw[blk / 8] >> (4 * (blk % 8))) & 15u;
              read_entry<NE>(tq + (blk * 16 + v) * NE, dst[k]);
            }
          };
          fetch(0, e[0]);
#pragma unroll
          for (int b0 = 0; b0 < NB; b0 += QB) {
            const int cur = (b0 / QB) & 1;
            if (b0 + QB < NB) fetch(b0 + QB, e[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < QB; ++k)
#pragma unroll
              for (int h = 0; h < NREP; ++h) aqj[h] += e[cur][k][h];
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (NREP > 4) {
          // codebook term for n_rep > 4: the row's code words are read once; chunks of 4
          // codes read their centroids and query values as one batch before the FMAs
          constexpr int CH = 4;
          constexpr int NCH = D / CH;
          uint32_t kw[G::WK];
#pragma unroll
          for (int w = 0; w < G::WK; ++w) kw[w] = krow[w];
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            float cb[CH], qv[NREP][CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
              const int j = c * CH + i;
              const uint32_t code = (kw[j / G::KPER] >> (KB * (j % G::KPER))) & (LK - 1);
              cb[i] = s_kcent[code];
            }
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              const float4 q4 = *reinterpret_cast<const float4*>(qa + h * D + c * CH);
              qv[h][0] = q4.x; qv[h][1] = q4.y; qv[h][2] = q4.z; qv[h][3] = q4.w;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              float a = alm[h];
#pragma unroll
              for (int i = 0; i < CH; ++i) a = fmaf(qv[h][i], cb[i], a);
              alm[h] = a;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (QJL) {
          const float nn = f16_to_f32(aux & 0xFFFFu);
          const float gm = f16_to_f32(aux >> 16);
#pragma unroll
          for (int h = 0; h < NREP; ++h) s2[h] = nn * fmaf(gm, aqj[h], alm[h]);
        } else {
          const float nn = __uint_as_float(aux);   // fp32 n
#pragma unroll
          for (int h = 0; h < NREP; ++h) s2[h] = nn * alm[h];
        }
      } else {
        float ag[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) { s2[h] = 0.f; ag[h] = 0.f; }
#pragma unroll 1
        for (int j0 = 0; j0 < D; j0 += 8) {
          const uint32_t w0 = krow[j0 / 4], w1 = krow[j0 / 4 + 1];
          float c[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            c[i] = (float)((w0 >> (8 * i)) & 0xFFu);
            c[4 + i] = (float)((w1 >> (8 * i)) & 0xFFu);
          }
#pragma unroll
          for (int h = 0; h < NREP; ++h) {
            const float4 q0 = *reinterpret_cast<const float4*>(qa + h * D + j0);
            const float4 q1 = *reinterpret_cast<const float4*>(qa + h * D + j0 + 4);
            float a = ag[h];
            a = fmaf(q0.x, c[0], a); a = fmaf(q0.y, c[1], a); a = fmaf(q0.z, c[2], a); a = fmaf(q0.w, c[3], a);
            a = fmaf(q1.x, c[4], a); a = fmaf(q1.y, c[5], a); a = fmaf(q1.z, c[6], a); a = fmaf(q1.w, c[7], a);
            ag[h] = a;
          }
          if (((j0 + 8) & 31) == 0) {   // end of a 32-block: fold in its scale and offset
            const int gi = j0 >> 5;
            const uint32_t aux = st_ak[lane * G::SAK + gi];
            const float a = f16_to_f32(aux & 0xFFFFu);
            const float m = f16_to_f32(aux >> 16);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
              s2[h] = fmaf(a, ag[h], fmaf(m, qb[h * (D / 32) + gi], s2[h]));
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
    if constexpr (VK == TQ_V_GROUP_SYM) {
      // two token slots per step.  Each token's weight (softmax weight times the group
      // scale) is rounded once to fp16, the pair packed; each code c becomes the fp16 value
      // 1 + c / 2^MV (the code dropped into the top mantissa bits under the exponent of
      // 1.0), the two tokens' values of one dimension packed alike; one dot instruction
      // adds both tokens' terms in fp32.  off[h] sums the same fp16 weights, so the 1 and
      // the (L-1)/2 offset are taken out exactly after the loop.
      constexpr uint32_t kOne = 0x3C003C00u;     // fp16 pair (1, 1)
      const int gi = prt / 4;                     // 32-group of these 8 dimensions
#pragma unroll 1
      for (int stp = 0; stp < kTile / G::SLOTS; stp += 2) {
        const int t1 = stp * G::SLOTS + slot, t2 = t1 + G::SLOTS;
        const uint32_t aw1 = st_av[t1 * G::SAV + (gi >> 1)], aw2 = st_av[t2 * G::SAV + (gi >> 1)];
        const float dl1 = f16_to_f32((aw1 >> (16 * (gi & 1))) & 0xFFFFu);
        const float dl2 = f16_to_f32((aw2 >> (16 * (gi & 1))) & 0xFFFFu);
        uint32_t wp[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          wp[h] = pack_f16x2(sp[h * kWave + t1] * dl1, sp[h * kWave + t2] * dl2);
          off[h] = dot2_f16(wp[h], kOne, off[h]);
        }
        uint32_t y[8];
        if constexpr (VB == 2) {
          // this lane's 8 codes are one half-word of each row: token 1's half below token
          // 2's, code e at bits 2e of its half, moved to the mantissa bits 8..9
          const uint32_t c1 = st_v[t1 * G::SV + (prt >> 1)], c2 = st_v[t2 * G::SV + (prt >> 1)];
          const uint32_t x = __builtin_amdgcn_perm(c2, c1, (prt & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t m = (e < 4) ? (x << (8 - 2 * e)) : (x >> (2 * e - 8));
            y[e] = (m & 0x03000300u) | kOne;
          }
        } else {
          // 4-bit codes: the 8 codes fill the word; the low and the high half-words of the
          // two rows are paired, code e at bits 4 (e % 4) of its half, moved to bits 6..9
          const uint32_t c1 = st_v[t1 * G::SV + prt], c2 = st_v[t2 * G::SV + prt];
          const uint32_t xl = __builtin_amdgcn_perm(c2, c1, 0x05040100u);
          const uint32_t xh = __builtin_amdgcn_perm(c2, c1, 0x07060302u);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t x = (e < 4) ? xl : xh;
            const int sh = 6 - 4 * (e % 4);
            const uint32_t m = (sh >= 0) ? (x << sh) : (x >> (-sh));
            y[e] = (m & 0x03C003C0u) | kOne;
          }
        }
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = dot2_f16(wp[h], y[e], acc[h][e]);
        }
      }
    } else {
#pragma unroll 2
      for (int stp = 0; stp < kTile / G::SLOTS; ++stp) {
        const int t = stp * G::SLOTS + slot;
        float pw[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) pw[h] = sp[h * kWave + t];
        float cv[8];
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
      // acc = sum w (1 + c / 2^MV), off = sum w  ->  sum w (c - (L-1)/2)
      constexpr float F = (VB == 2) ? 4.f : 16.f;
      const float o = (F + 0.5f * (float)(LV - 1)) * off[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(F, acc[h][e], -o);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int m = G::LPT; m < kWave; m <<= 1) acc[h][e] += __shfl_xor(acc[h][e], m);
    }
  }
  __syncthreads();   // every wave is done with its staging area
  float(*s_mrg_acc)[NREP * D] = reinterpret_cast<float(*)[NREP * D]>(stage);
  float* s_mrg_m = sm + G::OFF_MRG;            // [4][NREP]
  float* s_mrg_l = s_mrg_m + 4 * NREP;         // [4][NREP]
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
      s_mrg_m[wave * NREP + h] = m_run[h];
      s_mrg_l[wave * NREP + h] = l_run[h];
    }
  }
  __syncthreads();

  // ---- merge the four waves, write one partial per head ----------------------------------
  for (int i = threadIdx.x; i < NREP * D; i += blockDim.x) {
    const int h = i / D, j = i % D;
    float mx = s_mrg_m[h];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, s_mrg_m[w * NREP + h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_mrg_m[w * NREP + h];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - mx);
      a = fmaf(s_mrg_acc[w][h * D + j], sc, a);
      l = fmaf(s_mrg_l[w * NREP + h], sc, l);
    }
    float* dst = partial_ptr<D>(A, b, g * NREP + h, split);
    dst[4 + j] = a;
    if (j == 0) {
      dst[0] = mx;
      dst[1] = l;
    }
  }
}

// One instantiation: its launcher and its resident work-groups per CU.
struct MainKernel {
  hipError_t (*launch)(dim3 grid, hipStream_t st, const DecodeArgs& A);
  int (*blocks_per_cu)();
};

template <int D, int NREP, int KK, int KB, int VK, int VB>
hipError_t main_launch(dim3 grid, hipStream_t st, const DecodeArgs& A) {
  hipLaunchKernelGGL((decode_main_kernel<D, NREP, KK, KB, VK, VB>), grid, dim3(256), 0, st, A);
  return hipGetLastError();
}

template <int D, int NREP, int KK, int KB, int VK, int VB>
int main_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode_main_kernel<D, NREP, KK, KB, VK, VB>, 256, 0) !=
            hipSuccess || b <= 0)
      b = 1;
    return b;
  }();
  return n;
}

template <int D, int NREP, int KK, int KB, int VK, int VB>
constexpr MainKernel main_kernel() {
  return MainKernel{&main_launch<D, NREP, KK, KB, VK, VB>, &main_blocks_per_cu<D, NREP, KK, KB, VK, VB>};
}

// Lookup of the compiled instantiations (one file per key kind and head_dim).
MainKernel find_main_lm2_d64(int nrep, int vk, int vb);
MainKernel find_main_lm3_d64(int nrep, int vk, int vb);
MainKernel find_main_lm4_d64(int nrep, int vk, int vb);
MainKernel find_main_aff8_d64(int nrep, int vk, int vb);
MainKernel find_main_lm2_d128(int nrep, int vk, int vb);
MainKernel find_main_lm3_d128(int nrep, int vk, int vb);
MainKernel find_main_lm4_d128(int nrep, int vk, int vb);
MainKernel find_main_aff8_d128(int nrep, int vk, int vb);
MainKernel find_main_aff2_d64(int nrep, int vk, int vb);
MainKernel find_main_aff4_d64(int nrep, int vk, int vb);
MainKernel find_main_aff5_d64(int nrep, int vk, int vb);
MainKernel find_main_aff2_d128(int nrep, int vk, int vb);
MainKernel find_main_aff4_d128(int nrep, int vk, int vb);
MainKernel find_main_aff5_d128(int nrep, int vk, int vb);
MainKernel find_main_lm2_d256(int nrep, int vk, int vb);
MainKernel find_main_lm3_d256(int nrep, int vk, int vb);
MainKernel find_main_lm4_d256(int nrep, int vk, int vb);
MainKernel find_main_aff8_d256(int nrep, int vk, int vb);
MainKernel find_main_lmm2_d64(int nrep, int vk, int vb);
MainKernel find_main_lmm3_d64(int nrep, int vk, int vb);
MainKernel find_main_lmm4_d64(int nrep, int vk, int vb);
MainKernel find_main_lmm2_d128(int nrep, int vk, int vb);
MainKernel find_main_lmm3_d128(int nrep, int vk, int vb);
MainKernel find_main_lmm4_d128(int nrep, int vk, int vb);
MainKernel find_main_lmm2_d256(int nrep, int vk, int vb);
MainKernel find_main_lmm3_d256(int nrep, int vk, int vb);
MainKernel find_main_lmm4_d256(int nrep, int vk, int vb);
MainKernel find_main_f16_d64(int nrep, int vk, int vb);
MainKernel find_main_f16_d128(int nrep, int vk, int vb);
// 16-bit keys in fp16 storage on the matrix cores (n_rep 3..8)
MainKernel find_mma_f16_d64(int nrep, int vk, int vb);
MainKernel find_mma_f16_d256(int nrep, int vk, int vb);
// head_dim 512: every key / value kind on vector-ALU kernels, n_rep <= 8
MainKernel find_main_d512(const tq_layout& L);
// multi-query groups (LM + QJL keys, group values): n_rep heads x nq queries, vb value bits
MainKernel find_multi_lm3_d64(int nrep, int nq, int vb);
MainKernel find_multi_lm4_d64(int nrep, int nq, int vb);
MainKernel find_multi_lm3_d128(int nrep, int nq, int vb);
MainKernel find_multi_lm4_d128(int nrep, int nq, int vb);

}  // namespace tq

// Split-K decode attention on the fp16 matrix cores, for Lloyd-Max + QJL keys and
// group-32 symmetric values (gfx950, v_mfma_f32_16x16x32_f16).
//
// Same method, split plan, partial format and recent-buffer split as tq_decode_main.h
// (news page "vLLM, llama.cpp, MLX all follow up", oMLX section: attention straight from
// the packed indices; TurboQuant-MLX page, GPU kernel optimisation section: pre-rotated
// query, GQA without repeating KV; TurboQuant vLLM guide, section 2: the LM + QJL inner
// product <q, k> = n (<Pi q, c[idx]> + gamma sqrt(pi/2)/d <S Pi q, sigma>)).  What changes
// is how a 64-token tile is reduced.  With n_rep query heads per kv-head, both products of
// a tile are dense contractions once a code is replaced by its value:
//
//   scores  S^T[token, head] = A[token, k] B[k, head], the contraction index k running
//           over five blocks of d dimensions:
//             A = c_hi[idx]  B = q_hi        A = c_lo[idx]  B = q_hi
//             A = c_hi[idx]  B = q_lo        A = gamma*sigma  B = qb_hi,  A = gamma*sigma  B = qb_lo
//           where c_hi/c_lo are the fp16 halves of 8 c (a 21-bit centroid), q_hi/q_lo those
//           of the scaled rotated query and qb_hi/qb_lo those of the scaled projected query;
//           gamma*sigma is the key's fp16 gamma with the sign of its QJL bit, exact in fp16.
//           Every product is exact in fp32; the dropped c_lo q_lo term is ~2^-22 relative.
//           The token's norm n (and a power-of-two unscale) multiplies the sum afterwards.
//   values O[head, dim] = P'[head, token] V[token, dim] per 32-dimension group, with
//           P' = fp16(p * Delta) (the softmax weight times the token's group scale, rounded
//           once as in the vector-ALU kernel) and V the fp16 value 1 + c/2^m of the code
//           (exact); sum_t P' (the offset term) comes from fp16 dot instructions on the same
//           rounded weights, and F*O - (F + (L-1)/2) * sum P' is the group-dequantised sum.
//
// Operand layouts (16x16x32 f16): A lane l holds row l%16, k = 8(l/16)..+7; B lane l holds
// column l%16, the same k; C lane l holds column l%16, rows 4(l/16)..+3.  The k order inside a
// 32-wide block is free as long as A and B agree: the value product takes the 8 tokens
// {4q..4q+3, 16+4q..16+4q+3} (q = l/16) of a 32-token block, which are exactly the rows a
// lane holds in the score accumulators of two 16-token blocks, so softmax weights go from the
// score accumulators to the value operands without leaving the lane.
//
// Per-block affine 8-bit keys (vllm-metal guide, quantisation principle) take the same path with
// the codes themselves as exact fp16 operands (c - 128, from a byte permute and one packed fp16
// add) and the block's scale and offset applied to each 32-dimension partial sum:
//   s = sum_blk a (sum_j (c_j - 128) q_j) + (m + 128 a) sum_j q_j.
// Group-32 min/max values (benchmark page, compression details) reuse the group path with
// a = the group's step and an extra fp32 sum of p m per group (the offset term).
// Rotated Lloyd-Max values (vllm-metal guide; TurboQuant-MLX page: 3-bit codes ten per word) use
// P'' = p n (hi/lo fp16) against the centroid values (hi/lo, through a value code-pair table);
// their sum stays in the rotated domain for the merge kernel's single inverse butterfly.
//
// Codes become operands through LDS tables: a (hi pair, lo pair) entry per pair of 2/3-bit
// codes; for 4-bit codes read straight into registers a (hi, lo) word per single code, paired
// with a query operand that holds every value twice; and a 16-byte entry of four fp16 +-1
// pairs per 8 sign bits.  The next tile's loads are in flight through the current tile; group
// value codes are staged row-major and read back with the transposing LDS read.
#pragma once

#include "tq_decode_main.h"

namespace tq {

typedef _Float16 mma_h8_t __attribute__((ext_vector_type(8)));
typedef float mma_f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t mma_u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mma_f4_t mma16(mma_u4_t a, mma_u4_t b, mma_f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mma_h8_t, a), __builtin_bit_cast(mma_h8_t, b),
                                                c, 0, 0, 0);
}

typedef __bf16 mma_b8_t __attribute__((ext_vector_type(8)));

// x of lane l + S within the lane's row of 16 (zero past the row's end)
template <int S>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + S, 0xF, 0xF, true));
}

__device__ __forceinline__ mma_f4_t mma16_bf(mma_u4_t a, mma_u4_t b, mma_f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mma_b8_t, a), __builtin_bit_cast(mma_b8_t, b),
                                                 c, 0, 0, 0);
}

// float -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Operand scales: centroids x 8 (O(1) values, fp16 halves both normal); the query operands
// carry 2^8 / 8 (codebook) and 2^8 (QJL) so that the sum is 2^8 times the log2-domain score.
constexpr float kMmaCentScale = 8.f;
constexpr float kMmaQScale = 256.f;
constexpr float kMmaUnscale = 1.f / 256.f;
constexpr float kMmaAffQScale = 16.f;        // affine keys: query operands carry 16

// fp16 pair (fp16(a x), fp16(b y)) of float a, b and the fp16 x, y held in half `hf` of words
// dx, dy: the mixed-precision multiply-add rounds each product to fp16 once
__device__ __forceinline__ uint32_t mul_f32_f16_pair(float a, uint32_t dx, float b, uint32_t dy, int hf) {
  uint32_t r;
  if (hf == 0) {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(dx));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(b), "v"(dy));
  } else {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(dx));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(b), "v"(dy));
  }
  return r;
}

// (a, b) -> fp16 hi pair and the pair of their fp16 remainders (a - hi_a, b - hi_b)
__device__ __forceinline__ void split_f16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  f16x2_t h, l;
  h.x = (_Float16)a;
  h.y = (_Float16)b;
  l.x = (_Float16)(a - (float)h.x);
  l.y = (_Float16)(b - (float)h.y);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

template <int D, int NREP, int KK, int KB, int VK, int VB, int TT = kTile>
struct MmaGeom {
  using G = DecodeGeom<D, NREP, KK, KB, VK, VB>;
  static constexpr bool QJL = KK == TQ_K_LM_QJL;
  static constexpr bool AFF = KK == TQ_K_AFFINE8;
  static constexpr bool F16K = KK == TQ_K_F16;  // 16-bit keys, used as stored (fp16 storage only)
  static constexpr int KPER = G::KPER, WK = G::WK;
  static constexpr int SK = F16K ? WK + 4 : G::SK;   // 16-bit rows: 16-byte aligned row stride
  static constexpr int WS = G::WS, SS = G::SS;
  static constexpr int WAK = G::WAK;            // key aux words per token: (n, gamma) / fp32 n / (a, m) per block
  static constexpr int WV = G::WV, WAV = G::WAV;
  static constexpr int TS = TT + 4;           // token stride of the transposed value planes
  static constexpr int NKB = D / 32;          // 32-dimension blocks of the score contraction
  static constexpr int NNB = D / 16;          // 16-dimension blocks of the value product
  static constexpr int NG = D / 32;           // value groups
  // Lloyd-Max keys (with or without the QJL sketch) at head_dim >= 128 come straight from
  // memory into registers in the matrix-core operand order; affine and 16-bit keys, and the
  // head_dim-64 rows (too short to keep four lanes' loads busy), are staged in LDS
  static constexpr bool DIRECT = !AFF && !F16K && D >= 128;
  // one wave's staging area (words): key rows, sign rows, key aux (word-major [block][token]
  // for affine keys), value codes and value aux word-major
  // group values (symmetric or min/max) in 64-token tiles: code rows kept row-major in LDS (a
  // two-word pad per row) and read back transposed, scale rows row-major and dense
  static constexpr bool TRV = VK != TQ_V_LM_ROT && TT == 64;
  static constexpr int LSV = WV + 2;
  static constexpr int OFF_SK = 0;
  static constexpr int OFF_SS = OFF_SK + (DIRECT ? 0 : TT * SK);
  static constexpr int OFF_SAK = OFF_SS + (DIRECT ? 0 : TT * SS);
  static constexpr int OFF_SV = OFF_SAK + (DIRECT ? 0 : (AFF ? WAK * TS : TT));
  static constexpr int OFF_SAV = OFF_SV + (TRV ? TT * LSV : WV * TS);
  static constexpr int STAGE = OFF_SAV + (TRV ? TT * WAV : WAV * TS);
  static_assert(OFF_SS % 4 == 0 && OFF_SAK % 4 == 0 && OFF_SV % 4 == 0 && OFF_SAV % 4 == 0 && STAGE % 4 == 0,
                "16-byte LDS reads");
  // group LDS (words): qa, qb as prepare_queries leaves them, the fp16 query operands
  // [4][NREP + 1][D] halves (q_hi, q_lo, qb_hi, qb_lo; row NREP is zero, the operand of
  // the columns beyond n_rep), the code-pair table, the sign table,
  // four staging areas, merge scalars
  static constexpr int NPT = (AFF || F16K) ? 0 : 1 << (2 * KB);       // key code pairs
  static constexpr int NVT = (VK == TQ_V_LM_ROT) ? 1 << (2 * VB) : 0;  // value code pairs
  static constexpr int OFF_BQ = (G::OFF_QB + NREP * D + 3) & ~3;
  static constexpr int NRB = NREP + 1;         // query operand rows: the heads, then a zero row
  // query operand rows padded by 4 words: the n_rep rows a 16-byte read spans fall in
  // different LDS banks
  static constexpr int QS = D / 2 + 4;         // words per query operand row
  static constexpr int OFF_PT = OFF_BQ + 4 * NRB * QS;
  // the lo words of a pair table sit PLO words after its hi words: a distance no paired LDS
  // read encodes (> 255 words, not a multiple of 64), so each read lands in its operand register
  static constexpr int plo(int n) { return n == 0 ? 0 : (n > 256 ? n : 256) + 1; }
  static constexpr int PLO = plo(NPT), VLO = plo(NVT);
  static constexpr int al4(int w) { return (w + 3) & ~3; }   // 16-byte alignment of the regions after
  static constexpr int OFF_VT = al4(OFF_PT + (NPT ? PLO + NPT : 0));
  // 3-bit rotated values (ten codes per word): per 16-dimension block and column l16 of it, the
  // word offset of dimension 16 nb + l16 in the transposed staging and its bit, (TS w) | bit << 16
  static constexpr int NVW = (VK == TQ_V_LM_ROT && VB == 3) ? D : 0;
  static constexpr int OFF_VW = al4(OFF_VT + (NVT ? VLO + NVT : 0));
  static constexpr int OFF_SGT = al4(OFF_VW + NVW);
  // 4-bit Lloyd-Max keys from registers with folded query columns: the score operand word is
  // (hi, lo) of ONE code, from a 16-entry table (its reads never collide in the LDS banks, where
  // the 256-entry pair table's did), against a query operand holding every value twice, so one
  // product sums c_hi q + c_lo q over 16 dimensions; rows of the doubled operand are D + 4 words
  static constexpr bool ILV = DIRECT && KB == 4 && 2 * NREP <= 16;
  static constexpr int QSD = D + 4;
  static constexpr int OFF_BQD = al4(OFF_SGT + (QJL ? 2 * 16 : 0));
  static constexpr int OFF_ST = al4(OFF_BQD + (ILV ? 2 * NRB * QSD : 0));
  static_assert(OFF_BQ % 4 == 0 && OFF_SGT % 4 == 0 && OFF_ST % 4 == 0, "16-byte LDS reads of the operand, sign and staging regions");
  // the four staging areas also hold the waves' value sums for the merge
  static constexpr int STAGE_ALL = (4 * STAGE > 4 * NREP * D) ? 4 * STAGE : 4 * NREP * D;
  static constexpr int OFF_MRG = OFF_ST + STAGE_ALL;
  static constexpr int OWN = OFF_MRG + 8 * NREP + 16;
  // the recent-buffer split: the queries (G::OFF_QA) and its scratch right after qa, qb
  static constexpr int OFF_RSCR = G::OFF_TQ;
  static constexpr int RECENT_NEED = OFF_RSCR + G::RECENT_SCRATCH;
  static constexpr int FLOATS = OWN > RECENT_NEED ? OWN : RECENT_NEED;
  static_assert(NREP <= 16, "one 16-column operand holds the heads");
};

// Lloyd-Max keys loaded straight into registers in the order the score product consumes
// them.  Lane (l16, q4) of 16-token block mb holds token 16 mb + l16's dimensions
// q4 D/4 .. q4 D/4 + D/4 - 1 (its code words and QJL sign bits) and that token's aux word
// (n and gamma); the score product's k slots 8 q4 .. 8 q4 + 7 of k-block kb are dimensions
// q4 D/4 + 8 kb .. + 7, and the query operand is read in the same order.  The lane also
// loads the aux words of the four tokens its score accumulators hold (16 mb + 4 q4 + r).
// Raw buffer loads over exactly the tile's rows: words past the tile read as zero.
template <int D, int KB, bool QJL, int TT>
struct DirectKeys {
  static constexpr int MB = TT / 16;
  static constexpr int DPL = D / 4;                         // dimensions per lane
  static constexpr int PER = (KB == 3) ? 10 : 32 / KB;
  static constexpr int WK = (D + PER - 1) / PER;            // code words per row
  static constexpr int WS = QJL ? D / 32 : 0;               // sign words per row
  static constexpr int first_word(int q) { return (DPL * q) / PER; }
  static constexpr int span(int q) { return (DPL * q + DPL - 1) / PER - first_word(q) + 1; }
  static constexpr int max_span() {
    int m = 0;
    for (int q = 0; q < 4; ++q) m = span(q) > m ? span(q) : m;
    return m;
  }
  static constexpr int KWL = (KB == 3) ? max_span() : DPL * KB / 32;   // code words per lane
  static constexpr int SWL = QJL ? (DPL >= 32 ? DPL / 32 : 1) : 1;    // sign words per lane
  static constexpr int SAL = (KB == 3) ? (3 * DPL + 31) / 32 : 1;     // aligned 3-bit stream words
  static_assert(KB == 3 || (DPL * KB) % 32 == 0, "a lane's codes fill whole words");
  uint32_t kc[MB][KWL];
  uint32_t ks[MB][SWL];
  uint32_t ka[MB];

  __device__ __forceinline__ void load(const uint32_t* kc_g, const uint32_t* ks_g, const uint32_t* ka_g, int rows,
                                       int l16, int q4) {
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kc_g), (short)0, 4 * rows * WK, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ka_g), (short)0, 4 * rows, kBufferRsrcWord3);
    const int w0 = (DPL * q4) / PER;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int tok = 16 * mb + l16;
      const int cb = 4 * (tok * WK + w0);
      if constexpr (KB != 3 && KWL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < KWL; i += 4) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, cb + 4 * i, 0, kTileLoadPolicy);
          kc[mb][i] = v[0]; kc[mb][i + 1] = v[1]; kc[mb][i + 2] = v[2]; kc[mb][i + 3] = v[3];
        }
      } else if constexpr (KB != 3 && KWL == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, cb, 0, kTileLoadPolicy);
        kc[mb][0] = v[0]; kc[mb][1] = v[1];
      } else {
#pragma unroll
        for (int i = 0; i < KWL; ++i) kc[mb][i] = __builtin_amdgcn_raw_buffer_load_b32(rc, cb + 4 * i, 0, kTileLoadPolicy);
      }
      ka[mb] = __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * tok, 0, kTileLoadPolicy);
      if constexpr (QJL) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(ks_g), (short)0, 4 * rows * WS, kBufferRsrcWord3);
        const int sw0 = (DPL * q4) / 32;
        if constexpr (SWL == 2) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, 4 * (tok * WS + sw0), 0, kTileLoadPolicy);
          ks[mb][0] = v[0]; ks[mb][1] = v[1];
        } else {
          ks[mb][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (tok * WS + sw0), 0, kTileLoadPolicy);
        }
      }
    }
  }

  // the lane's 8 codes of k-block kb (dimensions q4 D/4 + 8 kb ..) in the low 8 KB bits;
  // for 3-bit codes `al` is the lane's gap-free code stream (align3 below)
  __device__ __forceinline__ uint32_t codes(int mb, int kb, const uint32_t (&al)[SAL]) const {
    if constexpr (KB == 4) {
      return kc[mb][kb];
    } else if constexpr (KB == 2) {
      return kc[mb][kb >> 1] >> (16 * (kb & 1));
    } else {
      const int bit = 24 * kb;
      const uint32_t lo = al[bit >> 5];
      const uint32_t hi = ((bit >> 5) + 1 < SAL) ? al[(bit >> 5) + 1] : 0u;
      return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(bit & 31));
    }
  }

  // 3-bit codes, ten per word: the lane's words joined into one gap-free stream, shifted so
  // that its first dimension sits at bit 0
  __device__ __forceinline__ void align3(int mb, int q4, uint32_t (&al)[SAL]) const {
    if constexpr (KB == 3) {
      constexpr int NG3 = (30 * KWL + 31) / 32;
      uint32_t g[NG3 + 1];
#pragma unroll
      for (int j = 0; j <= NG3; ++j) g[j] = 0u;
#pragma unroll
      for (int i = 0; i < KWL; ++i) {
        const int b = 30 * i;                 // chunk i starts at stream bit 30 i
        g[b >> 5] |= kc[mb][i] << (b & 31);
        if ((b & 31) + 30 > 32) g[(b >> 5) + 1] |= kc[mb][i] >> (32 - (b & 31));
      }
      const uint32_t off = (uint32_t)(3 * (DPL * q4 - 10 * ((DPL * q4) / 10)));
#pragma unroll
      for (int j = 0; j < SAL; ++j) al[j] = __builtin_amdgcn_alignbit(g[j + 1], g[j], off);
    }
  }

  // the 8 QJL sign bits of k-block kb
  __device__ __forceinline__ uint32_t sign_byte(int mb, int kb, int q4) const {
    if constexpr (DPL >= 32) {
      return (ks[mb][kb >> 2] >> (8 * (kb & 3))) & 0xFFu;
    } else {
      return (ks[mb][0] >> (16 * (q4 & 1) + 8 * kb)) & 0xFFu;
    }
  }
};

// NQ > 1: a multi-query group.  The NQ x n_rep rows (query j, head h at row j n_rep + h) take
// the operand columns of the heads, so the score and value products cost the same per tile;
// only the softmax and the output rows grow.  Below, NREP counts rows.
// TT: tokens per wave tile (64; 32 at head_dim 256, where a 64-token tile's staging and
// registers would leave one wave per SIMD).
// Group values (symmetric or min/max, 2 or 4 bits) of a 64-token tile.  Code and scale rows
// arrive through 16-byte raw buffer loads over exactly the tile's rows (words past them read as
// zero) and go to LDS row-major: code rows padded to LSV words, scale rows dense.  The value
// product then reads the codes with the transposing LDS read (ds_read_b64_tr_b4): in each group
// of 16 lanes, lane k points at an 8-byte chunk of one token row and lane n receives nibble n of
// every chunk, i.e. one 4-bit code (or one pair of 2-bit codes) of 16 tokens.
template <int D, int VB, bool ASYMV, int TT>
struct GroupValueTile {
  static constexpr int WV = D * VB / 32;          // code words per token
  static constexpr int LSV = WV + 2;              // LDS row stride: 8-byte reads of 64 rows spread over the banks
  static constexpr int WAV = ASYMV ? D / 32 : D / 64;
  static constexpr int NVL = TT * WV / 256;       // 16-byte code loads per lane
  static constexpr int NS = TT * WAV / 64;        // scale words per lane
  static_assert(WV % 4 == 0 && NVL >= 1 && (NS == 1 || NS == 2 || NS == 4 || NS == 8), "tile geometry");
  uint32_t c[NVL][4];
  uint32_t sc[NS];

  __device__ __forceinline__ void load(const uint32_t* vc_g, const uint32_t* va_g, int rows, int lane) {
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(vc_g), (short)0, 4 * rows * WV, kBufferRsrcWord3);
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * (lane + 64 * u), 0, kTileLoadPolicy);
      c[u][0] = v[0]; c[u][1] = v[1]; c[u][2] = v[2]; c[u][3] = v[3];
    }
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(va_g), (short)0, 4 * rows * WAV, kBufferRsrcWord3);
    if constexpr (NS == 1) {
      sc[0] = __builtin_amdgcn_raw_buffer_load_b32(ra, 4 * lane, 0, kTileLoadPolicy);
    } else if constexpr (NS == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(ra, 8 * lane, 0, kTileLoadPolicy);
      sc[0] = v[0]; sc[1] = v[1];
    } else {
#pragma unroll
      for (int u = 0; u < NS / 4; ++u) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(ra, 4 * NS * lane + 16 * u, 0, kTileLoadPolicy);
        sc[4 * u] = v[0]; sc[4 * u + 1] = v[1]; sc[4 * u + 2] = v[2]; sc[4 * u + 3] = v[3];
      }
    }
  }

  __device__ __forceinline__ void store(uint32_t* __restrict__ codes, uint32_t* __restrict__ scales, int lane) const {
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int q = 4 * (lane + 64 * u);          // first word of the chunk in the tile
      uint32_t* d = codes + (q / WV) * LSV + q % WV;
      *reinterpret_cast<uint2*>(d) = make_uint2(c[u][0], c[u][1]);
      *reinterpret_cast<uint2*>(d + 2) = make_uint2(c[u][2], c[u][3]);
    }
    if constexpr (NS == 1) {
      scales[lane] = sc[0];
    } else if constexpr (NS == 2) {
      *reinterpret_cast<uint2*>(scales + 2 * lane) = make_uint2(sc[0], sc[1]);
    } else {
#pragma unroll
      for (int u = 0; u < NS / 4; ++u)
        *reinterpret_cast<uint4*>(scales + NS * lane + 4 * u) = make_uint4(sc[4 * u], sc[4 * u + 1], sc[4 * u + 2], sc[4 * u + 3]);
    }
  }
};

typedef int mma_i2_t __attribute__((ext_vector_type(2)));

// the 8 QJL sign bits of one k-block as the score operand's four fp16 pairs of +-1: two reads
// of the 16-entry table of 4-bit patterns (entry n: words 2 n, 2 n + 1)
__device__ __forceinline__ mma_u4_t sign_operand(const uint32_t* sgt, uint32_t sb) {
  const uint2 lo = *reinterpret_cast<const uint2*>(sgt + 2 * (sb & 15u));
  const uint2 hi = *reinterpret_cast<const uint2*>(sgt + 2 * ((sb >> 4) & 15u));
  return mma_u4_t{lo.x, lo.y, hi.x, hi.y};
}
// the same from byte offsets into the table: byte k of `ol` (`oh`) is 8 x the low (high) nibble
// of sign byte k, so one byte-select gives each read's address
__device__ __forceinline__ mma_u4_t sign_operand_at(const uint32_t* sgt, uint32_t ol, uint32_t oh, int k) {
  const char* t = reinterpret_cast<const char*>(sgt);
  const uint2 lo = *reinterpret_cast<const uint2*>(t + __builtin_amdgcn_perm(0u, ol, 0x0C0C0C00u | (uint32_t)k));
  const uint2 hi = *reinterpret_cast<const uint2*>(t + __builtin_amdgcn_perm(0u, oh, 0x0C0C0C00u | (uint32_t)k));
  return mma_u4_t{lo.x, lo.y, hi.x, hi.y};
}

// the transposing 8-byte LDS read (ds_read_b64_tr_b4) at word `w` of the LDS
__device__ __forceinline__ uint2 lds_read_tr4(const uint32_t* w) {
  const mma_i2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
      (__attribute__((address_space(3))) mma_i2_t*)((__attribute__((address_space(3))) uint32_t*)w));
  return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}

template <int D, int NREP_KV, int KK, int KB, int VK, int VB, int NQ = 1, int TT = kTile>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((D == 64 && KK != TQ_K_F16) ? 3 : (D == 256 ? 1 : 2))))
decode_mma_kernel(const DecodeArgs A) {
  constexpr int NREP = NQ * NREP_KV;
  using M = MmaGeom<D, NREP, KK, KB, VK, VB, TT>;
  constexpr int MB = TT / 16;                    // 16-token blocks per tile
  static_assert(TT == 64 || TT == 32, "tile of 32 or 64 tokens");
  constexpr bool QJL = M::QJL, AFF = M::AFF, F16K = M::F16K, ROT = VK == TQ_V_LM_ROT, ASYM = VK == TQ_V_GROUP_ASYM;
  constexpr int LK = 1 << KB;
  constexpr int LV = 1 << VB;
  constexpr int NKB = M::NKB, NNB = M::NNB, NG = M::NG;
  static_assert(KK == TQ_K_LM_QJL || KK == TQ_K_LM_MSE || KK == TQ_K_AFFINE8 || KK == TQ_K_F16, "key kind");
  static_assert(ROT ? (VB >= 2 && VB <= 4) : (VB == 2 || VB == 4), "value bits");
  static_assert(VK == TQ_V_GROUP_SYM || VK == TQ_V_GROUP_ASYM || VK == TQ_V_LM_ROT, "value kind");

  __shared__ __attribute__((aligned(16))) float sm[M::FLOATS];
  uint32_t* smw = reinterpret_cast<uint32_t*>(sm);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar tile bases
  const int l16 = lane & 15, q4 = lane >> 4;

  // grid: the compressed splits first, then one recent-buffer group per (batch, kv-head)
  const int n_comp = A.nsplit * A.Hkv * A.batch;
  if ((int)blockIdx.x >= n_comp) {
    const int u = blockIdx.x - n_comp;
    recent_split<D, NREP, KK, KB, VK, VB, NQ, M::OFF_RSCR>(A, u / A.Hkv, u % A.Hkv, sm);
    return;
  }
  const int split = blockIdx.x % A.nsplit;
  const int g = (blockIdx.x / A.nsplit) % A.Hkv;
  const int b = blockIdx.x / (A.nsplit * A.Hkv);
  const size_t slice = (size_t)b * A.Hkv + g;
  const int tb = split * A.chunk;
  const int te = min(A.n_c, tb + A.chunk);
  const int cap = A.cap;

  uint32_t* st = smw + M::OFF_ST + wave * M::STAGE;
  const uint32_t* stk = st + M::OFF_SK;
  const uint32_t* sts = st + M::OFF_SS;
  const uint32_t* stak = st + M::OFF_SAK;
  const uint32_t* stv = st + M::OFF_SV;
  const uint32_t* stav = st + M::OFF_SAV;

  // Branch-free dword loads keep the next tile's loads in flight through the score and PV
  // work (a vector/scalar split per chunk made the compiler wait for every outstanding load
  // at its join); as raw buffer loads they also cost no per-lane address arithmetic, which
  // leaves the affine-key kernels room to hold them without a spill.
  static constexpr bool DWL = true;
  RowLoader<M::WK, M::SK, TT, DWL> ld_k;
  RowLoader<M::WS, M::SS, TT, DWL> ld_s;
  RowLoader<M::WAK, AFF ? M::TS : 1, TT, DWL> ld_ak;
  RowLoader<M::TRV ? 0 : M::WV, M::TS, TT, DWL> ld_v;
  RowLoader<M::TRV ? 0 : M::WAV, M::TS, TT, DWL> ld_av;
  using GV = GroupValueTile<D, (M::TRV ? VB : 4), ASYM, 64>;
  GV gv;
  using DK = DirectKeys<D, (M::DIRECT ? KB : 2), QJL, TT>;
  DK dkn;                                       // the next tile's keys (Lloyd-Max kinds)
  auto issue = [&](int t0) {
    const int nv = min(TT, te - t0);
    const size_t row0 = slice * cap + t0;
    if constexpr (M::DIRECT) {
      dkn.load(A.kc + row0 * M::WK, A.ks + row0 * M::WS, A.ka + row0 * M::WAK, nv, l16, q4);
    } else {
      ld_k.load(A.kc + row0 * M::WK, nv, lane);
      ld_s.load(A.ks + row0 * M::WS, nv, lane);
      ld_ak.load(A.ka + row0 * M::WAK, nv, lane);
    }
    if constexpr (M::TRV) {
      gv.load(A.vc + row0 * M::WV, A.va + row0 * M::WAV, nv, lane);
    } else {
      ld_v.load(A.vc + row0 * M::WV, nv, lane);
      ld_av.load(A.va + row0 * M::WAV, nv, lane);
    }
  };
  if (tb + wave * TT < te) issue(tb + wave * TT);

  // code-pair tables: entry pc = (code a = low bits, code b): the hi pair of 8 c at word pc, the
  // lo pair at word PLO + pc
  if constexpr (M::ILV) {
    // single-code table: word c = (hi, lo) fp16 halves of 8 c[c]
    for (int i = threadIdx.x; i < 16; i += 256) {
      uint32_t hi, lo;
      split_f16x2(A.kcent[i] * kMmaCentScale, A.kcent[i] * kMmaCentScale, hi, lo);
      smw[M::OFF_PT + i] = (hi & 0xFFFFu) | (lo << 16);
    }
  } else {
    for (int i = threadIdx.x; i < M::NPT; i += 256) {
      uint32_t hi, lo;
      split_f16x2(A.kcent[i & (LK - 1)] * kMmaCentScale, A.kcent[i >> KB] * kMmaCentScale, hi, lo);
      smw[M::OFF_PT + i] = hi;
      smw[M::OFF_PT + M::PLO + i] = lo;
    }
  }
  for (int i = threadIdx.x; i < M::NVT; i += 256) {
    uint32_t hi, lo;
    split_f16x2(A.vcent[i & (LV - 1)] * kMmaCentScale, A.vcent[i >> VB] * kMmaCentScale, hi, lo);
    smw[M::OFF_VT + i] = hi;
    smw[M::OFF_VT + M::VLO + i] = lo;
  }
  for (int j = threadIdx.x; j < M::NVW; j += 256) smw[M::OFF_VW + j] = (j / 10) * M::TS | (3 * (j % 10)) << 16;
  // sign table: 4 stored bits (bit 1 <=> sigma = +1) -> 2 fp16 pairs of +-1; sixteen 8-byte
  // entries fill the 32 LDS banks once, so no two lanes' reads of it collide
  if constexpr (QJL) {
    if (threadIdx.x < 32) {
      const int i = threadIdx.x >> 1, k = threadIdx.x & 1;
      smw[M::OFF_SGT + threadIdx.x] = 0x3C003C00u ^ ((((i >> (2 * k)) & 1) ? 0u : 0x8000u) | (((i >> (2 * k + 1)) & 1) ? 0u : 0x80000000u));
    }
  }
  prepare_queries<D, NREP, KK, KB, VK, VB, false, NQ>(A, b, g, sm);
  // 16-bit keys at head_dim 256 come in either storage type: bf16 rows are bf16 matrix-core
  // operands against a three-term bf16 split of the query (hi + mid + lo carries its 24 bits)
  constexpr bool KBF = F16K && D == 256;
  const bool kbf = KBF && A.q_bf16;
  if (kbf) {
    const float* qa = sm + M::G::OFF_QA;
    uint16_t* bq = reinterpret_cast<uint16_t*>(smw + M::OFF_BQ);
    constexpr int RS = M::NRB * 2 * M::QS;
    for (int i = threadIdx.x; i < M::NRB * D; i += 256) {
      const float a = (i < NREP * D) ? qa[i] * kMmaAffQScale : 0.f;
      const uint32_t h = bf16_rne_bits(a);
      const float r = a - __uint_as_float(h << 16);
      const uint32_t m = bf16_rne_bits(r);
      const uint32_t l = bf16_rne_bits(r - __uint_as_float(m << 16));
      const int o = (i / D) * 2 * M::QS + i % D;
      bq[o] = (uint16_t)h;
      bq[RS + o] = (uint16_t)m;
      bq[2 * RS + o] = (uint16_t)l;
    }
  } else {
    // fp16 query operands (hi, lo) from the prepared fp32 queries
    const float* qa = sm + M::G::OFF_QA;
    const float* qb = sm + M::G::OFF_QB;
    _Float16* bq = reinterpret_cast<_Float16*>(smw + M::OFF_BQ);
    constexpr int RS = M::NRB * 2 * M::QS;       // halves per operand region
    constexpr float QA = (AFF || F16K) ? kMmaAffQScale : kMmaQScale / kMmaCentScale;
    for (int i = threadIdx.x; i < M::NRB * D; i += 256) {
      const bool on = i < NREP * D;
      const float a = on ? qa[i] * QA : 0.f;
      const float s = (on && QJL) ? qb[i] * kMmaQScale : 0.f;
      const _Float16 ah = (_Float16)a, sh = (_Float16)s;
      const int o = (i / D) * 2 * M::QS + i % D;
      bq[o] = ah;
      bq[RS + o] = (_Float16)(a - (float)ah);
      bq[2 * RS + o] = sh;
      bq[3 * RS + o] = (_Float16)(s - (float)sh);
      if constexpr (M::ILV) {
        // the same hi / lo halves, each value twice: rows [NRB][QSD] words, hi region then lo
        const uint32_t hb = __builtin_bit_cast(uint16_t, ah), lb = __builtin_bit_cast(uint16_t, (_Float16)(a - (float)ah));
        const int od = (i / D) * M::QSD + i % D;
        smw[M::OFF_BQD + od] = hb | (hb << 16);
        smw[M::OFF_BQD + M::NRB * M::QSD + od] = lb | (lb << 16);
      }
    }
  }
  __syncthreads();

  const uint32_t* bqw = smw + M::OFF_BQ;
  const uint32_t* ptab = smw + M::OFF_PT;
  const uint32_t* sgt = smw + M::OFF_SGT;
  const int hq = (l16 < NREP) ? l16 : NREP;    // operand column (head); the zero row beyond n_rep
  // Lloyd-Max keys with n_rep <= 8: score columns 0..NREP-1 take the hi parts of the heads' query
  // operands and columns NREP..2 NREP-1 their lo parts, folded onto the heads after the products,
  // so every key operand meets both parts of the query in one product
  constexpr bool FOLD = !AFF && !F16K && 2 * NREP <= 16;
  constexpr int RWQ = M::NRB * M::QS;          // words per query operand region
  const uint32_t* bqf = bqw + ((FOLD && l16 >= NREP && l16 < 2 * NREP) ? RWQ + (l16 - NREP) * M::QS : hq * M::QS);
  const uint32_t* vtab = smw + M::OFF_VT;
  // affine keys: per 32-dimension block, the sum of the lane's head's query operand
  float qsum[AFF ? NKB : 1];
  if constexpr (AFF) {
    const float* qb = sm + M::G::OFF_QB;      // prepare_queries: block sums of qa
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qsum[kb] = (l16 < NREP) ? qb[l16 * NKB + kb] * kMmaAffQScale : 0.f;
  }

  // group-value operands: lane l16 takes dimension 16 nb + l16, whose code sits in byte vbyte of
  // each token's word at bit vsh of that byte; perm selector gathering that byte of two tokens
  // into the low bytes of the two halves, mask of the code there, shift to bit MV
  constexpr int MV = (VB == 2) ? 8 : 6;
  const uint32_t vbyte = (VB == 2) ? (uint32_t)(l16 >> 2) : (uint32_t)((l16 & 7) >> 1);
  const uint32_t vsh = (VB == 2) ? (uint32_t)(2 * (l16 & 3)) : (uint32_t)(4 * (l16 & 1));
  const uint32_t vsel = vbyte | 0x0C00u | ((4u + vbyte) << 16) | 0x0C000000u;
  const uint32_t vmask = (((1u << VB) - 1u) * 0x00010001u) << vsh;
  const uint32_t vls = (uint32_t)MV - vsh;

  // scale of the score products to the log2 domain: affine and 16-bit keys carry the query
  // operands' 16, Lloyd-Max keys the 2^8 of the centroid and query operand scales
  constexpr float PS = (AFF || F16K) ? 1.f / kMmaAffQScale : kMmaUnscale;
  // zero kept opaque so that n (fp16) times the score stays one mixed-precision multiply-add
  float zero_v = 0.f;
  asm volatile("" : "+v"(zero_v));
  float m_run = -INFINITY, l_part = 0.f;        // head l16 (per lane: its tokens; product scale)
  float off[NG];                                // sum of P' per group, head l16
  float moff[ASYM ? NG : 1];                    // min/max values: sum of p m per group, head l16
  mma_f4_t acc[NNB];                            // head 4 q4 + r, dimension 16 nb + l16
#pragma unroll
  for (int k = 0; k < NG; ++k) off[k] = 0.f;
#pragma unroll
  for (int k = 0; k < (ASYM ? NG : 1); ++k) moff[k] = 0.f;
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) acc[nb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = tb + wave * TT; t0 < te; t0 += 4 * TT) {
    const int nv = min(TT, te - t0);
    const DK dk = dkn;
    if constexpr (!M::DIRECT) {
      ld_k.store(st + M::OFF_SK, lane);
      ld_s.store(st + M::OFF_SS, lane);
      if constexpr (AFF) ld_ak.store_transposed(st + M::OFF_SAK, lane);
      else ld_ak.store(st + M::OFF_SAK, lane);
    }
    if constexpr (M::TRV) {
      gv.store(st + M::OFF_SV, st + M::OFF_SAV, lane);
    } else {
      ld_v.store_transposed(st + M::OFF_SV, lane);
      ld_av.store_transposed(st + M::OFF_SAV, lane);
    }
    if (t0 + 4 * TT < te) issue(t0 + 4 * TT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- scores: four 16-token blocks ------------------------------------------------------
    // p[mb][r]: head l16, token 16 mb + 4 q4 + r (log2-domain score, then its weight)
    float p[MB][4];
    if constexpr (F16K) {
      // 16-bit keys: the stored rows are the A operand as they are, against the hi/lo (fp16
      // storage) or hi/mid/lo (bf16 storage) query operands (x16); every product exact
      mma_f4_t sacc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sacc[mb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int kw = 16 * kb + 4 * q4;
        constexpr int RW = M::NRB * M::QS;
        const uint32_t* src = bqw + hq * M::QS + kw;
        const uint4 r0 = *reinterpret_cast<const uint4*>(src);
        const uint4 r1 = *reinterpret_cast<const uint4*>(src + RW);
        const mma_u4_t bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
        const mma_u4_t bq1 = mma_u4_t{r1.x, r1.y, r1.z, r1.w};
        if (KBF && kbf) {
          const uint4 r2 = *reinterpret_cast<const uint4*>(src + 2 * RW);
          const mma_u4_t bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const uint4 w = *reinterpret_cast<const uint4*>(stk + (16 * mb + l16) * M::SK + kw);
            const mma_u4_t ak = mma_u4_t{w.x, w.y, w.z, w.w};
            sacc[mb] = mma16_bf(ak, bq0, sacc[mb]);
            sacc[mb] = mma16_bf(ak, bq1, sacc[mb]);
            sacc[mb] = mma16_bf(ak, bq2, sacc[mb]);
          }
          continue;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint4 w = *reinterpret_cast<const uint4*>(stk + (16 * mb + l16) * M::SK + kw);
          const mma_u4_t ak = mma_u4_t{w.x, w.y, w.z, w.w};
          sacc[mb] = mma16(ak, bq0, sacc[mb]);
          sacc[mb] = mma16(ak, bq1, sacc[mb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[mb][r] = sacc[mb][r];
    } else if constexpr (!AFF && !M::DIRECT) {
      mma_f4_t sacc[MB], sqj[QJL ? MB : 1];      // codebook term; QJL sign term (before gamma)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sacc[mb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < (QJL ? MB : 1); ++mb) sqj[mb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int kw = 16 * kb + 4 * q4;           // word offset of this lane's 8 dimensions
        mma_u4_t bq0, bq1, bq2, bq3;
        if constexpr (FOLD) {
          // folded columns: hi or lo part by lane (region 0 / 1; the projected query in 2 / 3)
          const uint32_t* src = bqf + kw;
          const uint4 r0 = *reinterpret_cast<const uint4*>(src);
          bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
          if constexpr (QJL) {
            const uint4 r2 = *reinterpret_cast<const uint4*>(src + 2 * RWQ);
            bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
          }
        } else {
          const uint32_t* src = bqw + hq * M::QS + kw;
          const uint4 r0 = *reinterpret_cast<const uint4*>(src);
          const uint4 r1 = *reinterpret_cast<const uint4*>(src + RWQ);
          bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
          bq1 = mma_u4_t{r1.x, r1.y, r1.z, r1.w};
          if constexpr (QJL) {
            const uint4 r2 = *reinterpret_cast<const uint4*>(src + 2 * RWQ);
            const uint4 r3 = *reinterpret_cast<const uint4*>(src + 3 * RWQ);
            bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
            bq3 = mma_u4_t{r3.x, r3.y, r3.z, r3.w};
          }
        }
        // one 16-token block at a time: its operands, then its products (the accumulator
        // chains through the matrix unit; few registers stay live)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int tok = 16 * mb + l16;
          const uint32_t* row = stk + tok * M::SK;
          // the lane's 8 codes (dimensions 32 kb + 8 q4 ..) as the low 8 KB bits of y
          uint32_t y;
          if constexpr (KB == 3) {
            const int a0 = 32 * kb + 8 * q4;
            const int w0 = a0 / 10, b0 = 3 * (a0 - 10 * w0);
            const uint32_t x0 = row[w0], x1 = row[w0 + 1];
            y = __builtin_amdgcn_alignbit(x1 >> 2, x0 | (x1 << 30), (uint32_t)b0);
          } else if constexpr (KB == 4) {
            y = row[4 * kb + q4];
          } else {
            y = row[2 * kb + (q4 >> 1)] >> (16 * (q4 & 1));
          }
          mma_u4_t ahi, alo;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const uint32_t pc = (y >> (2 * KB * pp)) & (M::NPT - 1);
            ahi[pp] = ptab[pc];
            alo[pp] = ptab[M::PLO + pc];
          }
          sacc[mb] = mma16(ahi, bq0, sacc[mb]);
          sacc[mb] = mma16(alo, bq0, sacc[mb]);
          if constexpr (!FOLD) sacc[mb] = mma16(ahi, bq1, sacc[mb]);
          if constexpr (QJL) {
            // the sign bits as +-1 operands; gamma scales the token's sum afterwards
            const mma_u4_t asg = sign_operand(sgt, (sts[tok * M::SS + kb] >> (8 * q4)) & 0xFFu);
            sqj[mb] = mma16(asg, bq2, sqj[mb]);
            if constexpr (!FOLD) sqj[mb] = mma16(asg, bq3, sqj[mb]);
          }
        }
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sacc[mb][r] += row_shl<FOLD ? NREP : 1>(sacc[mb][r]);
            if constexpr (QJL) sqj[mb][r] += row_shl<FOLD ? NREP : 1>(sqj[mb][r]);
          }
      }
      // times n (fp16 with gamma for LM + QJL keys, fp32 for MSE-only keys; the unscale PS is
      // applied in the softmax)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 nw = *reinterpret_cast<const uint4*>(stak + 16 * mb + 4 * q4);
        const uint32_t nn[4] = {nw.x, nw.y, nw.z, nw.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = QJL ? fmaf(f16_to_f32(nn[r] >> 16), sqj[QJL ? mb : 0][r], sacc[mb][r]) : sacc[mb][r];
          p[mb][r] = QJL ? fmaf(f16_to_f32(nn[r] & 0xFFFFu), sc, zero_v) : sc * __uint_as_float(nn[r]);
        }
      }
    } else if constexpr (!AFF) {
      mma_f4_t sacc[MB], sqj[QJL ? MB : 1];      // codebook term; QJL sign term (before gamma)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) sacc[mb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < (QJL ? MB : 1); ++mb) sqj[mb] = mma_f4_t{0.f, 0.f, 0.f, 0.f};
      uint32_t al[MB][DK::SAL];                  // 3-bit codes: each block's aligned stream
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) dk.align3(mb, q4, al[mb]);
      // QJL sign words as sign-table byte offsets: byte k of sol (soh) = 8 x nibble 0 (1) of byte k
      uint32_t sol[QJL ? MB : 1][DK::SWL], soh[QJL ? MB : 1][DK::SWL];
      if constexpr (QJL) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int w = 0; w < DK::SWL; ++w) {
            sol[mb][w] = (dk.ks[mb][w] << 3) & 0x78787878u;
            soh[mb][w] = (dk.ks[mb][w] >> 1) & 0x78787878u;
          }
      }
      if constexpr (M::ILV) {
        // 4-bit codes, single-code operands: per step (one k-block of one 16-token block) two
        // products of 16 dimensions; lane q4 takes dimensions q4 D/4 + 8 kb + 4 m .. + 3 (m = 0,
        // 1), k slots 2 i, 2 i + 1 = (hi, lo) of one code against that dimension's query value
        // twice (bqd0 / bqd1, read once per k-block).  The table reads of step s + 1 are issued
        // before the products of step s wait for theirs, so the LDS latency of each step hides
        // behind the previous step's products
        constexpr int NSTEP = NKB * MB;
        const char* tb = reinterpret_cast<const char*>(ptab);
        const uint32_t* bqd_row = smw + M::OFF_BQD +
            ((l16 >= NREP && l16 < 2 * NREP) ? M::NRB * M::QSD + (l16 - NREP) * M::QSD : hq * M::QSD) + 2 * q4 * (D / 8);
        struct Step { mma_u4_t a0, a1, sg; };
        auto operands = [&](int st) {
          const int kb = st / MB, mb = st % MB;
          const uint32_t y = dk.codes(mb, kb, al[mb]);
          // byte k of y << 2 (y >> 2), masked to 0x3C: 4 x code 2k (2k + 1), the entry's offset
          const uint32_t yy = (y << 2) & 0x3C3C3C3Cu, yo = (y >> 2) & 0x3C3C3C3Cu;
          auto T = [&](uint32_t w, int k) {
            return *reinterpret_cast<const uint32_t*>(tb + __builtin_amdgcn_perm(0u, w, 0x0C0C0C00u | (uint32_t)k));
          };
          Step o;
          o.a0 = mma_u4_t{T(yy, 0), T(yo, 0), T(yy, 1), T(yo, 1)};
          o.a1 = mma_u4_t{T(yy, 2), T(yo, 2), T(yy, 3), T(yo, 3)};
          if constexpr (QJL) o.sg = sign_operand_at(sgt, sol[mb][kb >> 2], soh[mb][kb >> 2], kb & 3);
          else o.sg = mma_u4_t{0u, 0u, 0u, 0u};
          return o;
        };
        Step cur = operands(0);
        mma_u4_t bqd0, bqd1, bq2;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
          const int kb = st / MB, mb = st % MB;
          if (mb == 0) {
            const uint4 d0 = *reinterpret_cast<const uint4*>(bqd_row + 8 * kb);
            const uint4 d1 = *reinterpret_cast<const uint4*>(bqd_row + 8 * kb + 4);
            bqd0 = mma_u4_t{d0.x, d0.y, d0.z, d0.w};
            bqd1 = mma_u4_t{d1.x, d1.y, d1.z, d1.w};
            if constexpr (QJL) {
              const uint4 r2 = *reinterpret_cast<const uint4*>(bqf + q4 * (D / 8) + 4 * kb + 2 * RWQ);
              bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
            }
          }
          Step nxt = cur;
          if (st + 1 < NSTEP) nxt = operands(st + 1);
          // the products of step st from here on (a volatile statement keeps the reads above it)
          asm volatile("" : "+v"(cur.a0), "+v"(cur.a1));
          if constexpr (QJL) asm volatile("" : "+v"(cur.sg));
          sacc[mb] = mma16(cur.a0, bqd0, sacc[mb]);
          sacc[mb] = mma16(cur.a1, bqd1, sacc[mb]);
          if constexpr (QJL) sqj[mb] = mma16(cur.sg, bq2, sqj[mb]);
          cur = nxt;
        }
      } else
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // 2/3-bit codes (and 4-bit codes with n_rep > 8): code-pair operands
        const int kw = q4 * (D / 8) + 4 * kb;     // word offset of this lane's 8 query dimensions
        mma_u4_t bq0, bq1, bq2, bq3;
        if constexpr (FOLD) {
          // folded columns: hi or lo part by lane (region 0 / 1; the projected query in 2 / 3)
          const uint32_t* src = bqf + kw;
          const uint4 r0 = *reinterpret_cast<const uint4*>(src);
          bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
          if constexpr (QJL) {
            const uint4 r2 = *reinterpret_cast<const uint4*>(src + 2 * RWQ);
            bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
          }
        } else {
          const uint32_t* src = bqw + hq * M::QS + kw;
          const uint4 r0 = *reinterpret_cast<const uint4*>(src);
          const uint4 r1 = *reinterpret_cast<const uint4*>(src + RWQ);
          bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
          bq1 = mma_u4_t{r1.x, r1.y, r1.z, r1.w};
          if constexpr (QJL) {
            const uint4 r2 = *reinterpret_cast<const uint4*>(src + 2 * RWQ);
            const uint4 r3 = *reinterpret_cast<const uint4*>(src + 3 * RWQ);
            bq2 = mma_u4_t{r2.x, r2.y, r2.z, r2.w};
            bq3 = mma_u4_t{r3.x, r3.y, r3.z, r3.w};
          }
        }
        // one 16-token block at a time: its operands, then its products (the accumulator
        // chains through the matrix unit; few registers stay live)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint32_t y = dk.codes(mb, kb, al[mb]);   // the lane's 8 codes, KB bits each
          mma_u4_t ahi, alo;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const uint32_t pc = (y >> (2 * KB * pp)) & (M::NPT - 1);
            ahi[pp] = ptab[pc];
            alo[pp] = ptab[M::PLO + pc];
          }
          sacc[mb] = mma16(ahi, bq0, sacc[mb]);
          sacc[mb] = mma16(alo, bq0, sacc[mb]);
          if constexpr (!FOLD) sacc[mb] = mma16(ahi, bq1, sacc[mb]);
          if constexpr (QJL) {
            // the sign bits as +-1 operands; gamma scales the token's sum afterwards
            static_assert(DK::DPL >= 32, "a lane's sign bits of a k-block are one byte of its words");
            const mma_u4_t asg = sign_operand_at(sgt, sol[mb][kb >> 2], soh[mb][kb >> 2], kb & 3);
            sqj[mb] = mma16(asg, bq2, sqj[mb]);
            if constexpr (!FOLD) sqj[mb] = mma16(asg, bq3, sqj[mb]);
          }
        }
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sacc[mb][r] += row_shl<FOLD ? NREP : 1>(sacc[mb][r]);
            if constexpr (QJL) sqj[mb][r] += row_shl<FOLD ? NREP : 1>(sqj[mb][r]);
          }
      }
      // times n (fp16 with gamma for LM + QJL keys, fp32 for MSE-only keys; the unscale PS is
      // applied in the softmax); accumulator row r of this lane is token 16 mb + 4 q4 + r, whose
      // aux word lane 4 q4 + r holds
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t nn = (uint32_t)__shfl((int)dk.ka[mb], 4 * q4 + r);
          const float sc = QJL ? fmaf(f16_to_f32(nn >> 16), sqj[QJL ? mb : 0][r], sacc[mb][r]) : sacc[mb][r];
          p[mb][r] = QJL ? fmaf(f16_to_f32(nn & 0xFFFFu), sc, zero_v) : sc * __uint_as_float(nn);
        }
      }
    } else {
      // affine keys: per 32-dimension block, sum_j (c_j - o) q_j on the matrix cores (o = 2^(KB-1),
      // the codes' centre), then a times it plus (m + o a) times the block's query sum
      constexpr float kAffOff = (float)(1 << (KB - 1));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[mb][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int kw = 16 * kb + 4 * q4;
        constexpr int RW = M::NRB * M::QS;
        const uint32_t* src = bqw + hq * M::QS + kw;
        const uint4 r0 = *reinterpret_cast<const uint4*>(src);
        const uint4 r1 = *reinterpret_cast<const uint4*>(src + RW);
        const mma_u4_t bq0 = mma_u4_t{r0.x, r0.y, r0.z, r0.w};
        const mma_u4_t bq1 = mma_u4_t{r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint32_t* krow = stk + (16 * mb + l16) * M::SK;
          mma_u4_t ac;
          if constexpr (KB == 8) {
            const uint32_t w0 = krow[8 * kb + 2 * q4], w1 = krow[8 * kb + 2 * q4 + 1];
            // bytes c -> fp16 1024 + c (0x64 over the byte) -> c - 128, exact
            const f16x2_t off = {(_Float16)-1152.f, (_Float16)-1152.f};
            ac[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) + off);
            ac[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) + off);
            ac[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) + off);
            ac[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) + off);
          } else {
            // 5/4/2-bit codes c of dimensions 32 kb + 8 q4 .. + 7 -> fp16 1024 + c -> c - 2^(KB-1), exact
            constexpr float kOff = 1024.f + (float)(1 << (KB - 1));
            const f16x2_t off = {(_Float16)-kOff, (_Float16)-kOff};
            uint32_t c8[8];
            if constexpr (KB == 2) {
              const uint32_t w = krow[2 * kb + (q4 >> 1)] >> (16 * (q4 & 1));
#pragma unroll
              for (int i = 0; i < 8; ++i) c8[i] = (w >> (2 * i)) & 3u;
            } else {
              const uint32_t w = krow[4 * kb + q4];        // eight low nibbles
#pragma unroll
              for (int i = 0; i < 8; ++i) c8[i] = (w >> (4 * i)) & 15u;
              if constexpr (KB == 5) {
                const uint32_t hb = krow[D / 8 + kb] >> (8 * q4);   // their fifth bits
#pragma unroll
                for (int i = 0; i < 8; ++i) c8[i] |= ((hb >> i) & 1u) << 4;
              }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
              ac[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (0x6400u | c8[2 * k]) | ((0x6400u | c8[2 * k + 1]) << 16)) + off);
          }
          mma_f4_t t = mma16(ac, bq0, mma_f4_t{0.f, 0.f, 0.f, 0.f});
          t = mma16(ac, bq1, t);
          const uint4 aw = *reinterpret_cast<const uint4*>(stak + kb * M::TS + 16 * mb + 4 * q4);
          const uint32_t am[4] = {aw.x, aw.y, aw.z, aw.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = f16_to_f32(am[r] & 0xFFFFu), m = f16_to_f32(am[r] >> 16);
            p[mb][r] = fmaf(a, t[r], fmaf(fmaf(kAffOff, a, m), qsum[kb], p[mb][r]));
          }
        }
      }
    }
    if (__builtin_amdgcn_readfirstlane(nv) < TT) {      // the last tile of a split: tokens past its end score -inf
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * mb + 4 * q4 + r >= nv) p[mb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, p[mb][r]);
    // ---- online softmax (log2 domain): head l16 spans lanes l16 + 16 q ------------------
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m_run, mx);
    // scores and the running maximum are held in the products' scale: the log2-domain value is
    // PS times them (a power of two, so exp2(PS p - PS mn) is exactly exp2 of the unscaled
    // difference).  v_exp_f32 directly: arguments are <= 0, results in [0, 1] (a result below
    // 2^-126 is flushed to zero, far below the fp32 sums it joins)
    const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m_run - mn) * PS);
    const float nms = -mn * PS;
    float ps = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mb][r] = __builtin_amdgcn_exp2f(fmaf(p[mb][r], PS, nms));
        ps += p[mb][r];
      }
    }
    l_part = fmaf(l_part, alpha, ps);
    m_run = mn;
    // (no branch around the rescale: a join inside the tile loop makes the compiler wait for
    // the next tile's loads there)
    {
#pragma unroll
      for (int k = 0; k < NG; ++k) off[k] *= alpha;
      if constexpr (ASYM) {
#pragma unroll
        for (int k = 0; k < NG; ++k) moff[k] *= alpha;
      }
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * q4 + r);
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] *= al[r];
    }

    // ---- weighted values: two 32-token blocks ------------------------------------------
    if constexpr (M::TRV) {
      // group values from the row-major tile.  Product j (tokens of blocks mb = 2j, 2j + 1): in
      // lane group q4, k-slots (2m, 2m + 1) are tokens 32 j + 4 q4 + m and 32 j + 16 + 4 q4 + m,
      // the two tokens of the lane's score rows p[2j][m], p[2j + 1][m].  The transposing read
      // gives lane (n, q4) nibble n of token tau(q4, k) = 16 (k >> 2) + 4 q4 + (k & 3) in its
      // nibble k: k = m and m + 4 of the low word for j = 0, of the high word for j = 1.
      constexpr uint32_t kOne = 0x3C003C00u;       // fp16 pair (1, 1)
      constexpr int MV = (VB == 2) ? 8 : 6;        // code c -> fp16 1 + c / 2^(10 - MV)
      constexpr int WAVv = M::WAV;
      const uint32_t* vrow = stv + (16 * (l16 >> 2) + 4 * q4 + (l16 & 3)) * M::LSV;   // token tau(q4, l16)
      // the constants in registers (one mask and the pair (1, 1)) turn mask-and-or into one instruction
      uint32_t vone = kOne, vmask4 = 0x000F000Fu << MV, vmask2 = 0x00030003u << MV;
      asm volatile("" : "+v"(vone), "+s"(vmask4), "+s"(vmask2));
#pragma unroll
      for (int j = 0; j < TT / 32; ++j) {
        // scale words of the lane's 8 tokens: rows 32 j + 4 q4 + m (blocks 2j) and + 16 (2j + 1)
        uint32_t sw[2][4 * WAVv];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t* src = stav + (32 * j + 16 * h2 + 4 * q4) * WAVv;
#pragma unroll
          for (int u = 0; u < WAVv; ++u) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * u);
            sw[h2][4 * u] = v.x; sw[h2][4 * u + 1] = v.y; sw[h2][4 * u + 2] = v.z; sw[h2][4 * u + 3] = v.w;
          }
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          // P' = fp16(p Delta) (or fp16(p a) for min/max groups) of the lane's 8 tokens
          const int w = ASYM ? gi : gi / 2, hf = ASYM ? 0 : gi % 2;
          mma_u4_t apv;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            apv[m] = mul_f32_f16_pair(p[2 * j][m], sw[0][m * WAVv + w], p[2 * j + 1][m], sw[1][m * WAVv + w], hf);
            off[gi] = dot2_f16(apv[m], kOne, off[gi]);
          }
          if constexpr (ASYM) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              moff[gi] = fmaf(p[2 * j][m], f16_to_f32(sw[0][m * WAVv + w] >> 16), moff[gi]);
              moff[gi] = fmaf(p[2 * j + 1][m], f16_to_f32(sw[1][m * WAVv + w] >> 16), moff[gi]);
            }
          }
          if constexpr (VB == 4) {
            // the group's two 16-dimension blocks: lane n takes dimension 16 nb + n
#pragma unroll
            for (int nb = 2 * gi; nb < 2 * gi + 2; ++nb) {
              const uint2 t = lds_read_tr4(vrow + 2 * nb);
              const uint32_t x = j ? t.y : t.x;
              mma_u4_t bv;
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                const uint32_t sh = (m < 2) ? (x << (MV - 4 * m)) : (x >> (4 * m - MV));
                bv[m] = (sh & vmask4) | vone;
              }
              acc[nb] = mma16(apv, bv, acc[nb]);
            }
          } else {
            // 2-bit codes: one read covers the group's 32 dimensions, lane n the pair 2n, 2n + 1
            // (block 2 gi: dimension 32 gi + 2 n, block 2 gi + 1: 32 gi + 2 n + 1)
            const uint2 t = lds_read_tr4(vrow + 2 * gi);
            const uint32_t x = j ? t.y : t.x;
            mma_u4_t be, bo;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const uint32_t xe = (4 * m <= MV) ? (x << (MV - 4 * m)) : (x >> (4 * m - MV));
              const uint32_t xo = (4 * m + 2 <= MV) ? (x << (MV - 4 * m - 2)) : (x >> (4 * m + 2 - MV));
              be[m] = (xe & vmask2) | vone;
              bo[m] = (xo & vmask2) | vone;
            }
            acc[2 * gi] = mma16(apv, be, acc[2 * gi]);
            acc[2 * gi + 1] = mma16(apv, bo, acc[2 * gi + 1]);
          }
        }
      }
    } else if constexpr (!ROT) {
      // group values: P' = fp16(p Delta) against the exact fp16 1 + c/2^m; min/max values
      // also sum p m per group in fp32 (their offset term)
      constexpr uint32_t kOne = 0x3C003C00u;       // fp16 pair (1, 1)
#pragma unroll
      for (int kb2 = 0; kb2 < TT / 32; ++kb2) {
        // k slot i of this lane: token 32 kb2 + 4 q4 + i (i < 4), 32 kb2 + 16 + 4 q4 + i - 4
        const int tk = 32 * kb2 + 4 * q4;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          // the group's scale (two fp16 per word for symmetric groups; one (a, m) word per
          // group for min/max values) for the lane's 8 tokens
          const int w = ASYM ? gi : gi / 2, hf = ASYM ? 0 : gi % 2;
          const uint4 d0 = *reinterpret_cast<const uint4*>(stav + w * M::TS + tk);
          const uint4 d1 = *reinterpret_cast<const uint4*>(stav + w * M::TS + tk + 16);
          const uint32_t dw[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          mma_u4_t apv;
          {
            // P' = fp16(p Delta) in one mixed-precision product per token
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int i0 = 2 * k, i1 = 2 * k + 1;
              apv[k] = mul_f32_f16_pair(p[2 * kb2 + (i0 >> 2)][i0 & 3], dw[i0], p[2 * kb2 + (i1 >> 2)][i1 & 3], dw[i1],
                                        hf);
              off[gi] = dot2_f16(apv[k], kOne, off[gi]);
            }
            if constexpr (ASYM) {
#pragma unroll
              for (int i = 0; i < 8; ++i) moff[gi] = fmaf(p[2 * kb2 + (i >> 2)][i & 3], f16_to_f32(dw[i] >> 16), moff[gi]);
            }
          }
          // the group's two 16-dimension blocks
#pragma unroll
          for (int nb = 2 * gi; nb < 2 * gi + 2; ++nb) {
            uint32_t x[8];
            {
              const uint32_t* src = (VB == 2) ? stv + nb * M::TS + tk : stv + (2 * nb + (l16 >> 3)) * M::TS + tk;
              const uint4 x0 = *reinterpret_cast<const uint4*>(src);
              const uint4 x1 = *reinterpret_cast<const uint4*>(src + 16);
              x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w; x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            }
            // code c -> fp16 1 + c / 2^MV (the code dropped into the mantissa under 1.0's
            // exponent): the byte holding dimension 16 nb + l16 of both tokens of a k-slot pair
            // gathered into the two halves, the code masked in place and shifted up to bit MV
            mma_u4_t bv;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              bv[k] = ((__builtin_amdgcn_perm(x[2 * k + 1], x[2 * k], vsel) & vmask) << vls) | kOne;
            acc[nb] = mma16(apv, bv, acc[nb]);
          }
        }
      }
    } else {
      // rotated Lloyd-Max values: P'' = p n (hi/lo) against 8 c (hi/lo) per 16 dimensions
#pragma unroll
      for (int kb2 = 0; kb2 < TT / 32; ++kb2) {
        const int tk = 32 * kb2 + 4 * q4;            // k slots as for the group values
        mma_u4_t aph, apl;
        {
          const uint4 n0 = *reinterpret_cast<const uint4*>(stav + tk);
          const uint4 n1 = *reinterpret_cast<const uint4*>(stav + tk + 16);
          const uint32_t nw[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
          float wt[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) wt[i] = p[2 * kb2 + (i >> 2)][i & 3] * __uint_as_float(nw[i]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t hi, lo;
            split_f16x2(wt[2 * k], wt[2 * k + 1], hi, lo);
            aph[k] = hi;
            apl[k] = lo;
          }
        }
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) {
          // dimension 16 nb + l16: its code in word j / VPER of each of the lane's 8 tokens
          constexpr int VPER = M::G::VPER;
          const int j = 16 * nb + l16;
          int wo, bit;
          if constexpr (VB == 3) {
            // read per block (LDS) rather than kept live across the tile loop for every block
            const uint32_t e = smw[M::OFF_VW + j];
            wo = (int)(e & 0xFFFFu);
            bit = (int)(e >> 16);
          } else {
            wo = (j / VPER) * M::TS;
            bit = VB * (j % VPER);
          }
          const uint32_t* src = stv + wo + tk;
          const uint4 x0 = *reinterpret_cast<const uint4*>(src);
          const uint4 x1 = *reinterpret_cast<const uint4*>(src + 16);
          const uint32_t x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          mma_u4_t bvh, bvl;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t c0 = __builtin_amdgcn_ubfe(x[2 * k], (uint32_t)bit, VB);
            const uint32_t c1 = __builtin_amdgcn_ubfe(x[2 * k + 1], (uint32_t)bit, VB);
            const uint32_t vc = c0 | (c1 << VB);
            bvh[k] = vtab[vc];
            bvl[k] = vtab[M::VLO + vc];
          }
          acc[nb] = mma16(aph, bvh, acc[nb]);
          acc[nb] = mma16(apl, bvh, acc[nb]);
          acc[nb] = mma16(aph, bvl, acc[nb]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- wave totals -------------------------------------------------------------------------
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    off[k] += __shfl_xor(off[k], 16);
    off[k] += __shfl_xor(off[k], 32);
  }
  if constexpr (ASYM) {
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      moff[k] += __shfl_xor(moff[k], 16);
      moff[k] += __shfl_xor(moff[k], 32);
    }
  }
  // group values: acc = sum P' (1 + c / F), off = sum P'  ->  sum P' (c - (L-1)/2) = F acc - (F + (L-1)/2) off;
  // rotated values: acc = sum P'' 8 c  ->  acc / 8 (still in the rotated domain)
  constexpr float F = ROT ? 1.f / kMmaCentScale : ((VB == 2) ? 4.f : 16.f);
  // min/max values: sum p (m + a c) = F acc - F off + sum p m
  constexpr float FO = ROT ? 0.f : (ASYM ? F : F + 0.5f * (float)(LV - 1));
  __syncthreads();   // every wave is done with its staging area
  float(*s_mrg_acc)[NREP * D] = reinterpret_cast<float(*)[NREP * D]>(smw + M::OFF_ST);
  float* s_mrg_m = sm + M::OFF_MRG;            // [4][NREP]
  float* s_mrg_l = s_mrg_m + 4 * NREP;         // [4][NREP]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * q4 + r;
    float o[NG], mo[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      o[k] = __shfl(off[k], h);
      mo[k] = ASYM ? __shfl(moff[k], h) : 0.f;
    }
    if (h < NREP) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        // 2-bit group values from the transposing reads: block nb holds dimensions 32 (nb/2) + 2 l16 + nb%2
        const int dim = (M::TRV && VB == 2) ? 32 * (nb >> 1) + 2 * l16 + (nb & 1) : 16 * nb + l16;
        s_mrg_acc[wave][h * D + dim] = ROT ? F * acc[nb][r] : fmaf(F, acc[nb][r], fmaf(-FO, o[nb / 2], mo[nb / 2]));
      }
    }
  }
  if (lane < NREP) {
    s_mrg_m[wave * NREP + lane] = m_run * PS;   // log2 domain
    s_mrg_l[wave * NREP + lane] = l_part;
  }
  __syncthreads();

  // ---- merge the four waves, write one partial per head ----------------------------------
  for (int i = threadIdx.x; i < NREP * D; i += blockDim.x) {
    const int h = i / D, j = i % D;
    float mxw = s_mrg_m[h];
#pragma unroll
    for (int w = 1; w < 4; ++w) mxw = fmaxf(mxw, s_mrg_m[w * NREP + h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_mrg_m[w * NREP + h];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - mxw);
      a = fmaf(s_mrg_acc[w][h * D + j], sc, a);
      l = fmaf(s_mrg_l[w * NREP + h], sc, l);
    }
    float* dst = partial_ptr<D>(A, b * NQ + h / NREP_KV, g * NREP_KV + h % NREP_KV, split);
    dst[4 + j] = a;
    if (j == 0) {
      dst[0] = mxw;
      dst[1] = l;
    }
  }
}

template <int D, int NREP, int KK, int KB, int VK, int VB, int NQ, int TT = kTile>
hipError_t mma_launch(dim3 grid, hipStream_t st, const DecodeArgs& A) {
  hipLaunchKernelGGL((decode_mma_kernel<D, NREP, KK, KB, VK, VB, NQ, TT>), grid, dim3(256), 0, st, A);
  return hipGetLastError();
}

template <int D, int NREP, int KK, int KB, int VK, int VB, int NQ, int TT = kTile>
int mma_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, decode_mma_kernel<D, NREP, KK, KB, VK, VB, NQ, TT>, 256, 0) !=
            hipSuccess ||
        b <= 0)
      b = 1;
    return b;
  }();
  return n;
}

// n_rep query heads per kv-head, NQ queries per step; LM + QJL keys with group values
template <int D, int NREP, int KB, int VB, int NQ = 1>
constexpr MainKernel mma_kernel() {
  return MainKernel{&mma_launch<D, NREP, TQ_K_LM_QJL, KB, TQ_V_GROUP_SYM, VB, NQ>,
                    &mma_blocks_per_cu<D, NREP, TQ_K_LM_QJL, KB, TQ_V_GROUP_SYM, VB, NQ>};
}

// any compiled key / value kind, TT tokens per wave tile
template <int D, int NREP, int KK, int KB, int VK, int VB, int TT = kTile>
constexpr MainKernel mma_kernel_kv() {
  return MainKernel{&mma_launch<D, NREP, KK, KB, VK, VB, 1, TT>, &mma_blocks_per_cu<D, NREP, KK, KB, VK, VB, 1, TT>};
}

}  // namespace tq

/*
 * tq.h -- C ABI of libtq: TurboQuant KV-cache encode and single-query decode
 * attention computed directly on the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (cited by title and section):
 *   [vllm-metal guide]   "vllm-metal TurboQuant" (wmrh.cn): quantisation principle
 *                        table, compression-ratio table, support limits (head_dim
 *                        64/128/256/512; unsupported models fail at start-up).
 *   [vLLM guide]         "TurboQuant vLLM integration" (kwkr.cn): section 2, the
 *                        five-step pipeline (rotation, Lloyd-Max, QJL residual signs,
 *                        group-32 values, bit packing); section 5, the exact
 *                        128-token recent buffer.
 *   [MLX page]           "TurboQuant-MLX" (pomoai.com): core technique (WHT, 8
 *                        centroids, ten 3-bit codes per uint32) and GPU kernel
 *                        optimisation (pre-rotated query, butterfly pulled out of the
 *                        weighted sum, wave-level reductions, GQA n_rep).
 *   [benchmark page]     "TurboQuant benchmark on Apple Silicon" (zingnex.cn):
 *                        compression details, 128-token flushes, key/value bit flags.
 *   [news page]          "vLLM, llama.cpp, MLX all follow up" (digipub.cc), oMLX
 *                        section: decode attention reads the packed indices directly.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device memory; "host" pointers are CPU memory.
 *     The caller owns all memory.  The library allocates nothing and keeps no state
 *     between calls; it is reentrant.  The one exception is tq_decode_attn_noalloc,
 *     whose split partials live in a static device array of the library (one per GPU).
 *   - `stream` is a hipStream_t (NULL = the default stream).  tq_encode,
 *     tq_decode_attn and tq_materialize validate their arguments on the host, then
 *     enqueue kernels on `stream` and return without synchronising.
 *   - Every call returns TQ_OK or a negative tq_status.  Argument checks run before
 *     any HIP call, so an invalid or unsupported configuration fails immediately and
 *     loudly instead of degrading.  tq_last_error() returns a message for the most
 *     recent failure on the calling thread.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,      /* null / misaligned pointer, bad size, workspace too small  */
  TQ_ERR_UNSUPPORTED = -2,  /* configuration outside what the library implements        */
  TQ_ERR_CAPACITY = -3,     /* dst_offset + n_tokens exceeds the cache capacity         */
  TQ_ERR_HIP = -4           /* a HIP launch or runtime call failed                       */
} tq_status;

typedef enum { TQ_F16 = 0, TQ_BF16 = 1 } tq_dtype;

/* Key encodings.
 * TQ_K_F16     (MLX page, V-only mode: keys stay 16-bit, only the values are compressed):
 *   the key row is stored as given (layout->in_dtype bits); k_bits must be 16; decode
 *   is compiled for head_dim 64, 128, 256 and 512, fp16 or bf16 storage.
 * TQ_K_LM_MSE  (vLLM guide section 2 steps 1-2 only: the MSE-optimal codes without the
 *   QJL residual sketch; vLLM guide, MSE score kernel): n = |k| stored fp32, y = Pi k/n,
 *   idx_j = #{i : t_i < y_j} (k_bits in {2,3,4}); decoded key n Pi^T c[idx].  Its
 *   scores are the codebook term only (a biased, shrunk inner-product estimate).
 * TQ_K_LM_QJL  (vLLM guide section 2 steps 1-3): n = |k|, y = Pi k/n with the
 *   randomised Hadamard rotation Pi = H diag(s)/sqrt(d), idx_j = #{i : t_i < y_j}
 *   (Lloyd-Max, k_bits in {2,3,4}), r = y - c[idx], gamma = |r|, one QJL bit per
 *   dimension: bit_j = (z_j >= 0), z = S r (S the d x d Gaussian matrix).
 * TQ_K_AFFINE8 (vllm-metal guide, quantisation principle table: per-block affine,
 *   no rotation; its compression-ratio table: q8_0, q5_0, q4_0 and the 2-bit uint2/int2
 *   key widths): per 32-block a = fp16((max-min)/(2^k_bits - 1)), m = fp16(min),
 *   q = clamp(rne((k - m)/a), 0, 2^k_bits - 1)  (q = 0 where a = 0); k_bits 8, 5, 4 or 2.
 *   Decode of the 5/4/2-bit widths is compiled for head_dim 64 and 128 with rotated
 *   Lloyd-Max values, and for 512 with every value kind (TQ_ERR_UNSUPPORTED otherwise). */
typedef enum { TQ_K_LM_QJL = 0, TQ_K_AFFINE8 = 1, TQ_K_LM_MSE = 2, TQ_K_F16 = 3 } tq_kkind;

/* Value encodings.
 * TQ_V_GROUP_SYM (vLLM guide section 2 step 4, symmetric group-of-32 scaling):
 *   Delta = fp16(2 amax/(L-1)), L = 2^v_bits, v_bits in {2,4};
 *   idx = clamp(rne(v/Delta + (L-1)/2), 0, L-1) with the stored Delta (ties to even);
 *   Delta = 0 gives idx = L-1 / 0 / L/2 for v > 0 / v < 0 / v = 0.
 * TQ_V_LM_ROT (vllm-metal guide principle table; MLX page core technique): n = |v|
 *   stored fp32, y = Pi v/n with the value rotation, idx by the value codebook
 *   (v_bits in {2,3,4}); decoded value n Pi^T c[idx].
 * TQ_V_GROUP_ASYM (benchmark page, compression details: values keep a per-group minimum
 *   and maximum): per 32-group a = fp16((max - min)/(L-1)), m = fp16(min), v_bits in
 *   {2,4}; idx = clamp(rne((v - m)/a), 0, L-1) with the stored a, m (ties to even; a = 0
 *   gives idx = 0); decoded value m + a idx; aux plane one (a, m) fp16 pair per group.  */
typedef enum { TQ_V_GROUP_SYM = 0, TQ_V_LM_ROT = 1, TQ_V_GROUP_ASYM = 2 } tq_vkind;

typedef struct {
  int32_t head_dim;      /* d in {64, 128, 256, 512} (512: one-wave-per-token kernels,   *
                          * every key / value kind, n_rep <= 8 in decode)               */
  int32_t n_q_heads;     /* Hq                                                          */
  int32_t n_kv_heads;    /* Hkv; Hq % Hkv == 0; n_rep = Hq/Hkv in 1..8; q-head h reads
                            kv-head floor(h / n_rep)                                    */
  int32_t k_kind;        /* tq_kkind                                                    */
  int32_t k_bits;        /* 2, 3, 4 (LM_QJL / LM_MSE); 8, 5, 4, 2 (AFFINE8); 16 (F16)     */
  int32_t v_kind;        /* tq_vkind                                                    */
  int32_t v_bits;        /* 2, 4 (GROUP_SYM) or 2, 3, 4 (LM_ROT)                        */
  int32_t in_dtype;      /* tq_dtype of K/V passed to tq_encode and of q                */
  int32_t recent_dtype;  /* tq_dtype of the recent-buffer K/V passed to tq_decode_attn  */
} tq_layout;

/* Per-layer method state (device pointers, read-only).  Shared by every head and
 * token of the layer: one key rotation, one value rotation, one QJL matrix.
 *   k_centroids  float[2^k_bits], ascending       (TQ_K_LM_QJL / LM_MSE; else may be NULL)
 *   k_thresholds float[2^k_bits - 1]              (midpoints, from tq_make_codebook)
 *   v_centroids, v_thresholds                     (TQ_V_LM_ROT; else may be NULL)
 *   k_signs      uint32[d/32]: bit j%32 of word j/32 set <=> s_j = -1  (TQ_K_LM_QJL / LM_MSE)
 *   v_signs      uint32[d/32], same convention     (TQ_V_LM_ROT)
 *   qjl          fp16 bits [d*d], row-major S, S[i*d + j] (TQ_K_LM_QJL), 16-byte
 *                aligned: the Gaussian sketch is stored at fp16 resolution (its
 *                statistics do not depend on more), which keeps it exact in the fp16
 *                matrix-core projection                                           */
typedef struct {
  const float* k_centroids;
  const float* k_thresholds;
  const float* v_centroids;
  const float* v_thresholds;
  const uint32_t* k_signs;
  const uint32_t* v_signs;
  const uint16_t* qjl;
} tq_state;

/* The packed cache: five device planes, each laid out [batch][n_kv_heads][capacity][row]
 * (token-major within each (batch, kv-head) slice).  Row contents:
 *   k_codes  LM_QJL: uint32[W], b-bit code j in bits b*(j%P).. of word j/P, P = 16/10/8
 *                    codes per word for b = 2/3/4 (3-bit: bits 30..31 zero; MLX page:
 *                    ten 3-bit codes per uint32; vLLM guide: four 2-bit codes per byte)
 *            AFFINE8: k_bits 8: uint8[d], byte j = code j;  k_bits 4 / 2: packed like the
 *                    LM codes (8 / 16 per word);  k_bits 5: uint32[d/8] low nibbles (code j's
 *                    low 4 bits at bits 4 (j%8) of word j/8), then uint32[d/32] fifth bits
 *                    (bit j%32 of word d/8 + j/32)
 *   k_signs  LM_QJL: uint32[d/32], bit j%32 of word j/32 = QJL bit j   (else unused)
 *   k_aux    LM_QJL: fp16[2] = (n, gamma);  AFFINE8: fp16[d/32][2] = (a, m) per block;
 *            LM_MSE: fp32 n  (LM_MSE codes are packed like LM_QJL codes)
 *            F16: k_codes holds the d 16-bit key values (in_dtype bits); no k_aux plane
 *   v_codes  uint32[W], same packing as LM codes (GROUP_SYM v_bits 2/4, LM_ROT 2/3/4)
 *   v_aux    GROUP_SYM: fp16[d/32] scales Delta;  LM_ROT: fp32 n
 * tq_cache_plane_bytes gives each plane's size.                                        */
typedef struct {
  void* k_codes;
  void* k_signs;
  void* k_aux;
  void* v_codes;
  void* v_aux;
  int32_t batch;
  int32_t capacity;      /* token slots per (batch, kv-head) slice */
} tq_cache;

/* Lloyd-Max codebook for one coordinate of a uniformly rotated unit vector in R^d
 * (vLLM guide section 2 step 2: the optimal codebook for the rotated coordinate's Beta
 * distribution).  Density f(x) = C_d (1-x^2)^((d-3)/2) on [-1,1]; iterates the midpoint
 * and conditional-mean conditions in float64 to convergence, then rounds to float32.
 *   head_dim    8..4096, power of two not required
 *   bits        1..4
 *   centroids   host float[2^bits]     (out, ascending, c_i = -c_{L-1-i})
 *   thresholds  host float[2^bits - 1] (out, fp32 of the float64 midpoints)
 *   distortion  host double* or NULL   (out, per-coordinate MSE of the codebook)
 * Returns TQ_OK, TQ_ERR_INVALID (null output) or TQ_ERR_UNSUPPORTED (range).        */
int tq_make_codebook(int head_dim, int bits, float* centroids, float* thresholds, double* distortion);

/* Seeded rotation state (vLLM guide section 8: random orthogonal rotation and QJL
 * matrix).  SplitMix64 (Steele, Lea, Flood 2014) seeded with `seed`:
 *   signs word w = low 32 bits of output w, w = 0..d/32-1;
 *   S filled row-major in pairs by Box-Muller from the next two outputs x1, x2:
 *   u1 = ((x1>>11)+1)*2^-53, u2 = (x2>>11)*2^-53, rho = sqrt(-2 ln u1),
 *   (rho cos 2 pi u2, rho sin 2 pi u2), each rounded from float64 to fp16 (nearest even).
 *   head_dim  power of two, 32..4096;  signs host uint32[d/32] (out);
 *   qjl       host fp16 bits uint16[d*d] (out) or NULL.
 * Returns TQ_OK, TQ_ERR_INVALID or TQ_ERR_UNSUPPORTED.                             */
int tq_make_rotation(int head_dim, uint64_t seed, uint32_t* signs, uint16_t* qjl);

/* Bytes of each plane for `batch` x n_kv_heads x `capacity` tokens:
 * out[0..4] = k_codes, k_signs, k_aux, v_codes, v_aux (k_signs is 0 for AFFINE8).
 * Returns TQ_OK or an error for an invalid/unsupported layout.                     */
int tq_cache_plane_bytes(const tq_layout* layout, int batch, int capacity, size_t out[5]);

/* Encode n_tokens new tokens of every (batch, kv-head) into cache slots
 * [dst_offset, dst_offset + n_tokens)  (one call per 128-token flush, or one call over
 * the whole history; benchmark page: 128-token flushes).
 *   k, v      device, [batch][n_kv_heads][n_tokens][head_dim] in layout->in_dtype,
 *             contiguous.  Either may be NULL to encode only the other half.
 *   batch     must equal cache->batch
 * Errors: TQ_ERR_CAPACITY if dst_offset + n_tokens > cache->capacity; TQ_ERR_INVALID
 * for null/misaligned planes of the half being encoded or negative sizes;
 * TQ_ERR_UNSUPPORTED for layouts outside the compiled set or n_tokens * head_dim / 8
 * above 2^30 (split such a call); TQ_ERR_HIP on launch failure.
 * n_tokens == 0 is a no-op.                                                         */
int tq_encode(const tq_layout* layout, const tq_state* state, const void* k, const void* v,
              int batch, int n_tokens, int dst_offset, const tq_cache* cache, void* stream);

/* Workspace bytes tq_decode_attn needs for any n_compressed <= max_compressed. */
size_t tq_decode_workspace_bytes(const tq_layout* layout, int batch, int max_compressed);

/* Single-query decode attention (news page, oMLX section: attention read straight from
 * the packed indices; MLX page: pre-rotated query, weighted sum formed in the rotated
 * domain then one inverse butterfly, GQA n_rep without replicating KV; vLLM guide
 * section 5: exact recent buffer).  For q-head h of batch b, kv-head g = h / n_rep:
 *   LM_QJL keys:  s_t = n_t/sqrt(d) (<Pi q, c[idx_t]> + gamma_t sqrt(pi/2)/d <S Pi q, sigma_t>)
 *   LM_MSE keys:  s_t = n_t/sqrt(d) <Pi q, c[idx_t]>;  F16 keys: s_t = <q, k_t>/sqrt(d)
 *   AFFINE8 keys: s_t = <q, m + a q8_t>/sqrt(d);  recent keys: s_r = <q, k_r>/sqrt(d)
 *   out = softmax-weighted sum of decoded values over all n_compressed + n_recent
 *   tokens (GROUP_SYM: Delta (idx-(L-1)/2); LM_ROT: n Pi_v^T c[idx]; recent: v_r).
 *   q          device [batch][n_q_heads][head_dim], layout->in_dtype
 *   cache      packed planes; slots [0, n_compressed) of every slice are read
 *   recent_k/v device [batch][n_kv_heads][recent_capacity][head_dim], recent_dtype;
 *              slots [0, n_recent) are used; may be NULL when n_recent == 0
 *   n_recent   0..128, <= recent_capacity
 *   out        device float [batch][n_q_heads][head_dim]
 *   workspace  device, >= tq_decode_workspace_bytes(layout, batch, n_compressed)
 * Accumulation is float32.  Where the query heads of a kv-head share a tile on the matrix
 * cores, scores use fp16 hi/lo halves of the centroids (x8) and of the scaled queries, so
 * every product is exact and only the dropped lo x lo term (~2^-22 relative) is lost; value
 * weights are rounded once to fp16 as in the vector path.  Errors: TQ_ERR_INVALID when n_compressed + n_recent == 0,
 * n_recent > 128, a needed pointer is null/misaligned or the workspace is too small;
 * TQ_ERR_CAPACITY when n_compressed > cache->capacity; TQ_ERR_UNSUPPORTED; TQ_ERR_HIP. */
int tq_decode_attn(const tq_layout* layout, const tq_state* state, const void* q,
                   const tq_cache* cache, int n_compressed,
                   const void* recent_k, const void* recent_v, int n_recent, int recent_capacity,
                   float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Single-query decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as tq_decode_attn minus the
 * workspace: the split partials live in a static device array of the library, 16 MiB
 * (tq_decode_noalloc_max_scratch_bytes()), one per GPU the library runs on, held until
 * the process ends.  A decode whose partials need more (tq_decode_workspace_bytes above
 * the maximum) fails with TQ_ERR_CAPACITY before any launch.  The call allocates nothing;
 * its first call on a device looks up that device's copy of the array.  The array keeps
 * the last call's contents; nothing in it needs clearing (every partial is written before
 * it is read).  Calls that overlap on one GPU share the array and race: serialise them
 * (one stream, or events) per device.                                                    */
int tq_decode_attn_noalloc(const tq_layout* layout, const tq_state* state, const void* q,
                           const tq_cache* cache, int n_compressed,
                           const void* recent_k, const void* recent_v, int n_recent, int recent_capacity,
                           float* out, void* stream);

/* Size of tq_decode_attn_noalloc's static scratch array in bytes. */
size_t tq_decode_noalloc_max_scratch_bytes(void);

/* Workspace bytes tq_decode_attn_multi needs for n_query queries and any
 * n_compressed <= max_compressed (0 for an invalid layout or n_query outside 1..8). */
size_t tq_decode_multi_workspace_bytes(const tq_layout* layout, int batch, int n_query, int max_compressed);

/* Multi-query decode attention: n_query consecutive query tokens per sequence (a short
 * suffix, or the draft tokens of a speculative step) scored against the same cache in
 * one pass over the packed planes (vllm-metal guide, prefill section: short suffixes,
 * decode steps and speculative verification stay on the compressed kernels; the scores
 * and values are those of tq_decode_attn).  The caller appends the queries' own keys
 * and values to the recent buffer first: its last n_query tokens are the queries', in
 * order, and query j (0-based) attends to every compressed token and to recent tokens
 * 0 .. n_recent - n_query + j (causal inside the suffix).  With n_query == 1 this is
 * exactly tq_decode_attn.
 *   q          device [batch][n_query][n_q_heads][head_dim], layout->in_dtype
 *   out        device float [batch][n_query][n_q_heads][head_dim]
 *   n_recent   n_query..128, <= recent_capacity; recent_k/v as for tq_decode_attn
 *   workspace  device, >= tq_decode_multi_workspace_bytes(layout, batch, n_query, n_compressed)
 * Compiled for LM_QJL keys (3 or 4 bits) with GROUP_SYM values (2 or 4 bits), head_dim 64
 * and 128: n_query 2 with n_rep 1..8, n_query 4 with n_rep 1, 2, 4, n_query 8 with n_rep
 * 1, 2 (n_query * n_rep <= 16: the query rows share one 16-column matrix-core operand);
 * other combinations with n_query > 1 return TQ_ERR_UNSUPPORTED.  Errors: TQ_ERR_INVALID when n_query is outside 1..8,
 * n_recent < n_query or > 128, a needed pointer is null/misaligned or the workspace is
 * too small; TQ_ERR_CAPACITY; TQ_ERR_UNSUPPORTED; TQ_ERR_HIP. */
int tq_decode_attn_multi(const tq_layout* layout, const tq_state* state, const void* q, int n_query,
                         const tq_cache* cache, int n_compressed,
                         const void* recent_k, const void* recent_v, int n_recent, int recent_capacity,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Materialisation: dequantise cache slots [t0, t0 + n_tokens) of every (batch,
 * kv-head) slice into natural-domain rows (vllm-metal guide, prefill section: long
 * prefills materialise the compressed history and run ordinary attention on it; vLLM
 * guide, section 7: the hybrid path dequantises the whole history).  Row t of slice
 * (b, g) is exactly the decoded vector the decode attention uses:
 *   LM_QJL keys:    k = n Pi^T (c[idx] + gamma sqrt(pi/2)/d S^T sigma)
 *   LM_MSE keys:    k = n Pi^T c[idx];   F16 keys: the stored row (converted to out_dtype)
 *   AFFINE8 keys:   k_j = m + a q8_j
 *   GROUP_SYM vals: v_j = Delta (idx_j - (L-1)/2)
 *   LM_ROT values:  v = n Pi_v^T c[idx]
 * computed in float32 (the S^T sigma term on fp16 matrix cores: sigma and S are exact
 * in fp16, the products exact, the sums fp32) and rounded once to out_dtype (nearest
 * even).
 *   out_k, out_v  device, [batch][n_kv_heads][n_tokens][head_dim] of out_dtype bits,
 *                 contiguous; either may be NULL to materialise only the other half
 *   out_dtype     TQ_F16 or TQ_BF16
 * The state fields the decode needs for a half are needed here too.  Errors:
 * TQ_ERR_INVALID for both outputs NULL, null/misaligned pointers or negative sizes;
 * TQ_ERR_CAPACITY if t0 + n_tokens > cache->capacity; TQ_ERR_UNSUPPORTED for an
 * unknown out_dtype or batch * n_kv_heads * n_tokens * head_dim / 8 >= 2^31
 * (split such a call); TQ_ERR_HIP.  n_tokens == 0 is a no-op.                       */
int tq_materialize(const tq_layout* layout, const tq_state* state, const tq_cache* cache, int t0, int n_tokens,
                   void* out_k, void* out_v, int out_dtype, void* stream);

/* Static description of a status code. */
const char* tq_strerror(int status);

/* Message for the most recent failed call on this thread ("" if none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */

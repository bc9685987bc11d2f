// Internal declarations shared by the host glue (tq_capi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/tq.h"

namespace tq {

// Tokens per encode tile and per decode tile.
constexpr int kTile = 64;
// Largest recent buffer accepted by the decode (vLLM guide, section 5: 128-token buffer).
constexpr int kMaxRecent = 128;
// Most queries of one multi-query decode step (vllm-metal guide, prefill section: short
// suffixes and speculative verification stay on the compressed kernels).
constexpr int kMaxQueries = 8;
// Decode work-group count the split bound is sized for (4 per CU on 256 CUs), and the
// fewest 64-token tiles a split gets (two per wave: the query preparation is amortised
// over eight tiles).
constexpr int kTargetDecodeGroups = 1024;
constexpr int kMinTilesPerSplit = 8;

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Words per row of each plane.
int lm_words(int d, int bits);          // LM / group codes: ceil(d / codes_per_word)
int k_code_words(const tq_layout& L);
int k_sign_words(const tq_layout& L);
int k_aux_words(const tq_layout& L);
int v_code_words(const tq_layout& L);
int v_aux_bytes(const tq_layout& L);

// Decode split policy (shared by the workspace size and the launch).
struct DecodePlan {
  int n_splits;      // splits per (batch, kv-head)
  int chunk;         // tokens per split (multiple of kTile)
  size_t q_floats;   // floats of the prepared query block per (batch, q-head)
  size_t part_stride;  // floats per partial result (m, l, pad, pad, acc[d])
  size_t ws_bytes;   // bytes this plan uses
};
DecodePlan plan_decode(const tq_layout& L, int batch, int n_compressed);
size_t decode_ws_bound(const tq_layout& L, int batch, int max_compressed);
size_t decode_multi_ws_bound(const tq_layout& L, int batch, int n_query, int max_compressed);

// Launchers (enqueue only; argument checks are done by the caller).
hipError_t launch_encode_k(const tq_layout& L, const tq_state& S, const void* k, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st);
hipError_t launch_encode_v(const tq_layout& L, const tq_state& S, const void* v, int batch, int n_tokens,
                           int dst_offset, const tq_cache& C, hipStream_t st);
hipError_t launch_decode(const tq_layout& L, const tq_state& S, const void* q, const tq_cache& C,
                         int n_compressed, const void* rk, const void* rv, int n_recent, int recent_cap,
                         float* out, void* ws, const DecodePlan& plan, hipStream_t st);

hipError_t launch_decode_multi(const tq_layout& L, const tq_state& S, const void* q, int n_query, const tq_cache& C,
                               int n_compressed, const void* rk, const void* rv, int n_recent, int recent_cap,
                               float* out, void* ws, const DecodePlan& plan, hipStream_t st);
hipError_t launch_materialize_k(const tq_layout& L, const tq_state& S, const tq_cache& C, int t0, int n_tokens,
                                void* out, int out_dtype, hipStream_t st);
hipError_t launch_materialize_v(const tq_layout& L, const tq_state& S, const tq_cache& C, int t0, int n_tokens,
                                void* out, int out_dtype, hipStream_t st);

// head_dim 512, rotated kinds (the other kinds use the generic templates).
hipError_t launch_encode_lm512(const tq_layout& L, const tq_state& S, const void* x, int batch, int n_tokens,
                               int dst_offset, const tq_cache& C, hipStream_t st, bool values);
hipError_t launch_materialize_lm512(const uint32_t* codes, const uint32_t* signs, const uint32_t* aux,
                                    const float* cent, const uint32_t* rsign, const uint16_t* S, int bits, bool qjl,
                                    long slices, int n, int cap, int t0, uint16_t* out, int out_dtype,
                                    hipStream_t st);

// Whether a kernel instantiation exists for this layout.
bool encode_k_compiled(const tq_layout& L);
bool encode_v_compiled(const tq_layout& L);
bool decode_compiled(const tq_layout& L);
bool decode_multi_compiled(const tq_layout& L, int n_query);
bool materialize_compiled(const tq_layout& L);

// Per-thread error message (set by the C-ABI entry points and launchers).
void set_error(const char* fmt, ...);

}  // namespace tq

// C ABI of libtq: argument validation, host-side method state, dispatch to the kernels.
// Every check here runs before any HIP call, so unsupported or invalid requests fail
// immediately with a status code and a message (vllm-metal TurboQuant guide, support
// limits section: unsupported configurations must fail at start-up, not degrade).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "tq_internal.h"

namespace tq {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int lm_words(int d, int bits) {
  const int per = (bits == 3) ? 10 : 32 / bits;
  return (d + per - 1) / per;
}
int k_code_words(const tq_layout& L) {
  if (L.k_kind == TQ_K_AFFINE8)   // per-block affine: bytes (8), nibble + fifth-bit planes (5), 4/2-bit words
    return L.k_bits == 8 ? L.head_dim / 4 : (L.k_bits == 5 ? L.head_dim / 8 + L.head_dim / 32 : L.head_dim * L.k_bits / 32);
  if (L.k_kind == TQ_K_F16) return L.head_dim / 2;
  return lm_words(L.head_dim, L.k_bits);
}
int k_sign_words(const tq_layout& L) { return L.k_kind == TQ_K_LM_QJL ? L.head_dim / 32 : 0; }
int k_aux_words(const tq_layout& L) {
  if (L.k_kind == TQ_K_AFFINE8) return L.head_dim / 32;
  return L.k_kind == TQ_K_F16 ? 0 : 1;
}
int v_code_words(const tq_layout& L) { return lm_words(L.head_dim, L.v_bits); }
int v_aux_bytes(const tq_layout& L) {
  if (L.v_kind == TQ_V_GROUP_SYM) return (L.head_dim / 32) * 2;
  if (L.v_kind == TQ_V_GROUP_ASYM) return (L.head_dim / 32) * 4;   // (a, m) fp16 per group
  return 4;
}

}  // namespace tq

using namespace tq;

namespace {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  set_error("%s: %s", tq_strerror(code), buf);
  return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

// Layout checks common to every call.  Returns TQ_OK or an error code (message set).
int check_layout(const tq_layout* L) {
  if (!L) return fail(TQ_ERR_INVALID, "layout is NULL");
  const int d = L->head_dim;
  if (!(d == 64 || d == 128 || d == 256 || d == 512))
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %d: must be 64, 128, 256 or 512", d);
  if (L->n_q_heads <= 0 || L->n_kv_heads <= 0)
    return fail(TQ_ERR_INVALID, "head counts must be positive (n_q_heads %d, n_kv_heads %d)", L->n_q_heads,
                L->n_kv_heads);
  if (L->n_q_heads % L->n_kv_heads)
    return fail(TQ_ERR_UNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d", L->n_q_heads, L->n_kv_heads);
  if (L->k_kind == TQ_K_LM_QJL || L->k_kind == TQ_K_LM_MSE) {
    if (L->k_bits < 2 || L->k_bits > 4) return fail(TQ_ERR_UNSUPPORTED, "LM keys need k_bits 2..4, got %d", L->k_bits);
  } else if (L->k_kind == TQ_K_AFFINE8) {
    if (L->k_bits != 8 && L->k_bits != 5 && L->k_bits != 4 && L->k_bits != 2)
      return fail(TQ_ERR_UNSUPPORTED, "affine keys need k_bits 8, 5, 4 or 2, got %d", L->k_bits);
  } else if (L->k_kind == TQ_K_F16) {
    if (L->k_bits != 16) return fail(TQ_ERR_UNSUPPORTED, "16-bit keys need k_bits 16, got %d", L->k_bits);
  } else {
    return fail(TQ_ERR_UNSUPPORTED, "unknown k_kind %d", L->k_kind);
  }
  if (L->v_kind == TQ_V_GROUP_SYM || L->v_kind == TQ_V_GROUP_ASYM) {
    if (L->v_bits != 2 && L->v_bits != 4) return fail(TQ_ERR_UNSUPPORTED, "group values need v_bits 2 or 4, got %d", L->v_bits);
  } else if (L->v_kind == TQ_V_LM_ROT) {
    if (L->v_bits < 2 || L->v_bits > 4) return fail(TQ_ERR_UNSUPPORTED, "rotated LM values need v_bits 2..4, got %d", L->v_bits);
  } else {
    return fail(TQ_ERR_UNSUPPORTED, "unknown v_kind %d", L->v_kind);
  }
  if (L->in_dtype != TQ_F16 && L->in_dtype != TQ_BF16) return fail(TQ_ERR_UNSUPPORTED, "in_dtype %d", L->in_dtype);
  if (L->recent_dtype != TQ_F16 && L->recent_dtype != TQ_BF16)
    return fail(TQ_ERR_UNSUPPORTED, "recent_dtype %d", L->recent_dtype);
  return TQ_OK;
}

int check_cache(const tq_cache* C, bool need_k, bool need_v, const tq_layout* L) {
  if (!C) return fail(TQ_ERR_INVALID, "cache is NULL");
  if (C->batch <= 0 || C->capacity <= 0)
    return fail(TQ_ERR_INVALID, "cache batch %d / capacity %d must be positive", C->batch, C->capacity);
  if (need_k) {
    const bool aux = L->k_kind != TQ_K_F16;   // 16-bit keys have no aux plane
    if (!C->k_codes || !aligned16(C->k_codes) || (aux && (!C->k_aux || !aligned16(C->k_aux))))
      return fail(TQ_ERR_INVALID, "key planes must be non-NULL and 16-byte aligned");
    if (L->k_kind == TQ_K_LM_QJL && (!C->k_signs || !aligned16(C->k_signs)))
      return fail(TQ_ERR_INVALID, "k_signs plane must be non-NULL and 16-byte aligned");
  }
  if (need_v && (!C->v_codes || !C->v_aux || !aligned16(C->v_codes) || !aligned16(C->v_aux)))
    return fail(TQ_ERR_INVALID, "value planes must be non-NULL and 16-byte aligned");
  return TQ_OK;
}

int check_state(const tq_state* S, const tq_layout* L, bool need_k, bool need_v) {
  if (!S) return fail(TQ_ERR_INVALID, "state is NULL");
  if (need_k && L->k_kind == TQ_K_LM_QJL) {
    if (!S->k_centroids || !S->k_thresholds || !S->k_signs || !S->qjl)
      return fail(TQ_ERR_INVALID, "LM+QJL keys need k_centroids, k_thresholds, k_signs and qjl");
    if (!aligned4(S->k_centroids) || !aligned4(S->k_thresholds) || !aligned4(S->k_signs) || !aligned16(S->qjl))
      return fail(TQ_ERR_INVALID, "state arrays must be 4-byte aligned");
  }
  if (need_k && L->k_kind == TQ_K_LM_MSE) {
    if (!S->k_centroids || !S->k_thresholds || !S->k_signs)
      return fail(TQ_ERR_INVALID, "MSE-only LM keys need k_centroids, k_thresholds and k_signs");
    if (!aligned4(S->k_centroids) || !aligned4(S->k_thresholds) || !aligned4(S->k_signs))
      return fail(TQ_ERR_INVALID, "state arrays must be 4-byte aligned");
  }
  if (need_v && L->v_kind == TQ_V_LM_ROT) {
    if (!S->v_centroids || !S->v_thresholds || !S->v_signs)
      return fail(TQ_ERR_INVALID, "rotated LM values need v_centroids, v_thresholds and v_signs");
    if (!aligned4(S->v_centroids) || !aligned4(S->v_thresholds) || !aligned4(S->v_signs))
      return fail(TQ_ERR_INVALID, "state arrays must be 4-byte aligned");
  }
  return TQ_OK;
}

// Every host check of a single-query decode except the workspace; fills the split plan.
int check_decode(const tq_layout* L, const tq_state* S, const void* q, const tq_cache* C, int n_compressed,
                 const void* recent_k, const void* recent_v, int n_recent, int recent_capacity, float* out,
                 DecodePlan* plan) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (!q || !out) return fail(TQ_ERR_INVALID, "q and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(TQ_ERR_INVALID, "q and out must be 16-byte aligned");
  if (n_compressed < 0 || n_recent < 0) return fail(TQ_ERR_INVALID, "negative token count");
  if (n_recent > kMaxRecent) return fail(TQ_ERR_INVALID, "n_recent %d > %d", n_recent, kMaxRecent);
  if (n_compressed + n_recent == 0) return fail(TQ_ERR_INVALID, "nothing to attend to (no compressed and no recent tokens)");
  if (n_recent > 0) {
    if (!recent_k || !recent_v) return fail(TQ_ERR_INVALID, "recent_k/recent_v are NULL with n_recent %d", n_recent);
    if (!aligned16(recent_k) || !aligned16(recent_v)) return fail(TQ_ERR_INVALID, "recent buffers must be 16-byte aligned");
    if (recent_capacity < n_recent) return fail(TQ_ERR_INVALID, "recent_capacity %d < n_recent %d", recent_capacity, n_recent);
  }
  if ((rc = check_cache(C, n_compressed > 0, n_compressed > 0, L))) return rc;
  if ((rc = check_state(S, L, true, true))) return rc;
  if (L->k_kind == TQ_K_LM_QJL && (!S->k_signs || !S->qjl)) return fail(TQ_ERR_INVALID, "k_signs and qjl are needed");
  if (n_compressed > C->capacity)
    return fail(TQ_ERR_CAPACITY, "n_compressed %d > capacity %d", n_compressed, C->capacity);
  if (!decode_compiled(*L))
    return fail(TQ_ERR_UNSUPPORTED, "no decode kernel compiled for head_dim %d, n_rep %d, key/value kinds %d/%d bits %d/%d",
                L->head_dim, L->n_q_heads / L->n_kv_heads, L->k_kind, L->k_bits, L->v_kind, L->v_bits);
  *plan = plan_decode(*L, C->batch, n_compressed);
  return TQ_OK;
}

// ---------------------------------------------------------------------------------------
// Lloyd-Max codebook on the exact coordinate density, by Gauss-Legendre quadrature.
// ---------------------------------------------------------------------------------------
// Gauss-Legendre rule on [-1, 1]: nodes are the roots of the Legendre polynomial P_n,
// found by Newton's method from the Chebyshev-like start cos(pi (i - 1/4) / (n + 1/2));
// weights 2 / ((1 - x^2) P_n'(x)^2).
struct GaussLegendre {
  static constexpr int n = 16;
  double x[n], w[n];
  GaussLegendre() {
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5)), dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;   // P_0, P_1; recurrence k P_k = (2k-1) z P_{k-1} - (k-1) P_{k-2}
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};
const GaussLegendre& gl_rule() {
  static const GaussLegendre r;
  return r;
}

struct Density {
  int d;
  double logc;   // log of Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2))
  explicit Density(int dd) : d(dd) {
    logc = std::lgamma(0.5 * dd) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (dd - 1));
  }
  double f(double x) const {
    const double u = 1.0 - x * x;
    if (u <= 0.0) return 0.0;
    return std::exp(logc + 0.5 * (d - 3) * std::log(u));
  }
  // (mass, first moment) over [a, b], composite 16-point Gauss-Legendre on panels of
  // width <= 1/(4 sqrt(d)) (the density's scale is 1/sqrt(d)).
  void moments(double a, double b, double* m0, double* m1) const {
    const GaussLegendre& gl = gl_rule();
    const double hmax = 0.25 / std::sqrt((double)d);
    const int n = std::max(1, (int)std::ceil((b - a) / hmax));
    const double h = (b - a) / n;
    double s0 = 0.0, s1 = 0.0;
    for (int i = 0; i < n; ++i) {
      const double mid = a + (i + 0.5) * h, half = 0.5 * h;
      for (int k = 0; k < GaussLegendre::n; ++k) {
        const double x = mid + half * gl.x[k];
        const double w = half * gl.w[k] * f(x);
        s0 += w;
        s1 += w * x;
      }
    }
    *m0 = s0;
    *m1 = s1;
  }
};

// inverse standard normal CDF by bisection (only used for the starting point)
double norm_quantile(double p) {
  double lo = -10.0, hi = 10.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// float64 -> fp16 bits, round to nearest even (directly, no float32 step).
uint16_t f64_to_f16_bits(double x) {
  uint64_t b;
  std::memcpy(&b, &x, 8);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  b &= 0x7FFFFFFFFFFFFFFFull;
  if (b >= 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7C00u | (b > 0x7FF0000000000000ull ? 0x200u : 0u));
  if (b == 0) return (uint16_t)sign;
  const int e = (int)(b >> 52) - 1023;
  const uint64_t m = (b & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
  if (e < -25) return (uint16_t)sign;
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  uint64_t keep = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) keep += 1;
  if (e >= -14) {
    int ee = e + 15;
    if (keep == (1ull << 11)) { keep >>= 1; ee += 1; }
    if (ee >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)ee << 10) | ((uint32_t)keep & 0x3FFu));
  }
  return (uint16_t)(sign | (uint32_t)keep);
}

}  // namespace

extern "C" {

int tq_materialize(const tq_layout* L, const tq_state* S, const tq_cache* C, int t0, int n_tokens, void* out_k,
                   void* out_v, int out_dtype, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (!out_k && !out_v) return fail(TQ_ERR_INVALID, "both out_k and out_v are NULL");
  if ((out_k && !aligned16(out_k)) || (out_v && !aligned16(out_v)))
    return fail(TQ_ERR_INVALID, "out_k/out_v must be 16-byte aligned");
  if (out_dtype != TQ_F16 && out_dtype != TQ_BF16) return fail(TQ_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if ((rc = check_cache(C, out_k != nullptr, out_v != nullptr, L))) return rc;
  if ((rc = check_state(S, L, out_k != nullptr, out_v != nullptr))) return rc;
  if (t0 < 0 || n_tokens < 0) return fail(TQ_ERR_INVALID, "t0 %d / n_tokens %d negative", t0, n_tokens);
  if ((long)t0 + n_tokens > C->capacity)
    return fail(TQ_ERR_CAPACITY, "t0 %d + n_tokens %d > capacity %d", t0, n_tokens, C->capacity);
  if ((long)C->batch * L->n_kv_heads * n_tokens * (L->head_dim / 8) > 0x7FFFFFFFL)
    return fail(TQ_ERR_UNSUPPORTED, "batch x kv-heads x n_tokens too large for one call (split it)");
  if (!materialize_compiled(*L))
    return fail(TQ_ERR_UNSUPPORTED, "no materialisation kernel compiled for head_dim %d", L->head_dim);
  if (n_tokens == 0) return TQ_OK;
  hipStream_t st = (hipStream_t)stream;
  if (out_k) {
    hipError_t e = launch_materialize_k(*L, *S, *C, t0, n_tokens, out_k, out_dtype, st);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "key materialisation launch: %s", hipGetErrorString(e));
  }
  if (out_v) {
    hipError_t e = launch_materialize_v(*L, *S, *C, t0, n_tokens, out_v, out_dtype, st);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "value materialisation launch: %s", hipGetErrorString(e));
  }
  return TQ_OK;
}

const char* tq_strerror(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_CAPACITY: return "cache capacity exceeded";
    case TQ_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* tq_last_error(void) { return g_err; }

int tq_make_codebook(int head_dim, int bits, float* centroids, float* thresholds, double* distortion) {
  if (!centroids || !thresholds) return fail(TQ_ERR_INVALID, "centroids/thresholds output is NULL");
  if (head_dim < 8 || head_dim > 4096) return fail(TQ_ERR_UNSUPPORTED, "head_dim %d outside 8..4096", head_dim);
  if (bits < 1 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits %d outside 1..4", bits);
  const int L = 1 << bits;
  const Density den(head_dim);
  std::vector<double> c(L), nc(L), t(L + 1), p(L);
  for (int i = 0; i < L; ++i) c[i] = norm_quantile((i + 0.5) / L) / std::sqrt((double)head_dim);
  double best = 1e300;
  int stall = 0;
  for (int it = 0; it < 200000; ++it) {
    t[0] = -1.0;
    t[L] = 1.0;
    for (int i = 1; i < L; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
    for (int i = 0; i < L; ++i) {
      double m0, m1;
      den.moments(t[i], t[i + 1], &m0, &m1);
      nc[i] = m1 / m0;
      p[i] = m0;
    }
    double delta = 0.0;
    for (int i = 0; i < L; ++i) {
      const double sym = 0.5 * (nc[i] - nc[L - 1 - i]);   // the density is even
      delta = std::max(delta, std::fabs(sym - c[i]));
      c[i] = sym;
    }
    if (delta < best) { best = delta; stall = 0; } else { ++stall; }
    if (delta <= 4e-16 || (best < 1e-13 && stall >= 50)) break;
  }
  if (best > 1e-12) return fail(TQ_ERR_UNSUPPORTED, "Lloyd-Max did not converge (d=%d, bits=%d)", head_dim, bits);
  double dist = 1.0 / head_dim;
  for (int i = 0; i < L; ++i) {
    centroids[i] = (float)c[i];
    dist -= p[i] * c[i] * c[i];
  }
  for (int i = 0; i + 1 < L; ++i) thresholds[i] = (float)(0.5 * (c[i] + c[i + 1]));
  if (distortion) *distortion = dist;
  return TQ_OK;
}

int tq_make_rotation(int head_dim, uint64_t seed, uint32_t* signs, uint16_t* qjl) {
  if (!signs) return fail(TQ_ERR_INVALID, "signs output is NULL");
  if (head_dim < 32 || head_dim > 4096 || (head_dim & (head_dim - 1)))
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %d must be a power of two in 32..4096", head_dim);
  uint64_t state = seed;
  auto next = [&state]() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  for (int w = 0; w < head_dim / 32; ++w) signs[w] = (uint32_t)(next() & 0xFFFFFFFFull);
  if (qjl) {
    const size_t n = (size_t)head_dim * head_dim;
    for (size_t i = 0; i < n; i += 2) {
      const uint64_t x1 = next(), x2 = next();
      const double u1 = (double)((x1 >> 11) + 1) * 0x1.0p-53;
      const double u2 = (double)(x2 >> 11) * 0x1.0p-53;
      const double rho = std::sqrt(-2.0 * std::log(u1));
      qjl[i] = f64_to_f16_bits(rho * std::cos(2.0 * M_PI * u2));
      qjl[i + 1] = f64_to_f16_bits(rho * std::sin(2.0 * M_PI * u2));
    }
  }
  return TQ_OK;
}

int tq_cache_plane_bytes(const tq_layout* L, int batch, int capacity, size_t out[5]) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (!out) return fail(TQ_ERR_INVALID, "out is NULL");
  if (batch <= 0 || capacity <= 0) return fail(TQ_ERR_INVALID, "batch %d / capacity %d must be positive", batch, capacity);
  const size_t rows = (size_t)batch * L->n_kv_heads * capacity;
  out[0] = rows * 4 * k_code_words(*L);
  out[1] = rows * 4 * k_sign_words(*L);
  out[2] = rows * 4 * k_aux_words(*L);
  out[3] = rows * 4 * v_code_words(*L);
  out[4] = rows * v_aux_bytes(*L);
  return TQ_OK;
}

int tq_encode(const tq_layout* L, const tq_state* S, const void* k, const void* v, int batch, int n_tokens,
              int dst_offset, const tq_cache* C, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (!k && !v) return fail(TQ_ERR_INVALID, "both k and v are NULL");
  if ((k && !aligned16(k)) || (v && !aligned16(v))) return fail(TQ_ERR_INVALID, "k/v inputs must be 16-byte aligned");
  if ((rc = check_cache(C, k != nullptr, v != nullptr, L))) return rc;
  if ((rc = check_state(S, L, k != nullptr, v != nullptr))) return rc;
  if (batch != C->batch) return fail(TQ_ERR_INVALID, "batch %d != cache batch %d", batch, C->batch);
  if (n_tokens < 0 || dst_offset < 0) return fail(TQ_ERR_INVALID, "n_tokens %d / dst_offset %d negative", n_tokens, dst_offset);
  if ((long)dst_offset + n_tokens > C->capacity)
    return fail(TQ_ERR_CAPACITY, "dst_offset %d + n_tokens %d > capacity %d", dst_offset, n_tokens, C->capacity);
  if ((long)n_tokens * (L->head_dim / 8) > (1L << 30))
    return fail(TQ_ERR_UNSUPPORTED, "n_tokens %d too large for one call (split it)", n_tokens);
  if (k && !encode_k_compiled(*L)) return fail(TQ_ERR_UNSUPPORTED, "no key encoder compiled for this layout (head_dim %d)", L->head_dim);
  if (v && !encode_v_compiled(*L)) return fail(TQ_ERR_UNSUPPORTED, "no value encoder compiled for this layout (head_dim %d)", L->head_dim);
  if (n_tokens == 0) return TQ_OK;
  hipStream_t st = (hipStream_t)stream;
  if (k) {
    hipError_t e = launch_encode_k(*L, *S, k, batch, n_tokens, dst_offset, *C, st);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "key encode launch: %s", hipGetErrorString(e));
  }
  if (v) {
    hipError_t e = launch_encode_v(*L, *S, v, batch, n_tokens, dst_offset, *C, st);
    if (e != hipSuccess) return fail(TQ_ERR_HIP, "value encode launch: %s", hipGetErrorString(e));
  }
  return TQ_OK;
}

size_t tq_decode_workspace_bytes(const tq_layout* L, int batch, int max_compressed) {
  if (check_layout(L) || batch <= 0 || max_compressed < 0) return 0;
  return decode_ws_bound(*L, batch, max_compressed);
}

int tq_decode_attn(const tq_layout* L, const tq_state* S, const void* q, const tq_cache* C, int n_compressed,
                   const void* recent_k, const void* recent_v, int n_recent, int recent_capacity, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(TQ_ERR_INVALID, "workspace must be non-NULL");
  if (!aligned16(workspace)) return fail(TQ_ERR_INVALID, "workspace must be 16-byte aligned");
  DecodePlan plan{};
  int rc = check_decode(L, S, q, C, n_compressed, recent_k, recent_v, n_recent, recent_capacity, out, &plan);
  if (rc) return rc;
  if (workspace_bytes < plan.ws_bytes)
    return fail(TQ_ERR_INVALID, "workspace %zu bytes < %zu needed", workspace_bytes, plan.ws_bytes);
  hipError_t e = launch_decode(*L, *S, q, *C, n_compressed, recent_k, recent_v, n_recent,
                               n_recent > 0 ? recent_capacity : 1, out, workspace, plan, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Decode without a caller workspace: the split partials live in a fixed device array of
// this library (one copy per GPU, held until the process ends).  The host never touches the
// array through its name: the device address comes from hipGetSymbolAddress, once per
// device, with that device current.  The partials are written in full before the merge
// reads them, so nothing has to be cleared between calls; calls that overlap on one GPU
// share the array and race.
// ---------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call on the device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TQ_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

size_t tq_decode_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

int tq_decode_attn_noalloc(const tq_layout* L, const tq_state* S, const void* q, const tq_cache* C, int n_compressed,
                           const void* recent_k, const void* recent_v, int n_recent, int recent_capacity, float* out,
                           void* stream) {
  DecodePlan plan{};
  int rc = check_decode(L, S, q, C, n_compressed, recent_k, recent_v, n_recent, recent_capacity, out, &plan);
  if (rc) return rc;
  if (plan.ws_bytes > kScratchBytes)
    return fail(TQ_ERR_CAPACITY, "this decode needs %zu bytes of split partials, above the %zu-byte static scratch of "
                "tq_decode_attn_noalloc (use tq_decode_attn with a workspace)", plan.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  hipError_t e = launch_decode(*L, *S, q, *C, n_compressed, recent_k, recent_v, n_recent,
                               n_recent > 0 ? recent_capacity : 1, out, ws, plan, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

size_t tq_decode_multi_workspace_bytes(const tq_layout* L, int batch, int n_query, int max_compressed) {
  if (check_layout(L) || batch <= 0 || n_query <= 0 || n_query > kMaxQueries || max_compressed < 0) return 0;
  return decode_multi_ws_bound(*L, batch, n_query, max_compressed);
}

int tq_decode_attn_multi(const tq_layout* L, const tq_state* S, const void* q, int n_query, const tq_cache* C,
                         int n_compressed, const void* recent_k, const void* recent_v, int n_recent,
                         int recent_capacity, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layout(L);
  if (rc) return rc;
  if (n_query < 1 || n_query > kMaxQueries) return fail(TQ_ERR_INVALID, "n_query %d outside 1..%d", n_query, kMaxQueries);
  if (n_recent < n_query)
    return fail(TQ_ERR_INVALID, "n_recent %d < n_query %d: the queries' own keys/values must be the last recent tokens",
                n_recent, n_query);
  if (n_query == 1)
    return tq_decode_attn(L, S, q, C, n_compressed, recent_k, recent_v, n_recent, recent_capacity, out, workspace,
                          workspace_bytes, stream);
  if (!q || !out || !workspace) return fail(TQ_ERR_INVALID, "q, out and workspace must be non-NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(TQ_ERR_INVALID, "q, out and workspace must be 16-byte aligned");
  if (n_compressed < 0) return fail(TQ_ERR_INVALID, "negative token count");
  if (n_recent > kMaxRecent) return fail(TQ_ERR_INVALID, "n_recent %d > %d", n_recent, kMaxRecent);
  if (!recent_k || !recent_v) return fail(TQ_ERR_INVALID, "recent_k/recent_v are NULL with n_recent %d", n_recent);
  if (!aligned16(recent_k) || !aligned16(recent_v)) return fail(TQ_ERR_INVALID, "recent buffers must be 16-byte aligned");
  if (recent_capacity < n_recent) return fail(TQ_ERR_INVALID, "recent_capacity %d < n_recent %d", recent_capacity, n_recent);
  if ((rc = check_cache(C, n_compressed > 0, n_compressed > 0, L))) return rc;
  if ((rc = check_state(S, L, true, true))) return rc;
  if (L->k_kind == TQ_K_LM_QJL && (!S->k_signs || !S->qjl)) return fail(TQ_ERR_INVALID, "k_signs and qjl are needed");
  if (n_compressed > C->capacity)
    return fail(TQ_ERR_CAPACITY, "n_compressed %d > capacity %d", n_compressed, C->capacity);
  if (!decode_multi_compiled(*L, n_query))
    return fail(TQ_ERR_UNSUPPORTED,
                "no multi-query decode kernel for head_dim %d, n_rep %d, n_query %d, key/value kinds %d/%d bits %d/%d",
                L->head_dim, L->n_q_heads / L->n_kv_heads, n_query, L->k_kind, L->k_bits, L->v_kind, L->v_bits);
  DecodePlan plan = plan_decode(*L, C->batch, n_compressed);
  const size_t need = decode_multi_ws_bound(*L, C->batch, n_query, n_compressed);
  if (workspace_bytes < need) return fail(TQ_ERR_INVALID, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  hipError_t e = launch_decode_multi(*L, *S, q, n_query, *C, n_compressed, recent_k, recent_v, n_recent,
                                     recent_capacity, out, workspace, plan, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "multi-query decode launch: %s", hipGetErrorString(e));
  return TQ_OK;
}

}  // extern "C"

// C ABI of the RMM hot path: argument validation, workspace sizing and the
// launch sequence of every entry point.  Nothing here allocates device
// memory, synchronises or reads device data back; every entry point enqueues
// on the caller's stream and returns.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

#define RMM_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[256] = "";

rmm_status_t fail(rmm_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
rmm_status_t fail(rmm_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

rmm_status_t ok() {
  g_last_error[0] = '\0';
  return RMM_OK;
}

rmm_status_t hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(RMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t esize(rmm_dtype_t dt) { return dt == RMM_BF16 ? 2 : 4; }
bool dtype_ok(rmm_dtype_t dt) { return dt == RMM_BF16 || dt == RMM_F32; }
bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kMaxDim = (int64_t)1 << 31;  // indices are int32

inline size_t align256(size_t x) { return rmm::align_up(x, 256); }

// Workspace carving: successive 256-byte aligned regions.
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *p) : base(static_cast<char *>(p)) {}
  void *take(size_t bytes) {
    void *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  }
};


rmm::ColnormPlan plan_for(rmm_dtype_t dt, const void *A, int64_t m, int64_t d, int64_t lda,
                          int64_t batch, int64_t bs, bool causal = false) {
  const int64_t v = 16 / (int64_t)esize(dt);
  const bool vec = aligned(A, 16) && lda % v == 0 && (batch == 1 || bs % v == 0);
  return rmm::colnorm_plan(dt, m, d, batch, vec, causal);
}

// Worst case over alignments and the causal / full plans (they may differ in
// chunk count): the largest of the four.
size_t colnorm_ws(rmm_dtype_t dt, int64_t m, int64_t d, int64_t batch) {
  size_t best = 0;
  for (int v = 0; v < 2; ++v)
    for (int c = 0; c < 2; ++c) {
      const size_t b = rmm::colnorm_ws_bytes(rmm::colnorm_plan(dt, m, d, batch, v != 0, c != 0), d, batch);
      if (b > best) best = b;
    }
  return best;
}

}  // namespace

rmm_status_t rmm::set_error(rmm_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

// ------------------------------------------------------------------ misc
RMM_API int rmm_version(void) { return 100; }

RMM_API const char *rmm_status_string(int s) {
  switch (s) {
    case RMM_OK: return "RMM_OK";
    case RMM_ERR_INVALID_ARG: return "RMM_ERR_INVALID_ARG";
    case RMM_ERR_UNSUPPORTED: return "RMM_ERR_UNSUPPORTED";
    case RMM_ERR_WORKSPACE: return "RMM_ERR_WORKSPACE";
    case RMM_ERR_HIP: return "RMM_ERR_HIP";
    default: return "RMM_ERR_UNKNOWN";
  }
}

RMM_API const char *rmm_last_error(void) { return g_last_error; }

// rho as the decimal the caller wrote: the shortest decimal string that reads
// back as the same double, mantissa digits p and exponent q (rho = p * 10^-q),
// among equally short strings the one nearest rho.  Returns false only if no
// string of at most 17 significant digits round-trips (cannot happen for a
// finite double).
static bool shortest_decimal(double rho, uint64_t *p_out, int *q_out) {
  for (int prec = 0; prec <= 16; ++prec) {
    char buf[64];
    snprintf(buf, sizeof(buf), "%.*e", prec, rho);
    // digits before 'e' (any decimal separator skipped), then the exponent
    uint64_t mant = 0;
    int ndig = 0;
    const char *c = buf;
    for (; *c && *c != 'e' && *c != 'E'; ++c)
      if (*c >= '0' && *c <= '9') {
        mant = mant * 10 + (uint64_t)(*c - '0');
        ++ndig;
      }
    if (*c != 'e' && *c != 'E') return false;
    const int e10 = atoi(c + 1);
    // rho = mant * 10^(e10 - (ndig - 1)).  The nearest string of this length
    // (the correctly rounded one) is tried first; when it does not read back
    // (rho a power of two, whose rounding interval is lopsided), the one
    // neighbour on the far side of rho may.  No other string of this length
    // can: the rounding interval is contiguous and holds rho.
    const int q = (ndig - 1) - e10;
    uint64_t best = 0;
    const uint64_t cands[3] = {mant, mant - 1, mant + 1};
    for (int ci = 0; ci < 3 && best == 0; ++ci) {
      if (cands[ci] == 0) continue;
      char tb[64];
      snprintf(tb, sizeof(tb), "%llue%d", (unsigned long long)cands[ci], -q);
      if (strtod(tb, nullptr) == rho) best = cands[ci];
    }
    if (best != 0) {
      // strip trailing zeros so that p and q are in lowest decimal form
      int qq = q;
      while (best % 10 == 0 && best != 0) {
        best /= 10;
        --qq;
      }
      *p_out = best;
      *q_out = qq;
      return true;
    }
  }
  return false;
}

RMM_API rmm_status_t rmm_k_from_rho(double rho, int64_t d, int64_t *k) {
  if (!k) return fail(RMM_ERR_INVALID_ARG, "k_from_rho: k is NULL");
  if (!(rho > 0.0 && rho <= 1.0)) return fail(RMM_ERR_INVALID_ARG, "k_from_rho: rho must lie in (0, 1]");
  if (d < 1 || d >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "k_from_rho: d out of range");
  // k = ceil(p * d / 10^q), exact in 128-bit integers: p < 10^17 and d < 2^31,
  // so p * d < 10^27; for q >= 27 the quotient lies in (0, 1) and k = 1.
  uint64_t p = 0;
  int q = 0;
  if (!shortest_decimal(rho, &p, &q)) return fail(RMM_ERR_INVALID_ARG, "k_from_rho: rho has no decimal form");
  const unsigned __int128 num = (unsigned __int128)p * (unsigned __int128)(uint64_t)d;
  int64_t kk;
  if (q <= 0) {
    // rho = p * 10^|q| <= 1 means p = 1, q = 0
    unsigned __int128 v = num;
    for (int i = 0; i < -q; ++i) v *= 10;
    kk = v > (unsigned __int128)d ? d : (int64_t)v;
  } else if (q >= 27) {
    kk = 1;
  } else {
    unsigned __int128 den = 1;
    for (int i = 0; i < q; ++i) den *= 10;
    kk = (int64_t)((num + den - 1) / den);
  }
  if (kk < 1) kk = 1;
  if (kk > d) kk = d;
  *k = kk;
  return ok();
}

RMM_API int64_t rmm_k_pad(int64_t k) {
  if (k < 1) return 0;
  return rmm::ceil_div(k, rmm::kKTile) * rmm::kKTile;
}

// ------------------------------------------------------------------ colnorm
RMM_API size_t rmm_colnorm_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t d, int64_t batch) {
  if (!dtype_ok(dt) || m < 1 || d < 1 || batch < 1) return 0;
  return colnorm_ws(dt, m, d, batch);
}

static rmm_status_t check_colnorm(rmm_dtype_t dt, const void *A, int64_t m, int64_t d,
                                  int64_t lda, int64_t batch, int64_t bs, const float *scores) {
  if (!dtype_ok(dt)) return fail(RMM_ERR_INVALID_ARG, "colnorm: unknown dtype");
  if (!A || !scores) return fail(RMM_ERR_INVALID_ARG, "colnorm: NULL pointer");
  if (m < 1 || d < 1 || d >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "colnorm: need m >= 1 and 1 <= d < 2^31");
  if (lda < d) return fail(RMM_ERR_INVALID_ARG, "colnorm: lda < d");
  if (batch < 1 || batch > kMaxBatch) return fail(RMM_ERR_INVALID_ARG, "colnorm: batch out of [1, 65535]");
  if (batch > 1 && bs < 0) return fail(RMM_ERR_INVALID_ARG, "colnorm: negative batch stride");
  if (!aligned(A, esize(dt)) || !aligned(scores, 4)) return fail(RMM_ERR_INVALID_ARG, "colnorm: misaligned pointer");
  return RMM_OK;
}

RMM_API rmm_status_t rmm_colnorm(rmm_dtype_t dt, const void *A, int64_t m, int64_t d, int64_t lda,
                                 int64_t batch, int64_t bs, float *scores, void *ws,
                                 size_t ws_bytes, rmm_stream_t stream) {
  rmm_status_t s = check_colnorm(dt, A, m, d, lda, batch, bs, scores);
  if (s != RMM_OK) return s;
  const rmm::ColnormPlan p = plan_for(dt, A, m, d, lda, batch, bs);
  const size_t need = rmm::colnorm_ws_bytes(p, d, batch);
  if (need > ws_bytes || (need && !ws)) return fail(RMM_ERR_WORKSPACE, "colnorm: workspace needs %zu bytes", need);
  // A matrix larger than the memory-side cache is streamed with
  // non-temporal loads (faster); a smaller one is read through the caches so
  // that the gather of its kept columns that follows can hit them.
  const bool big = (double)m * (double)d * (double)esize(dt) * (double)batch > rmm::kStreamBytes;
  return hip_status(rmm::launch_colnorm(dt, A, m, d, lda, batch, batch > 1 ? bs : 0, scores, ws, p,
                                        (hipStream_t)stream, false, 0, big),
                    "colnorm launch");
}

// ------------------------------------------------------------------ top-k
RMM_API size_t rmm_topk_workspace_bytes(int64_t, int64_t) { return 0; }

RMM_API rmm_status_t rmm_topk(const float *scores, int64_t batch, int64_t d, int64_t k,
                              int32_t *idx, void *, size_t, rmm_stream_t stream) {
  if (!scores || !idx) return fail(RMM_ERR_INVALID_ARG, "topk: NULL pointer");
  if (batch < 1 || batch > kMaxBatch) return fail(RMM_ERR_INVALID_ARG, "topk: batch out of [1, 65535]");
  if (d < 1 || d >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "topk: d out of range");
  if (k < 1 || k > d) return fail(RMM_ERR_INVALID_ARG, "topk: need 1 <= k <= d");
  if (!aligned(scores, 4) || !aligned(idx, 4)) return fail(RMM_ERR_INVALID_ARG, "topk: misaligned pointer");
  return hip_status(rmm::launch_topk(scores, batch, d, k, rmm_k_pad(k), idx, (hipStream_t)stream),
                    "topk launch");
}

// ------------------------------------------------------------------ gemm
// Many-row bf16 products also keep a transposed copy of the kept weight rows.
// The persistent 256 x 256 NT kernel needs enough output tiles to occupy the
// chip; smaller outputs (e.g. 2048 x 2048) run on the 128 x 128 row-gather core.
constexpr int64_t kNtMinTiles = 192;
static bool gemm_uses_nt(rmm_dtype_t dt, int64_t m, int64_t n = -1) {
  if (dt != RMM_BF16 || m < 1024) return false;
  if (n < 0) return true;
  return ((m + 255) / 256) * ((n + 255) / 256) >= kNtMinTiles;
}

RMM_API size_t rmm_gemm_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t n, int64_t k) {
  if (!dtype_ok(dt) || m < 1 || k < 1 || n < 1) return 0;
  const int64_t k_pad = rmm_k_pad(k);
  size_t b = align256((size_t)m * (size_t)k_pad * esize(dt)) + align256((size_t)k_pad * 4);
  if (gemm_uses_nt(dt, m, n)) b += rmm::gemm_nt_bt_bytes(n, k_pad);
  if (dt == RMM_BF16 && m <= 32) b += align256(rmm::skinny_part_bytes(false, m, n, k_pad));
  return b;
}

// The reduced product, and optionally the column scores of its output Y
// (y_scores != NULL; the extra workspace starts at offset `base`).
rmm_status_t rmm::gemm_args_check(const char *name, rmm_dtype_t dt, const void *A, int64_t lda, const void *B,
                                   int64_t ldb, const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k,
                                   const void *Y, int64_t ldy, const float *y_scores) {
  if (!dtype_ok(dt)) return fail(RMM_ERR_INVALID_ARG, "%s: unknown dtype", name);
  if (!A || !B || !idx || !Y) return fail(RMM_ERR_INVALID_ARG, "%s: NULL pointer", name);
  if (m < 1 || n < 1 || d < 1 || d >= kMaxDim || n >= kMaxDim)
    return fail(RMM_ERR_INVALID_ARG, "%s: bad m, n or d", name);
  if (k < 1 || k > d) return fail(RMM_ERR_INVALID_ARG, "%s: need 1 <= k <= d", name);
  if (lda < d || ldb < n || ldy < n) return fail(RMM_ERR_INVALID_ARG, "%s: leading dimension too small", name);
  const size_t e = esize(dt);
  if (!aligned(A, e) || !aligned(B, e) || !aligned(Y, e) || !aligned(idx, 4) || (y_scores && !aligned(y_scores, 4)))
    return fail(RMM_ERR_INVALID_ARG, "%s: misaligned pointer", name);
  return RMM_OK;
}

static rmm_status_t gemm_impl(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                              const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                              int64_t ldy, float *y_scores, void *ws, size_t ws_bytes, hipStream_t st) {
  const char *name = y_scores ? "gemm_scored" : "gemm";
  const rmm_status_t chk = rmm::gemm_args_check(name, dt, A, lda, B, ldb, idx, m, d, n, k, Y, ldy, y_scores);
  if (chk != RMM_OK) return chk;
  const size_t e = esize(dt);
  const size_t base = rmm_gemm_workspace_bytes(dt, m, n, k);
  const size_t need = y_scores ? rmm_gemm_scored_workspace_bytes(dt, m, n, k) : base;
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RMM_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned)", name, need);
  const int64_t k_pad = rmm_k_pad(k);
  char *w = static_cast<char *>(ws);
  int32_t *idx_clean = reinterpret_cast<int32_t *>(w + align256((size_t)m * k_pad * e));
  hipError_t he = rmm::launch_pack(dt, A, lda, 0, idx, 0, 1, m, d, k, k_pad, ws, idx_clean, st);
  if (he != hipSuccess) return hip_status(he, "gemm pack launch");
  if (gemm_uses_nt(dt, m, n) && rmm::gemm_nt_ok(m, n, d, ldb, k_pad)) {
    void *bt = w + align256((size_t)m * k_pad * e) + align256((size_t)k_pad * 4);
    return hip_status(rmm::launch_gemm_nt(ws, idx_clean, B, ldb, d, bt, Y, ldy, m, n, k_pad, st, y_scores,
                                          reinterpret_cast<float *>(w + base)),
                      "gemm launch");
  }
  if (dt == RMM_BF16 && rmm::skinny_ok(m, B, ldb, false, d, n)) {
    float *part = reinterpret_cast<float *>(w + align256((size_t)m * k_pad * e) + align256((size_t)k_pad * 4));
    he = rmm::launch_gemm_skinny(ws, idx_clean, B, false, nullptr, ldb, d, m, n, k_pad, Y, ldy, part, st);
  } else {
    rmm::GemmArgs g{};
    g.A = ws;
    g.idx = idx_clean;
    g.idx_stride = k_pad;
    g.B = B;
    g.ldb = ldb;
    g.b_batch_stride = 0;
    g.Y = Y;
    g.ldy = ldy;
    g.y_batch_stride = 0;
    g.batch = 1;
    g.hq = 1;
    g.hkv = 1;
    g.m = m;
    g.n = n;
    g.d = d;
    g.k = k;
    g.k_pad = k_pad;
    he = dt == RMM_BF16 ? rmm::launch_gemm_bf16(g, rmm::OutType::BF16, st) : rmm::launch_gemm_f32(g, st);
  }
  if (he != hipSuccess || !y_scores) return hip_status(he, "gemm launch");
  // Other kernels: the column scores of the written Y in a separate pass.
  const rmm::ColnormPlan p = plan_for(dt, Y, m, n, ldy, 1, 0);
  return hip_status(rmm::launch_colnorm(dt, Y, m, n, ldy, 1, 0, y_scores, w + base, p, st),
                    "gemm scores launch");
}

RMM_API rmm_status_t rmm_gemm(rmm_dtype_t dt, const void *A, int64_t lda, const void *B,
                              int64_t ldb, const int32_t *idx, int64_t m, int64_t d, int64_t n,
                              int64_t k, void *Y, int64_t ldy, void *ws, size_t ws_bytes,
                              rmm_stream_t stream) {
  return gemm_impl(dt, A, lda, B, ldb, idx, m, d, n, k, Y, ldy, nullptr, ws, ws_bytes, (hipStream_t)stream);
}

RMM_API size_t rmm_gemm_scored_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t n, int64_t k) {
  const size_t base = rmm_gemm_workspace_bytes(dt, m, n, k);
  if (!base) return 0;
  const size_t extra = gemm_uses_nt(dt, m, n) ? rmm::gemm_nt_ypart_bytes(m, n) : colnorm_ws(dt, m, n, 1);
  return base + (extra > 0 ? extra : 256);
}

RMM_API rmm_status_t rmm_gemm_scored(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                                     const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                                     int64_t ldy, float *y_scores, void *ws, size_t ws_bytes, rmm_stream_t stream) {
  if (!y_scores) return fail(RMM_ERR_INVALID_ARG, "gemm_scored: y_scores is NULL");
  return gemm_impl(dt, A, lda, B, ldb, idx, m, d, n, k, Y, ldy, y_scores, ws, ws_bytes, (hipStream_t)stream);
}

// ------------------------------------------------------------------ int8 weights
// Workspace: packed A_I, cleaned indices, then for m <= 32 the partial sums of
// the few-row kernel, else the dequantized kept rows Bd [k_pad][n], an index
// list 0..k-1 over them and, for m >= 1024, the NT GEMM's B_I^T.
struct W8Layout {
  size_t a, idx, part, bd, iota, bt, total;
};
static W8Layout w8_layout(int64_t m, int64_t n, int64_t k) {
  const int64_t k_pad = rmm_k_pad(k);
  W8Layout L{};
  Carve c(nullptr);
  L.a = c.off;    c.take((size_t)m * k_pad * 2);
  L.idx = c.off;  c.take((size_t)k_pad * 4);
  if (m <= 32) {
    L.part = c.off; c.take(rmm::skinny_part_bytes(true, m, n, k_pad));
  } else {
    L.bd = c.off;   c.take((size_t)k_pad * n * 2);
    L.iota = c.off; c.take((size_t)k_pad * 4);
    if (gemm_uses_nt(RMM_BF16, m, n)) {
      L.bt = c.off;
      c.take(rmm::gemm_nt_bt_bytes(n, k_pad));
    }
  }
  L.total = c.off;
  return L;
}

RMM_API size_t rmm_gemm_w8_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || k < 1 || n < 1) return 0;
  return w8_layout(m, n, k).total;
}

RMM_API rmm_status_t rmm_gemm_w8(const void *A, int64_t lda, const void *Bq, int64_t ldb, const float *scale,
                                 const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                                 int64_t ldy, void *ws, size_t ws_bytes, rmm_stream_t stream) {
  if (!A || !Bq || !scale || !idx || !Y) return fail(RMM_ERR_INVALID_ARG, "gemm_w8: NULL pointer");
  if (m < 1 || n < 1 || d < 1 || d >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "gemm_w8: bad m, n or d");
  if (k < 1 || k > d) return fail(RMM_ERR_INVALID_ARG, "gemm_w8: need 1 <= k <= d");
  if (lda < d || ldb < n || ldy < n) return fail(RMM_ERR_INVALID_ARG, "gemm_w8: leading dimension too small");
  if (!aligned(A, 2) || !aligned(Y, 2) || !aligned(scale, 4) || !aligned(idx, 4))
    return fail(RMM_ERR_INVALID_ARG, "gemm_w8: misaligned pointer");
  if (m <= 32 && !rmm::skinny_ok(m, Bq, ldb, true, d, n))
    return fail(RMM_ERR_UNSUPPORTED, "gemm_w8: m <= 32 needs 16-byte aligned weight rows (Bq %% 16 == 0, ldb %% 16 == 0) "
                "spanning less than 4 GiB");
  const W8Layout L = w8_layout(m, n, k);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(RMM_ERR_WORKSPACE, "gemm_w8: workspace needs %zu bytes (256-byte aligned)", L.total);
  const int64_t k_pad = rmm_k_pad(k);
  hipStream_t st = (hipStream_t)stream;
  char *w = static_cast<char *>(ws);
  int32_t *idx_clean = reinterpret_cast<int32_t *>(w + L.idx);
  hipError_t he = rmm::launch_pack(RMM_BF16, A, lda, 0, idx, 0, 1, m, d, k, k_pad, w + L.a, idx_clean, st);
  if (he != hipSuccess) return hip_status(he, "gemm_w8 pack launch");
  if (m <= 32)
    return hip_status(rmm::launch_gemm_skinny(w + L.a, idx_clean, Bq, true, scale, ldb, d, m, n, k_pad, Y, ldy,
                                              reinterpret_cast<float *>(w + L.part), st),
                      "gemm_w8 launch");
  // Many rows: the product is bound by MFMA, not by the weight bytes, so the
  // kept rows are dequantized once and multiplied by the bf16 path.
  he = rmm::launch_w8_dequant_rows(Bq, ldb, scale, idx_clean, k_pad, n, w + L.bd, st);
  if (he != hipSuccess) return hip_status(he, "gemm_w8 dequant launch");
  int32_t *iota = reinterpret_cast<int32_t *>(w + L.iota);
  he = rmm::launch_topk(nullptr, 1, k, k, k_pad, iota, st);   // k == d: 0..k-1, then -1
  if (he != hipSuccess) return hip_status(he, "gemm_w8 index launch");
  if (gemm_uses_nt(RMM_BF16, m, n) && rmm::gemm_nt_ok(m, n, k_pad, n, k_pad))
    return hip_status(rmm::launch_gemm_nt(w + L.a, iota, w + L.bd, n, k_pad, w + L.bt, Y, ldy, m, n, k_pad, st),
                      "gemm_w8 launch");
  rmm::GemmArgs g{};
  g.A = w + L.a;
  g.idx = iota;
  g.idx_stride = k_pad;
  g.B = w + L.bd;
  g.ldb = n;
  g.Y = Y;
  g.ldy = ldy;
  g.batch = 1;
  g.hq = 1;
  g.hkv = 1;
  g.m = m;
  g.n = n;
  g.d = k_pad;
  g.k = k;
  g.k_pad = k_pad;
  return hip_status(rmm::launch_gemm_bf16(g, rmm::OutType::BF16, st), "gemm_w8 launch");
}

// ------------------------------------------------------------------ producer-fused scores
RMM_API size_t rmm_swiglu_scored_workspace_bytes(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return align256(rmm::swiglu_part_bytes(m, n));
}

RMM_API rmm_status_t rmm_swiglu_scored(const void *G, int64_t ldg, const void *U, int64_t ldu, int64_t m, int64_t n,
                                       void *H, int64_t ldh, float *scores, void *ws, size_t ws_bytes,
                                       rmm_stream_t stream) {
  if (!G || !U || !H || !scores) return fail(RMM_ERR_INVALID_ARG, "swiglu_scored: NULL pointer");
  if (m < 1 || n < 1 || n >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "swiglu_scored: bad m or n");
  if (ldg < n || ldu < n || ldh < n) return fail(RMM_ERR_INVALID_ARG, "swiglu_scored: leading dimension too small");
  if (!aligned(scores, 4)) return fail(RMM_ERR_INVALID_ARG, "swiglu_scored: misaligned pointer");
  if (!rmm::swiglu_ok(G, ldg, U, ldu, H, ldh, n))
    return fail(RMM_ERR_UNSUPPORTED, "swiglu_scored: needs 16-byte aligned rows (pointers, leading dimensions and n multiples of 8 elements)");
  const size_t need = rmm_swiglu_scored_workspace_bytes(m, n);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(RMM_ERR_WORKSPACE, "swiglu_scored: workspace needs %zu bytes (256-byte aligned)", need);
  return hip_status(rmm::launch_swiglu_scored(G, ldg, U, ldu, m, n, H, ldh, scores, static_cast<float *>(ws),
                                              (hipStream_t)stream),
                    "swiglu_scored launch");
}

RMM_API size_t rmm_rmsnorm_scored_workspace_bytes(int64_t m, int64_t d) {
  if (m < 1 || d < 1) return 0;
  return align256(rmm::rmsnorm_part_bytes(m, d));
}

RMM_API rmm_status_t rmm_rmsnorm_scored(const void *X, int64_t ldx, const void *w, float eps, int64_t m, int64_t d,
                                        void *Y, int64_t ldy, float *scores, void *ws, size_t ws_bytes,
                                        rmm_stream_t stream) {
  if (!X || !w || !Y || !scores) return fail(RMM_ERR_INVALID_ARG, "rmsnorm_scored: NULL pointer");
  if (m < 1 || d < 1 || d >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "rmsnorm_scored: bad m or d");
  if (!(eps >= 0.f) || eps > 3.0e38f) return fail(RMM_ERR_INVALID_ARG, "rmsnorm_scored: eps must be finite and >= 0");
  if (ldx < d || ldy < d) return fail(RMM_ERR_INVALID_ARG, "rmsnorm_scored: leading dimension too small");
  if (!aligned(scores, 4)) return fail(RMM_ERR_INVALID_ARG, "rmsnorm_scored: misaligned pointer");
  if (!rmm::rmsnorm_ok(X, ldx, w, Y, ldy, d))
    return fail(RMM_ERR_UNSUPPORTED,
                "rmsnorm_scored: needs d a multiple of 512 up to 8192 and 16-byte aligned rows and weight");
  const size_t need = rmm_rmsnorm_scored_workspace_bytes(m, d);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(RMM_ERR_WORKSPACE, "rmsnorm_scored: workspace needs %zu bytes (256-byte aligned)", need);
  return hip_status(rmm::launch_rmsnorm_scored(X, ldx, w, eps, m, d, Y, ldy, scores, static_cast<float *>(ws),
                                               (hipStream_t)stream),
                    "rmsnorm_scored launch");
}

// ------------------------------------------------------------------ attention
static size_t qk_layout(int64_t Lq, int64_t Hq, int64_t dh, int64_t k, size_t *o_scores,
                        size_t *o_part, size_t *o_pack, size_t *o_idx) {
  Carve c(nullptr);
  *o_scores = c.off;
  c.take((size_t)Hq * dh * 4);
  *o_part = c.off;
  c.take(colnorm_ws(RMM_BF16, Lq, dh, Hq));
  *o_pack = c.off;
  c.take((size_t)Hq * Lq * rmm_k_pad(k) * 2);
  *o_idx = c.off;
  c.take((size_t)Hq * rmm_k_pad(k) * 4);
  return c.off;
}

RMM_API size_t rmm_qk_workspace_bytes(int64_t Lq, int64_t Hq, int64_t dh, int64_t k) {
  if (Lq < 1 || Hq < 1 || dh < 1 || k < 1) return 0;
  size_t a, b, c, e;
  return qk_layout(Lq, Hq, dh, k, &a, &b, &c, &e);
}

RMM_API rmm_status_t rmm_qk(const void *Q, int64_t Lq, int64_t Hq, int64_t dh, int64_t q_tok_stride,
                            int64_t q_head_stride, const void *Kt, int64_t Lk, int64_t Hkv,
                            int64_t kt_head_stride, int64_t ldkt, int64_t k, int causal, float *S,
                            int64_t s_head_stride, int64_t lds, int32_t *idx, float *feat_scores,
                            void *ws, size_t ws_bytes, rmm_stream_t stream) {
  if (!Q || !Kt || !S || !idx) return fail(RMM_ERR_INVALID_ARG, "qk: NULL pointer");
  if (Lq < 1 || Lk < 1 || dh < 1 || Lk >= kMaxDim || dh >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "qk: bad Lq, Lk or dh");
  if (Hq < 1 || Hq > kMaxBatch || Hkv < 1 || Hkv > Hq || Hq % Hkv != 0)
    return fail(RMM_ERR_INVALID_ARG, "qk: need 1 <= Hkv <= Hq <= 65535 and Hq %% Hkv == 0");
  if (k < 1 || k > dh) return fail(RMM_ERR_INVALID_ARG, "qk: need 1 <= k <= dh");
  if (q_tok_stride < 0 || q_head_stride < 0 || kt_head_stride < 0 || s_head_stride < 0)
    return fail(RMM_ERR_INVALID_ARG, "qk: negative stride");
  if (ldkt < Lk || lds < Lk || q_tok_stride < dh) return fail(RMM_ERR_INVALID_ARG, "qk: leading dimension too small");
  if (!aligned(Q, 2) || !aligned(Kt, 2) || !aligned(S, 4) || !aligned(idx, 4) ||
      (feat_scores && !aligned(feat_scores, 4)))
    return fail(RMM_ERR_INVALID_ARG, "qk: misaligned pointer");
  const int64_t k_pad = rmm_k_pad(k);
  if (!rmm::qk_layout_ok(Lq, dh, ldkt, Lk, k_pad))
    return fail(RMM_ERR_UNSUPPORTED, "qk: the rows of one key head exceed 4 GiB");
  if (!rmm::qk_tiles_ok(Lq, Lk, causal != 0))
    return fail(RMM_ERR_UNSUPPORTED, "qk: the tile list of Lq = %lld, Lk = %lld is not served",
                (long long)Lq, (long long)Lk);
  size_t o_sc, o_part, o_pack, o_idx;
  const size_t need = qk_layout(Lq, Hq, dh, k, &o_sc, &o_part, &o_pack, &o_idx);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return fail(RMM_ERR_WORKSPACE, "qk: workspace needs %zu bytes (256-byte aligned)", need);
  char *w = static_cast<char *>(ws);
  float *scores = feat_scores ? feat_scores : reinterpret_cast<float *>(w + o_sc);
  hipStream_t st = (hipStream_t)stream;

  const rmm::ColnormPlan p = plan_for(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride);
  hipError_t he = rmm::launch_colnorm(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride, scores,
                                      w + o_part, p, st);
  if (he != hipSuccess) return hip_status(he, "qk colnorm launch");
  he = rmm::launch_topk(scores, Hq, dh, k, k_pad, idx, st);
  if (he != hipSuccess) return hip_status(he, "qk topk launch");
  int32_t *idx_clean = reinterpret_cast<int32_t *>(w + o_idx);
  he = rmm::launch_pack(RMM_BF16, Q, q_tok_stride, q_head_stride, idx, k_pad, Hq, Lq, dh, k, k_pad,
                        w + o_pack, idx_clean, st);
  if (he != hipSuccess) return hip_status(he, "qk pack launch");
  return hip_status(rmm::launch_qk(w + o_pack, idx_clean, Kt, kt_head_stride, ldkt, S, s_head_stride, lds, Hq,
                                   Hkv, Lq, Lk, dh, k_pad, causal != 0, st),
                    "qk gemm launch");
}

static size_t pv_layout(int64_t Hq, int64_t Lq, int64_t Lk, int64_t k, size_t *o_scores,
                        size_t *o_part, size_t *o_plan) {
  (void)k;
  Carve c(nullptr);
  *o_scores = c.off;
  c.take((size_t)Hq * Lk * 4);
  *o_part = c.off;
  c.take(colnorm_ws(RMM_BF16, Lq, Lk, Hq));
  *o_plan = c.off;
  c.take(rmm::pv_plan_bytes(Hq, Lk));
  return c.off;
}

RMM_API size_t rmm_pv_workspace_bytes(int64_t Hq, int64_t Lq, int64_t Lk, int64_t k) {
  if (Lq < 1 || Hq < 1 || Lk < 1 || k < 1) return 0;
  size_t a, b, c;
  return pv_layout(Hq, Lq, Lk, k, &a, &b, &c);
}

RMM_API rmm_status_t rmm_pv(const void *P, int64_t Hq, int64_t Lq, int64_t Lk, int64_t p_head_stride,
                            int64_t ldp, const void *V, int64_t Hkv, int64_t dh,
                            int64_t v_tok_stride, int64_t v_head_stride, int64_t k, int causal, void *O,
                            int64_t o_tok_stride, int64_t o_head_stride, int32_t *idx, float *tok_scores,
                            void *ws, size_t ws_bytes, rmm_stream_t stream) {
  if (!P || !V || !O || !idx) return fail(RMM_ERR_INVALID_ARG, "pv: NULL pointer");
  if (Lq < 1 || Lk < 1 || dh < 1 || Lk >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "pv: bad Lq, Lk or dh");
  if (Lk > rmm::pv_max_tokens()) return fail(RMM_ERR_UNSUPPORTED, "pv: Lk above %lld", (long long)rmm::pv_max_tokens());
  if (Hq < 1 || Hq > kMaxBatch || Hkv < 1 || Hkv > Hq || Hq % Hkv != 0)
    return fail(RMM_ERR_INVALID_ARG, "pv: need 1 <= Hkv <= Hq <= 65535 and Hq %% Hkv == 0");
  if (k < 1 || k > Lk) return fail(RMM_ERR_INVALID_ARG, "pv: need 1 <= k <= Lk");
  if (p_head_stride < 0 || v_tok_stride < 0 || v_head_stride < 0 || o_tok_stride < 0 || o_head_stride < 0)
    return fail(RMM_ERR_INVALID_ARG, "pv: negative stride");
  if (ldp < Lk) return fail(RMM_ERR_INVALID_ARG, "pv: ldp < Lk");
  if (!aligned(P, 2) || !aligned(V, 2) || !aligned(O, 2) || !aligned(idx, 4) ||
      (tok_scores && !aligned(tok_scores, 4)))
    return fail(RMM_ERR_INVALID_ARG, "pv: misaligned pointer");
  if (!rmm::pv_layout_ok(P, ldp, p_head_stride, V, v_tok_stride, v_head_stride, Lk, dh))
    return fail(RMM_ERR_UNSUPPORTED, "pv: a 256-row block of P or the rows of one V head exceed 4 GiB");
  size_t o_sc, o_part, o_plan;
  const size_t need = pv_layout(Hq, Lq, Lk, k, &o_sc, &o_part, &o_plan);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return fail(RMM_ERR_WORKSPACE, "pv: workspace needs %zu bytes (256-byte aligned)", need);
  char *w = static_cast<char *>(ws);
  float *scores = tok_scores ? tok_scores : reinterpret_cast<float *>(w + o_sc);
  hipStream_t st = (hipStream_t)stream;
  const int64_t k_pad = rmm_k_pad(k);

  const rmm::ColnormPlan p = plan_for(RMM_BF16, P, Lq, Lk, ldp, Hq, p_head_stride, causal != 0);
  hipError_t he = rmm::launch_colnorm(RMM_BF16, P, Lq, Lk, ldp, Hq, p_head_stride, scores, w + o_part, p, st,
                                      causal != 0, Lk - Lq, /*stream_loads=*/true);
  if (he != hipSuccess) return hip_status(he, "pv colnorm launch");
  he = rmm::launch_topk(scores, Hq, Lk, k, k_pad, idx, st);
  if (he != hipSuccess) return hip_status(he, "pv topk launch");
  he = rmm::launch_pv(P, ldp, p_head_stride, V, v_tok_stride, v_head_stride, O, o_tok_stride, o_head_stride,
                      idx, k_pad, k, Hq, Hkv, Lq, Lk, dh, causal != 0, w + o_plan, st);
  return hip_status(he, "pv gemm launch");
}

// ------------------------------------------------------------------ fused attention
struct AttnLayout {
  size_t sc, part, qi, idxf, ki, stats, tok, kj, vjt, opart, total;
};
static AttnLayout attn_layout(int64_t Lq, int64_t Lk, int64_t Hq, int64_t dh, int64_t kf, int64_t kt) {
  const size_t kfp = (size_t)rmm_k_pad(kf), ktp = (size_t)rmm_k_pad(kt);
  AttnLayout L;
  Carve c(nullptr);
  L.sc = c.off;   c.take((size_t)Hq * dh * 4);
  L.part = c.off; c.take(colnorm_ws(RMM_BF16, Lq, dh, Hq));
  L.qi = c.off;   c.take((size_t)Hq * Lq * kfp * 2);
  L.idxf = c.off; c.take((size_t)Hq * kfp * 4);
  L.ki = c.off;   c.take((size_t)Hq * Lk * kfp * 2);
  L.stats = c.off; c.take((size_t)2 * Hq * Lq * 4);
  L.tok = c.off;  c.take((size_t)Hq * Lk * 4);
  L.kj = c.off;   c.take((size_t)Hq * ktp * kfp * 2);
  L.vjt = c.off;  c.take((size_t)Hq * dh * ktp * 2);
  L.opart = c.off; c.take((size_t)((Lq + 255) / 256) * Hq * dh * 4);
  L.total = c.off;
  return L;
}

// Few queries (decode steps): the scores S of every key instead of packed
// operands.  Both layouts start at offset 0; the query returns the larger.
struct AttnDecLayout {
  size_t sc, part, S, pstat, nml, tok, opart, total;
};
static AttnDecLayout attn_dec_layout(int64_t Lq, int64_t Lk, int64_t Hq, int64_t dh, int64_t kt) {
  const rmm::AttnDecodeSizes z = rmm::attn_decode_sizes(Lq, Lk, Hq, kt);
  AttnDecLayout L;
  Carve c(nullptr);
  L.sc = c.off;    c.take((size_t)Hq * dh * 4);
  L.part = c.off;  c.take(colnorm_ws(RMM_BF16, Lq, dh, Hq));
  L.S = c.off;     c.take(z.s_bytes);
  L.pstat = c.off; c.take(z.pstat_bytes);
  L.nml = c.off;   c.take(z.nml_bytes);
  L.tok = c.off;   c.take((size_t)Hq * Lk * 4);
  L.opart = c.off; c.take(z.opart_bytes);
  L.total = c.off;
  return L;
}

RMM_API size_t rmm_attention_workspace_bytes(int64_t Lq, int64_t Lk, int64_t Hq, int64_t dh, int64_t k_feat,
                                             int64_t k_tok) {
  if (Lq < 1 || Lk < 1 || Hq < 1 || dh < 1 || k_feat < 1 || k_tok < 1) return 0;
  size_t t = attn_layout(Lq, Lk, Hq, dh, k_feat, k_tok).total;
  if (rmm::attn_decode_ok(Lq, dh)) {
    const size_t td = attn_dec_layout(Lq, Lk, Hq, dh, k_tok).total;
    if (td > t) t = td;
  }
  return t;
}

RMM_API rmm_status_t rmm_attention(const void *Q, int64_t Lq, int64_t Hq, int64_t dh, int64_t q_tok_stride,
                                   int64_t q_head_stride, const void *Kt, int64_t Lk, int64_t Hkv,
                                   int64_t kt_head_stride, int64_t ldkt, const void *V, int64_t v_tok_stride,
                                   int64_t v_head_stride, int64_t k_feat, int64_t k_tok, int causal, void *O,
                                   int64_t o_tok_stride, int64_t o_head_stride, int32_t *idx_feat,
                                   int32_t *idx_tok, float *tok_scores, float *o_scores, void *ws,
                                   size_t ws_bytes, rmm_stream_t stream) {
  if (!Q || !Kt || !V || !O || !idx_feat || !idx_tok) return fail(RMM_ERR_INVALID_ARG, "attention: NULL pointer");
  if (Lq < 1 || Lk < 1 || dh < 1 || Lk >= kMaxDim || Lq >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "attention: bad Lq, Lk or dh");
  if (Hq < 1 || Hq > kMaxBatch || Hkv < 1 || Hkv > Hq || Hq % Hkv != 0)
    return fail(RMM_ERR_INVALID_ARG, "attention: need 1 <= Hkv <= Hq <= 65535 and Hq %% Hkv == 0");
  if (k_feat < 1 || k_feat > dh) return fail(RMM_ERR_INVALID_ARG, "attention: need 1 <= k_feat <= dh");
  if (k_tok < 1 || k_tok > Lk) return fail(RMM_ERR_INVALID_ARG, "attention: need 1 <= k_tok <= Lk");
  if (causal && Lq > Lk) return fail(RMM_ERR_INVALID_ARG, "attention: causal needs Lq <= Lk");
  if (q_tok_stride < dh || ldkt < Lk || v_tok_stride < dh || o_tok_stride < dh || q_head_stride < 0 ||
      kt_head_stride < 0 || v_head_stride < 0 || o_head_stride < 0)
    return fail(RMM_ERR_INVALID_ARG, "attention: bad stride");
  if (!aligned(Q, 2) || !aligned(Kt, 2) || !aligned(V, 2) || !aligned(O, 2) || !aligned(idx_feat, 4) ||
      !aligned(idx_tok, 4) || (tok_scores && !aligned(tok_scores, 4)) || (o_scores && !aligned(o_scores, 4)))
    return fail(RMM_ERR_INVALID_ARG, "attention: misaligned pointer");
  const int64_t kfp = rmm_k_pad(k_feat), ktp = rmm_k_pad(k_tok);
  if (!rmm::attn_supported(dh, kfp)) return fail(RMM_ERR_UNSUPPORTED, "attention: needs dh == 128");
  if ((uint64_t)((dh - 1) * ldkt + Lk) * 2 >= rmm::mg::kMaxRecords ||
      (uint64_t)((Lk - 1) * v_tok_stride + dh) * 2 >= rmm::mg::kMaxRecords ||
      (uint64_t)Lk * kfp * 2 >= rmm::mg::kMaxRecords)
    return fail(RMM_ERR_UNSUPPORTED, "attention: a key or value head spans 4 GiB or more");
  const size_t need = rmm_attention_workspace_bytes(Lq, Lk, Hq, dh, k_feat, k_tok);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RMM_ERR_WORKSPACE, "attention: workspace needs %zu bytes (256-byte aligned)", need);
  char *w = static_cast<char *>(ws);
  hipStream_t st = (hipStream_t)stream;
  if (rmm::attn_decode_ok(Lq, dh) && aligned(V, 16) && v_tok_stride % 8 == 0 && v_head_stride % 8 == 0) {
    // a few queries after a long context: passes split over keys
    const AttnDecLayout D = attn_dec_layout(Lq, Lk, Hq, dh, k_tok);
    const bool fused_sel = rmm::attn_decode_select_fused(Lk);
    float *tokd = tok_scores ? tok_scores : fused_sel ? nullptr : reinterpret_cast<float *>(w + D.tok);
    hipError_t he;
    if (Lq == 1) {
      he = rmm::launch_dec_feat1(Q, 0, q_head_stride, 1, Hq, k_feat, kfp, idx_feat, st);
      if (he != hipSuccess) return hip_status(he, "attention feature selection launch");
    } else {
      const rmm::ColnormPlan p = plan_for(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride);
      he = rmm::launch_colnorm(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride,
                               reinterpret_cast<float *>(w + D.sc), w + D.part, p, st);
      if (he != hipSuccess) return hip_status(he, "attention colnorm launch");
      he = rmm::launch_topk(reinterpret_cast<float *>(w + D.sc), Hq, dh, k_feat, kfp, idx_feat, st);
      if (he != hipSuccess) return hip_status(he, "attention topk launch");
    }
    rmm::AttnDecodeDesc dd{};
    dd.Q = Q;
    dd.q_ts = q_tok_stride;
    dd.q_hs = q_head_stride;
    dd.Kt = Kt;
    dd.kt_hs = kt_head_stride;
    dd.ldkt = ldkt;
    dd.V = V;
    dd.v_ts = v_tok_stride;
    dd.v_hs = v_head_stride;
    dd.I = idx_feat;
    dd.J = idx_tok;
    dd.S = reinterpret_cast<float *>(w + D.S);
    dd.pstat = reinterpret_cast<float *>(w + D.pstat);
    dd.nml = reinterpret_cast<float *>(w + D.nml);
    dd.tok = tokd;
    dd.opart = reinterpret_cast<float *>(w + D.opart);
    dd.O = O;
    dd.o_ts = o_tok_stride;
    dd.o_hs = o_head_stride;
    dd.o_scores = o_scores;
    dd.hq = Hq;
    dd.hkv = Hkv;
    dd.Lq = Lq;
    dd.Lk = Lk;
    dd.kf = k_feat;
    dd.kf_pad = kfp;
    dd.kt = k_tok;
    dd.kt_pad = ktp;
    dd.causal = causal != 0;
    he = rmm::launch_attn_decode(0, dd, st);
    if (he != hipSuccess) return hip_status(he, "attention scores launch");
    if (fused_sel) {
      he = rmm::launch_attn_decode(4, dd, st);
      if (he != hipSuccess) return hip_status(he, "attention token selection launch");
    } else {
      he = rmm::launch_attn_decode(1, dd, st);
      if (he != hipSuccess) return hip_status(he, "attention token scores launch");
      he = rmm::launch_topk(tokd, Hq, Lk, k_tok, ktp, idx_tok, st);
      if (he != hipSuccess) return hip_status(he, "attention token topk launch");
    }
    he = rmm::launch_attn_decode(2, dd, st);
    if (he != hipSuccess) return hip_status(he, "attention output launch");
    return hip_status(rmm::launch_attn_decode(3, dd, st), "attention output merge launch");
  }
  const AttnLayout L = attn_layout(Lq, Lk, Hq, dh, k_feat, k_tok);
  float *tok = tok_scores ? tok_scores : reinterpret_cast<float *>(w + L.tok);
  int32_t *idx_clean = reinterpret_cast<int32_t *>(w + L.idxf);

  // feature selection and the packed Q[:, I] (as rmm_qk)
  const rmm::ColnormPlan p = plan_for(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride);
  hipError_t he = rmm::launch_colnorm(RMM_BF16, Q, Lq, dh, q_tok_stride, Hq, q_head_stride,
                                      reinterpret_cast<float *>(w + L.sc), w + L.part, p, st);
  if (he != hipSuccess) return hip_status(he, "attention colnorm launch");
  he = rmm::launch_topk(reinterpret_cast<float *>(w + L.sc), Hq, dh, k_feat, kfp, idx_feat, st);
  if (he != hipSuccess) return hip_status(he, "attention topk launch");
  he = rmm::launch_pack(RMM_BF16, Q, q_tok_stride, q_head_stride, idx_feat, kfp, Hq, Lq, dh, k_feat, kfp,
                        w + L.qi, idx_clean, st);
  if (he != hipSuccess) return hip_status(he, "attention pack launch");
  {
    // K[:, I] per query head: K_I[h][u][f] = Kt_g[I_h[f]][u]
    rmm::KernelTimer timer("attn_kpack", st);
    he = rmm::launch_bt_pack(Kt, ldkt, dh, Lk, idx_clean, kfp, w + L.ki, Hq, Hq, Hkv, kt_head_stride, kfp,
                             Lk * kfp, st);
    if (he != hipSuccess) return hip_status(he, "attention key pack launch");
  }
  rmm::AttnDesc d{};
  d.QI = w + L.qi;
  d.KI = w + L.ki;
  d.KJ = w + L.kj;
  d.VJT = w + L.vjt;
  d.J = idx_tok;
  {
    float *st2 = reinterpret_cast<float *>(w + L.stats);
    d.nml = st2;
    d.n2ml = st2 + Hq * Lq;
  }
  d.tok = tok;
  d.opart = o_scores ? reinterpret_cast<float *>(w + L.opart) : nullptr;
  d.O = O;
  d.o_ts = o_tok_stride;
  d.o_hs = o_head_stride;
  d.hq = Hq;
  d.Lq = Lq;
  d.Lk = Lk;
  d.dh = dh;
  d.kf_pad = kfp;
  d.kt = k_tok;
  d.kt_pad = ktp;
  d.causal = causal != 0;
  he = rmm::launch_attn_passes(0, d, st);
  if (he != hipSuccess) return hip_status(he, "attention row statistics launch");
  he = rmm::launch_attn_passes(1, d, st);
  if (he != hipSuccess) return hip_status(he, "attention token scores launch");
  he = rmm::launch_topk(tok, Hq, Lk, k_tok, ktp, idx_tok, st);
  if (he != hipSuccess) return hip_status(he, "attention token topk launch");
  he = rmm::launch_attn_passes(2, d, st);
  if (he != hipSuccess) return hip_status(he, "attention key gather launch");
  {
    // V_J^T[h][j][u] = V_g[J_h[u]][j]
    rmm::KernelTimer timer("attn_vpack", st);
    he = rmm::launch_bt_pack(V, v_tok_stride, Lk, dh, idx_tok, ktp, w + L.vjt, Hq, Hq, Hkv, v_head_stride, ktp,
                             dh * ktp, st);
    if (he != hipSuccess) return hip_status(he, "attention value pack launch");
  }
  he = rmm::launch_attn_passes(3, d, st);
  if (he != hipSuccess || !o_scores) return hip_status(he, "attention output launch");
  return hip_status(rmm::launch_colnorm_finish(d.opart, (Lq + 255) / 256, Hq * dh, o_scores, st),
                    "attention output scores launch");
}

// ------------------------------------------------------------------ batched decode attention
// One new token for each of nseq sequences, each over its own cache: the rows
// of the decode passes are the (sequence, head) pairs.
struct AttnBatchLayout {
  size_t sc, S, pstat, nml, tok, opart, total;
};
static AttnBatchLayout attn_batch_layout(int64_t nseq, int64_t Hq, int64_t Lmax, int64_t kt_max) {
  const int64_t rows = nseq * Hq;
  const rmm::AttnDecodeSizes z = rmm::attn_decode_sizes(1, Lmax, rows, kt_max);
  AttnBatchLayout L;
  Carve c(nullptr);
  L.sc = c.off;    c.take((size_t)rows * 128 * 4);
  L.S = c.off;     c.take(z.s_bytes);
  L.pstat = c.off; c.take(z.pstat_bytes);
  L.nml = c.off;   c.take(z.nml_bytes);
  L.tok = c.off;   c.take((size_t)rows * Lmax * 4);
  L.opart = c.off; c.take(z.opart_bytes);
  L.total = c.off;
  return L;
}

RMM_API size_t rmm_attention_decode_batch_workspace_bytes(int64_t nseq, int64_t Hq, int64_t dh, int64_t Lmax,
                                                          int64_t kt_max) {
  if (nseq < 1 || Hq < 1 || dh != 128 || Lmax < 1 || kt_max < 1) return 0;
  return attn_batch_layout(nseq, Hq, Lmax, kt_max).total;
}

RMM_API rmm_status_t rmm_attention_decode_batch(
    const void *Q, int64_t q_seq_stride, int64_t q_head_stride, const void *Kt, int64_t kt_seq_stride,
    int64_t kt_head_stride, int64_t ldkt, const void *V, int64_t v_seq_stride, int64_t v_tok_stride,
    int64_t v_head_stride, const int32_t *lens, const int32_t *k_tok, int64_t nseq, int64_t Hq, int64_t Hkv,
    int64_t dh, int64_t Lmax, int64_t k_feat, int64_t kt_max, void *O, int64_t o_seq_stride,
    int64_t o_head_stride, int32_t *idx_feat, int32_t *idx_tok, float *tok_scores, void *ws, size_t ws_bytes,
    rmm_stream_t stream) {
  if (!Q || !Kt || !V || !lens || !k_tok || !O || !idx_feat || !idx_tok)
    return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: NULL pointer");
  if (nseq < 1 || Lmax < 1 || Lmax >= kMaxDim) return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: bad nseq or Lmax");
  if (Hq < 1 || Hkv < 1 || Hkv > Hq || Hq % Hkv != 0 || nseq * Hq > kMaxBatch)
    return fail(RMM_ERR_INVALID_ARG,
                "attention_decode_batch: need 1 <= Hkv <= Hq, Hq %% Hkv == 0 and nseq * Hq <= 65535");
  if (dh != 128) return fail(RMM_ERR_UNSUPPORTED, "attention_decode_batch: needs dh == 128");
  if (k_feat < 1 || k_feat > dh) return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: need 1 <= k_feat <= dh");
  if (kt_max < 1 || kt_max > Lmax) return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: need 1 <= kt_max <= Lmax");
  if (q_head_stride < 0 || q_seq_stride < 0 || kt_head_stride < 0 || kt_seq_stride < 0 || ldkt < Lmax ||
      v_tok_stride < dh || v_head_stride < 0 || v_seq_stride < 0 || o_head_stride < 0 || o_seq_stride < 0)
    return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: bad stride");
  if (!aligned(Q, 2) || !aligned(Kt, 2) || !aligned(O, 2) || !aligned(lens, 4) || !aligned(k_tok, 4) ||
      !aligned(idx_feat, 4) || !aligned(idx_tok, 4) || (tok_scores && !aligned(tok_scores, 4)))
    return fail(RMM_ERR_INVALID_ARG, "attention_decode_batch: misaligned pointer");
  if (!aligned(V, 16) || v_tok_stride % 8 != 0 || v_head_stride % 8 != 0 || v_seq_stride % 8 != 0)
    return fail(RMM_ERR_UNSUPPORTED, "attention_decode_batch: value rows must be 16-byte aligned");
  const size_t need = rmm_attention_decode_batch_workspace_bytes(nseq, Hq, dh, Lmax, kt_max);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(RMM_ERR_WORKSPACE, "attention_decode_batch: workspace needs %zu bytes (256-byte aligned)", need);
  char *w = static_cast<char *>(ws);
  hipStream_t st = (hipStream_t)stream;
  const AttnBatchLayout D = attn_batch_layout(nseq, Hq, Lmax, kt_max);
  const int64_t kfp = rmm_k_pad(k_feat), ktp = rmm_k_pad(kt_max), rows = nseq * Hq;
  const bool fused_sel = rmm::attn_decode_select_fused(Lmax);
  float *tokd = tok_scores ? tok_scores : fused_sel ? nullptr : reinterpret_cast<float *>(w + D.tok);
  hipError_t he = rmm::launch_dec_feat1(Q, q_seq_stride, q_head_stride, nseq, Hq, k_feat, kfp, idx_feat, st);
  if (he != hipSuccess) return hip_status(he, "attention_decode_batch feature selection launch");
  rmm::AttnDecodeDesc dd{};
  dd.Q = Q;
  dd.q_ts = dh;
  dd.q_hs = q_head_stride;
  dd.Kt = Kt;
  dd.kt_hs = kt_head_stride;
  dd.ldkt = ldkt;
  dd.V = V;
  dd.v_ts = v_tok_stride;
  dd.v_hs = v_head_stride;
  dd.I = idx_feat;
  dd.J = idx_tok;
  dd.S = reinterpret_cast<float *>(w + D.S);
  dd.pstat = reinterpret_cast<float *>(w + D.pstat);
  dd.nml = reinterpret_cast<float *>(w + D.nml);
  dd.tok = tokd;
  dd.opart = reinterpret_cast<float *>(w + D.opart);
  dd.O = O;
  dd.o_ts = dh;
  dd.o_hs = o_head_stride;
  dd.o_scores = nullptr;
  dd.hq = Hq;
  dd.hkv = Hkv;
  dd.Lq = 1;
  dd.Lk = Lmax;
  dd.kf = k_feat;
  dd.kf_pad = kfp;
  dd.kt = kt_max;
  dd.kt_pad = ktp;
  dd.causal = true;   // the new token is the last position of its sequence
  dd.nseq = nseq;
  dd.q_ss = q_seq_stride;
  dd.kt_ss = kt_seq_stride;
  dd.v_ss = v_seq_stride;
  dd.o_ss = o_seq_stride;
  dd.lens = lens;
  dd.kts = k_tok;
  he = rmm::launch_attn_decode(0, dd, st);
  if (he != hipSuccess) return hip_status(he, "attention_decode_batch scores launch");
  if (fused_sel) {
    he = rmm::launch_attn_decode(4, dd, st);
    if (he != hipSuccess) return hip_status(he, "attention_decode_batch token selection launch");
  } else {
    he = rmm::launch_attn_decode(1, dd, st);
    if (he != hipSuccess) return hip_status(he, "attention_decode_batch token scores launch");
    he = rmm::launch_topk(tokd, rows, Lmax, kt_max, ktp, idx_tok, st, k_tok, (int)Hq, lens);
    if (he != hipSuccess) return hip_status(he, "attention_decode_batch token topk launch");
  }
  he = rmm::launch_attn_decode(2, dd, st);
  if (he != hipSuccess) return hip_status(he, "attention_decode_batch output launch");
  return hip_status(rmm::launch_attn_decode(3, dd, st), "attention_decode_batch output merge launch");
}

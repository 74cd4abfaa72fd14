// Internal declarations shared by the RMM kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmm.h"

namespace rmm {

// ---------------------------------------------------------------- bf16 helpers
// bf16 values travel as raw 16-bit words.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 with round to nearest even (NaN stays NaN): the hardware
// conversion, one v_cvt_pk_bf16_f32 per pair on gfx950.
typedef __bf16 rmm_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const rmm_bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

// Record a one-line failure message for rmm_last_error() on this thread and
// return s.
rmm_status_t set_error(rmm_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Host-side argument checks of the reduced product (everything but the
// workspace); records the failure and returns its status, else RMM_OK.
rmm_status_t gemm_args_check(const char *name, rmm_dtype_t dt, const void *A, int64_t lda, const void *B,
                             int64_t ldb, const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k,
                             const void *Y, int64_t ldy, const float *y_scores);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kKTile = 64;  // K tile of the reduced GEMM; index rows are padded to it
// Matrices above this size are streamed with non-temporal loads or stores
// (read once, or written for a consumer that cannot find them in the
// 256 MB memory-side cache anyway).
constexpr double kStreamBytes = 192.0 * 1024 * 1024;

// ------------------------------------------------------------------ colnorm
struct ColnormPlan {
  int vec;               // elements per lane load (8 bf16 / 4 f32 / 1 scalar)
  int tpr;               // lanes per row (power of two <= 64)
  int64_t col_tiles;     // ceil(d / (tpr*vec))
  int64_t rows_per_chunk;
  int64_t chunks;        // row chunks; partial sums per chunk when > 1
};
ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t m, int64_t d, int64_t batch, bool vec_ok,
                         bool causal = false);
size_t colnorm_ws_bytes(const ColnormPlan &p, int64_t d, int64_t batch);
// causal (bf16 only): entry (i, j) is zero and not read when j > i + coff.
// stream (bf16): non-temporal loads, for a matrix far larger than the caches.
hipError_t launch_colnorm(rmm_dtype_t dt, const void *A, int64_t m, int64_t d, int64_t lda,
                          int64_t batch, int64_t batch_stride, float *scores, void *ws,
                          const ColnormPlan &p, hipStream_t stream, bool causal = false,
                          int64_t coff = 0, bool stream_loads = false);

// scores[j] = sqrt(sum over c < chunks of part[c][j]) for j < n, chunks added in a fixed order.
hipError_t launch_colnorm_finish(const float *part, int64_t chunks, int64_t n, float *scores, hipStream_t stream);

// ------------------------------------------------------------------ producer-fused scores
// H = bf16(silu(G) * U) for bf16 G, U [m][n] and the column scores of H (its
// bf16 values).  Rows 16-byte aligned, n % 8 == 0.  part: swiglu_part_bytes.
bool swiglu_ok(const void *G, int64_t ldg, const void *U, int64_t ldu, const void *H, int64_t ldh, int64_t n);
size_t swiglu_part_bytes(int64_t m, int64_t n);
hipError_t launch_swiglu_scored(const void *G, int64_t ldg, const void *U, int64_t ldu, int64_t m, int64_t n,
                                void *H, int64_t ldh, float *scores, float *part, hipStream_t stream);

// Y = bf16(X * w / sqrt(mean(X^2 over the row) + eps)) for bf16 X [m][d], w [d],
// and the column scores of Y.  d = 512 c, c = 1 .. 16; rows 16-byte aligned.
bool rmsnorm_ok(const void *X, int64_t ldx, const void *w, const void *Y, int64_t ldy, int64_t d);
size_t rmsnorm_part_bytes(int64_t m, int64_t d);
hipError_t launch_rmsnorm_scored(const void *X, int64_t ldx, const void *w, float eps, int64_t m, int64_t d, void *Y,
                                 int64_t ldy, float *scores, float *part, hipStream_t stream);

// ------------------------------------------------------------------ top-k
// k_rows / len_rows (optional, device): per-row kept count and valid length of
// row b read at [b / k_div]; the count is clamped to [1, min(k, d, length)].
hipError_t launch_topk(const float *scores, int64_t batch, int64_t d, int64_t k, int64_t k_pad,
                       int32_t *idx, hipStream_t stream, const int32_t *k_rows = nullptr, int k_div = 1,
                       const int32_t *len_rows = nullptr);

// ------------------------------------------------------------------ pack
// out[b][i][t] = A[b][i][idx[b][t]] for t < k (0 when idx is out of [0,d)), 0 for k <= t < k_pad.
// idx_clean (optional) [batch][k_pad]: idx[b][t] when t < k and 0 <= idx < d, else -1.
hipError_t launch_pack(rmm_dtype_t dt, const void *A, int64_t lda, int64_t a_batch_stride,
                       const int32_t *idx, int64_t idx_batch_stride, int64_t batch, int64_t m,
                       int64_t d, int64_t k, int64_t k_pad, void *out, int32_t *idx_clean,
                       hipStream_t stream);

// ------------------------------------------------------------------ gathered GEMM
struct GemmArgs {
  const void *A;          // packed [batch][m][k_pad]
  const int32_t *idx;     // [batch][idx_stride]
  int64_t idx_stride;
  const void *B;          // rows gathered via idx: B + g*b_batch_stride + idx*ldb
  int64_t ldb, b_batch_stride;
  void *Y;                // Y + b*y_batch_stride + i*ldy + j
  int64_t ldy, y_batch_stride;
  int64_t batch, hq, hkv; // batch b reads B group floor(b*hkv/hq)
  int64_t m, n, d, k, k_pad;
};
enum class OutType { BF16, F32 };
hipError_t launch_gemm_bf16(const GemmArgs &a, OutType out, hipStream_t stream);
hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t stream);

// ------------------------------------------------------------------ GEMM for few rows (m <= 32)
// B bf16 (w8 false) or int8 with a float scale per column (w8 true); rows of B
// must be 16-byte aligned.  part: skinny_part_bytes of fp32 partial sums.
bool skinny_ok(int64_t m, const void *B, int64_t ldb, bool w8, int64_t d, int64_t n);
size_t skinny_part_bytes(bool w8, int64_t m, int64_t n, int64_t k_pad);
hipError_t launch_gemm_skinny(const void *A_packed, const int32_t *idx_clean, const void *B, bool w8,
                              const float *scale, int64_t ldb, int64_t d, int64_t m, int64_t n, int64_t k_pad,
                              void *Y, int64_t ldy, float *part, hipStream_t stream);
// Bd[t][c] = bf16(Bq[idx[t]][c] * scale[c]) for t < k_pad (zero where idx < 0); Bd is k_pad x n.
hipError_t launch_w8_dequant_rows(const void *Bq, int64_t ldb, const float *scale, const int32_t *idx_clean,
                                  int64_t k_pad, int64_t n, void *Bd, hipStream_t stream);

// ------------------------------------------------------------------ NT GEMM for many rows
size_t gemm_nt_bt_bytes(int64_t n, int64_t k_pad);
// BT[b][c][t] = B_g[idx[b][t]][c] for c < n, t < k_pad (zero where idx < 0), batch
// entry b reading group g = floor(b * hkv / hq) of B (group stride b_gs); B rows
// have ldb elements, d rows.  BT entries are n x k_pad apart (bt_bs).
hipError_t launch_bt_pack(const void *B, int64_t ldb, int64_t d, int64_t n, const int32_t *idx_clean,
                          int64_t k_pad, void *BT, int64_t batch, int64_t hq, int64_t hkv, int64_t b_gs,
                          int64_t idx_bs, int64_t bt_bs, hipStream_t stream);
bool gemm_nt_ok(int64_t m, int64_t n, int64_t d, int64_t ldb, int64_t k_pad);
// y_scores (optional) [n]: column scores of the bf16 Y, formed in the epilogue
// from per-slab partials in ypart (gemm_nt_ypart_bytes) and finished in order.
hipError_t launch_gemm_nt(const void *A_packed, const int32_t *idx_clean, const void *B, int64_t ldb,
                          int64_t d, void *BT_ws, void *Y, int64_t ldy, int64_t m, int64_t n,
                          int64_t k_pad, hipStream_t stream, float *y_scores = nullptr, float *ypart = nullptr);
size_t gemm_nt_ypart_bytes(int64_t m, int64_t n);

// ------------------------------------------------------------------ feature-reduced Q K^T
bool qk_layout_ok(int64_t Lq, int64_t dh, int64_t ldkt, int64_t Lk, int64_t k_pad);
// The closed-form tile list of the (causal) product agrees with its direct sum.
bool qk_tiles_ok(int64_t Lq, int64_t Lk, bool causal);
hipError_t launch_qk(const void *Apacked, const int32_t *idx_clean, const void *Kt, int64_t kt_hs,
                     int64_t ldkt, float *S, int64_t s_hs, int64_t lds, int64_t hq, int64_t hkv,
                     int64_t Lq, int64_t Lk, int64_t dh, int64_t k_pad, bool causal, hipStream_t stream);

// ------------------------------------------------------------------ token-reduced P V
int64_t pv_max_tokens();
bool pv_layout_ok(const void *P, int64_t ldp, int64_t p_hs, const void *V, int64_t v_ts, int64_t v_hs,
                  int64_t Lk, int64_t dh);
size_t pv_plan_bytes(int64_t hq, int64_t Lk);
hipError_t launch_pv(const void *P, int64_t ldp, int64_t p_hs, const void *V, int64_t v_ts,
                     int64_t v_hs, void *O, int64_t o_ts, int64_t o_hs, const int32_t *idx,
                     int64_t idx_stride, int64_t k, int64_t hq, int64_t hkv, int64_t Lq, int64_t Lk,
                     int64_t dh, bool causal, void *plan_ws, hipStream_t stream);

// ---------------------------------------------------------------- fused reduced attention
// Device buffers of one fused call (packed operands in the workspace).
struct AttnDesc {
  const void *QI, *KI;   // [hq][Lq][kf_pad], [hq][Lk][kf_pad] bf16
  void *KJ;              // [hq][kt_pad][kf_pad] bf16 (written by pass 2)
  const void *VJT;       // [hq][dh][kt_pad] bf16
  const int32_t *J;      // [hq][kt_pad]
  float *nml, *n2ml;     // [hq][Lq] -(row max of c S) - log2(row sum), and twice that
  float *tok;            // [hq][Lk]
  float *opart;          // [ceil(Lq/256)][hq][128] column sums of O^2 per 256-query block, or null
  void *O;               // bf16, [Lq tokens of o_ts] x [hq of o_hs] x dh
  int64_t o_ts, o_hs;
  int64_t hq, Lq, Lk, dh, kf_pad, kt, kt_pad;
  bool causal;
};
bool attn_supported(int64_t dh, int64_t kf_pad);
// pass 0: row statistics, 1: token scores, 2: gather of the kept K rows, 3: output
hipError_t launch_attn_passes(int pass, const AttnDesc &d, hipStream_t stream);

// ------------------------------------------------------------------ reduced attention, few queries
// Lq <= 16 new tokens after a longer context (decode steps), dh == 128; V rows
// 16-byte aligned.  Passes: 0 scores S (+ block statistics), 1 token scores,
// 2 partial outputs over kept tokens, 3 merged output (+ column scores of O).
struct AttnDecodeDesc {
  const void *Q;  int64_t q_ts, q_hs;     // bf16
  const void *Kt; int64_t kt_hs, ldkt;    // bf16, feature-major
  const void *V;  int64_t v_ts, v_hs;     // bf16
  const int32_t *I;                       // [hq][kf_pad] kept features
  int32_t *J;                             // [hq][kt_pad] kept tokens
  float *S, *pstat, *nml, *tok, *opart;   // workspace (attn_decode_sizes), tok [hq][Lk] (may be null for pass 4)
  void *O; int64_t o_ts, o_hs;            // bf16
  float *o_scores;                        // [hq][128] or null
  int64_t hq, hkv, Lq, Lk, kf, kf_pad, kt, kt_pad;
  bool causal;
  // batch of sequences (rows of I, J and the workspace arrays: nseq * hq);
  // Lk and kt are then the largest context and kept-token count
  int64_t nseq = 1;
  int64_t q_ss = 0, kt_ss = 0, v_ss = 0, o_ss = 0;   // sequence strides (elements)
  const int32_t *lens = nullptr;                     // [nseq] context lengths
  const int32_t *kts = nullptr;                      // [nseq] kept tokens
};
struct AttnDecodeSizes {
  int nblk, ntokblk, nsplit;   // score blocks, token-score blocks, output splits
  size_t s_bytes, pstat_bytes, nml_bytes, opart_bytes;
};
bool attn_decode_ok(int64_t Lq, int64_t dh);
AttnDecodeSizes attn_decode_sizes(int64_t Lq, int64_t Lk, int64_t Hq, int64_t kt);
// pass 0: scores and block statistics; 1: token scores (dec_tok); 4: token
// scores and token selection in one launch (needs attn_decode_select_fused);
// 2: output partials; 3: output merge.
hipError_t launch_attn_decode(int pass, const AttnDecodeDesc &d, hipStream_t stream);
bool attn_decode_select_fused(int64_t Lk);
// Feature selection of one new token per (sequence, head) row r = b * hq + h:
// the k_feat largest |Q[b][h][f]| of the 128 features, ties to the lower
// index, ascending in I[r][0, kf), then -1 up to kf_pad.
hipError_t launch_dec_feat1(const void *Q, int64_t q_ss, int64_t q_hs, int64_t nseq, int64_t hq, int64_t kf,
                            int64_t kf_pad, int32_t *I, hipStream_t stream);

}  // namespace rmm

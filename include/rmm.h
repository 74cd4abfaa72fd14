/*
 * rmm.h - C ABI of the Reduced Matrix Multiplication (RMM) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes comes from the pages titled "Reduced Matrix
 * Multiplication: Input-Adaptive Matrix-Product Reduction for LLM Inference"
 * (gist.science explainer, es/zh editions, section "Metodología" / "方法论";
 * arXiv:2608.13426 abstract):
 *   every Transformer product is Y = A B with A the activation and B a weight
 *   or intermediate; contraction index j is scored by s_j = ||A[:, j]||_2; the
 *   k = ceil(rho d) best-scored indices I are kept; A[:, I] B[I, :] replaces
 *   A B.  Sites: projections X W (hidden dim), Q K^T (head-feature dim) and
 *   P V (token dim).
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) must be device memory visible to the current
 *     HIP device; (host) pointers are ordinary host memory.
 *   - Element types: RMM_BF16 = IEEE bfloat16 stored as 16-bit words, RMM_F32 =
 *     IEEE binary32.  Every pointer must be aligned to its element size.
 *     Vectorised 16-byte paths are taken automatically when base addresses and
 *     strides allow; other layouts run a scalar path with identical results.
 *   - Strides and leading dimensions are counted in elements, not bytes.
 *   - All matrices are row-major: element (i, j) of a matrix with leading
 *     dimension ld lives at base[i * ld + j].
 *   - Ownership: the caller allocates and frees every buffer (inputs, outputs,
 *     index lists and workspace).  The library never allocates, frees, caches
 *     or synchronises; it enqueues kernels on `stream` and returns.  Buffers
 *     must stay alive until that stream work completes.  Outputs must not
 *     alias inputs or each other.
 *   - Workspace: `ws` (device) of at least the size returned by the matching
 *     *_workspace_bytes query (0 is allowed when the query returns 0).  The
 *     workspace holds no state between calls.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a rejected call enqueues nothing and returns
 *     RMM_ERR_INVALID_ARG / RMM_ERR_UNSUPPORTED / RMM_ERR_WORKSPACE.  A failed
 *     kernel launch returns RMM_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation, as usual for HIP.  No call aborts or
 *     prints; rmm_last_error() gives a one-line description of the last
 *     failure on the calling thread.
 *   - Determinism: every result is bitwise reproducible for fixed inputs and
 *     shapes (fixed-order reductions, no floating-point atomics).
 *   - Index lists: rmm_topk writes, for each batch row, the k kept indices in
 *     ascending order followed by -1 up to rmm_k_pad(k) entries, so a row of
 *     an index list is rmm_k_pad(k) int32 words long.
 */
#ifndef RMM_H_
#define RMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RMM_OK = 0,
  RMM_ERR_INVALID_ARG = 1, /* bad size, stride, pointer or ratio            */
  RMM_ERR_UNSUPPORTED = 2, /* valid request the library does not serve     */
  RMM_ERR_WORKSPACE = 3,   /* ws_bytes below the size the query returns     */
  RMM_ERR_HIP = 4          /* the HIP runtime rejected a launch             */
} rmm_status_t;

typedef enum { RMM_BF16 = 0, RMM_F32 = 1 } rmm_dtype_t;

/* A hipStream_t; NULL means the device's null stream. */
typedef void *rmm_stream_t;

/* Library version, as major*10000 + minor*100 + patch. */
int rmm_version(void);

/* Static string naming a status code. */
const char *rmm_status_string(int status);

/* One-line description of the last failure on the calling thread ("" if none). */
const char *rmm_last_error(void);

/*
 * rmm_k_from_rho - number of kept indices, k = ceil(rho * d).
 * Source: "Estrategia de Selección" (k = ceil(rho d), rho the retention ratio).
 * rho is read as the decimal the caller wrote: the shortest decimal string
 * that reads back as the same double (of equally short ones, the nearest),
 * p * 10^-q, and k = ceil(p * d / 10^q) in exact integer arithmetic.  So
 * rho = 0.55, d = 100 gives 55 (a naive binary product gives 56), and
 * rho = 0.1 + 0.2 (shortest string 0.30000000000000004), d = 10 gives 4.
 *   rho  in (0, 1]; d >= 1; k (host) receives the result, 1 <= k <= d.
 * Returns RMM_ERR_INVALID_ARG for rho outside (0, 1] (or NaN), d < 1 or k NULL.
 */
rmm_status_t rmm_k_from_rho(double rho, int64_t d, int64_t *k);

/* Length of one index-list row for k kept indices: k rounded up to a
 * multiple of 64 (the K tile of the reduced GEMM).  Returns 0 for k < 1. */
int64_t rmm_k_pad(int64_t k);

/*
 * rmm_colnorm - column scores s_j = ||A[:, j]||_2 over all m rows, for each of
 * `batch` matrices.  Source: "Estrategia de Selección" (s_j = ||A_{:,j}||_2).
 *   dt            RMM_BF16 or RMM_F32 element type of A.
 *   A (device)    batch matrices of m x d; matrix b starts at A + b*batch_stride,
 *                 row i of it at + i*lda.
 *   lda >= d; batch >= 1; batch_stride >= 0 (any value when batch == 1).
 *   scores (device, float) [batch][d], written.
 * Accumulation is float32 in a fixed blocked order (per-lane partial sums over
 * row subsets, combined by a fixed tree), then a correctly rounded sqrt.
 */
size_t rmm_colnorm_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t d, int64_t batch);
rmm_status_t rmm_colnorm(rmm_dtype_t dt, const void *A, int64_t m, int64_t d, int64_t lda,
                         int64_t batch, int64_t batch_stride, float *scores, void *ws,
                         size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_topk - the k largest scores of each batch row.  Source: "Estrategia de
 * Selección" (keep the top-k indices).  Ties at the k-th score go to the lower
 * index; the output is in ascending index order.
 *   scores (device, float) [batch][d].  Any finite values; -0.0 ranks as +0.0.
 *   1 <= k <= d.
 *   idx (device, int32) [batch][rmm_k_pad(k)]: row b receives its k indices
 *   ascending, then -1 in the remaining rmm_k_pad(k) - k slots.
 * Exact: the selection is a radix select on the float bit patterns, with no
 * rounding anywhere.
 */
size_t rmm_topk_workspace_bytes(int64_t batch, int64_t d);
rmm_status_t rmm_topk(const float *scores, int64_t batch, int64_t d, int64_t k, int32_t *idx,
                      void *ws, size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_gemm - the reduced product Y = A[:, I] B[I, :] for one projection.
 * Source: "Mecanismo Central" (compute A_{:,I} B_{I,:} in place of A B) and
 * "Alcance de Aplicación" (hidden dimension of X W).  No rescaling.
 *   dt           RMM_BF16 (float32 accumulation, bf16 output) or RMM_F32
 *                (float32 throughout).
 *   A (device)   m x d activation, leading dimension lda >= d.
 *   B (device)   d x n weight stored with the contraction index as rows
 *                (row t is B + t*ldb), ldb >= n.  B is only read: kept rows
 *                are streamed as they lie in memory.
 *   idx (device, int32) the kept indices; entries 0..k-1 are read (an index
 *                list row from rmm_topk, or any k indices).  Entries outside
 *                [0, d) contribute zero instead of being dereferenced.
 *   1 <= k <= d; m, n >= 1.
 *   Y (device)   m x n output of element type dt, leading dimension ldy >= n.
 *   ws           at least rmm_gemm_workspace_bytes(dt, m, n, k) bytes,
 *                256-byte aligned; holds the packed A[:, I] and a cleaned
 *                copy of the k indices.
 */
size_t rmm_gemm_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t n, int64_t k);
rmm_status_t rmm_gemm(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                      int64_t ldy, void *ws, size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_gemm_scored - rmm_gemm that also returns the column scores of its
 * output: y_scores[c] = ||Y[:, c]||_2 over the m rows of the values written
 * (bf16-rounded for RMM_BF16), float32 accumulation in a fixed order.
 * Source: "Estrategia de Selección" (a product's contraction index is scored
 * by the column norm of its activation; when Y is the activation of a later
 * reduced product, its producer scores it, so rmm_topk can follow without an
 * rmm_colnorm pass over Y).  For the many-row bf16 products the squares are
 * summed in the GEMM's epilogue from registers (one partial per 128-row slab,
 * then a fixed-order finish); other shapes score Y in a second pass.
 *   Arguments and results as rmm_gemm (Y bitwise equal to rmm_gemm's), plus
 *   y_scores (device, float) [n], not NULL.
 *   ws: at least rmm_gemm_scored_workspace_bytes(dt, m, n, k) bytes, 256-byte aligned.
 */
size_t rmm_gemm_scored_workspace_bytes(rmm_dtype_t dt, int64_t m, int64_t n, int64_t k);
rmm_status_t rmm_gemm_scored(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                             const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                             int64_t ldy, float *y_scores, void *ws, size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_gemm_noalloc - rmm_gemm with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * errors as rmm_gemm (bitwise equal outputs), but the scratch memory (the
 * packed A[:, I], the cleaned index copy, the transposed kept weight rows or
 * the few-row kernel's partial sums) lives in a fixed device array inside the
 * library, RMM_NOALLOC_SCRATCH_BYTES long, one per device, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *   A product whose rmm_gemm_workspace_bytes(dt, m, n, k) exceeds
 *   RMM_NOALLOC_SCRATCH_BYTES is rejected with RMM_ERR_UNSUPPORTED before
 *   anything is enqueued.
 *   Every call on one device shares that device's array: calls that overlap
 *   on one GPU (different streams or threads) race on it and must be
 *   serialised by the caller.  The first call on a device looks up the
 *   array's device address (a HIP symbol query, no allocation).
 */
#define RMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
rmm_status_t rmm_gemm_noalloc(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                              const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                              int64_t ldy, rmm_stream_t stream);

/*
 * rmm_gemm_w8 - the reduced product with INT8 weights: Y = A[:, I] (Bq[I, :] * scale),
 * scale applied per output column.  Source: "Mecanismo Central" (the reduced
 * product) with the compatibility with INT8 weights stated in the abstract;
 * selection still reads A only.
 *   A (device, bf16) m x d, leading dimension lda >= d.
 *   Bq (device, int8) d x n quantized weight, contraction index as rows,
 *                leading dimension ldb >= n; only read.
 *   scale (device, float) [n]: column c of the weight is Bq[:, c] * scale[c].
 *   idx (device, int32) the kept indices, as for rmm_gemm.
 *   Y (device, bf16) m x n, leading dimension ldy >= n.
 *   m <= 32 (decode batches): the kept int8 rows are read once, converted to
 *   bf16 exactly, multiplied with float32 accumulation, and the sum is scaled;
 *   this path needs 16-byte aligned weight rows (Bq and ldb multiples of 16)
 *   spanning less than 4 GiB, else RMM_ERR_UNSUPPORTED.  m > 32: the kept rows
 *   are dequantized once to bf16(q * scale) and multiplied by the bf16 path.
 *   ws: at least rmm_gemm_w8_workspace_bytes(m, n, k) bytes, 256-byte aligned.
 */
size_t rmm_gemm_w8_workspace_bytes(int64_t m, int64_t n, int64_t k);
rmm_status_t rmm_gemm_w8(const void *A, int64_t lda, const void *Bq, int64_t ldb, const float *scale,
                         const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                         int64_t ldy, void *ws, size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_swiglu_scored - the gated MLP activation with its column scores in one
 * pass: H = silu(G) * U elementwise (silu(x) = x / (1 + e^-x), float32
 * arithmetic, bf16 result) and scores[j] = ||H[:, j]||_2 over the m rows of the
 * bf16 values written, float32 accumulation in a fixed order.  Source:
 * "Estrategia de Selección" (scores are column norms of the activation, a
 * light vector operation): the producer of the down projection's input
 * scores it, so rmm_topk can follow without a separate rmm_colnorm pass.
 *   G, U (device, bf16) m x n gate and up projections, leading dimensions
 *                ldg, ldu >= n (e.g. two halves of one fused GEMM output).
 *   H (device, bf16) m x n output, leading dimension ldh >= n; may not alias G or U.
 *   scores (device, float) [n].
 *   Pointers and leading dimensions must give 16-byte aligned rows and n must
 *   be a multiple of 8, else RMM_ERR_UNSUPPORTED.
 *   ws: rmm_swiglu_scored_workspace_bytes(m, n) bytes (0: none), 256-byte aligned.
 */
size_t rmm_swiglu_scored_workspace_bytes(int64_t m, int64_t n);
rmm_status_t rmm_swiglu_scored(const void *G, int64_t ldg, const void *U, int64_t ldu, int64_t m, int64_t n,
                               void *H, int64_t ldh, float *scores, void *ws, size_t ws_bytes,
                               rmm_stream_t stream);

/*
 * rmm_rmsnorm_scored - RMS normalisation of each row with the column scores of
 * the result in one pass: Y[i][j] = X[i][j] * w[j] / sqrt(mean_j'(X[i][j']^2)
 * + eps) in float32 arithmetic, rounded to bf16, and scores[j] =
 * ||Y[:, j]||_2 over the m rows of the bf16 values written (float32
 * accumulation in a fixed order).  Source: "Estrategia de Selección" (the
 * score of an index is the norm of that column of A, computed beside the
 * product): in a LLaMA-style layer the normalised hidden state is the A of
 * the q, k, v, gate and up projections, so its producer scores it and
 * rmm_topk follows with no rmm_colnorm pass.
 *   X (device, bf16) m x d, leading dimension ldx >= d.
 *   w (device, bf16) [d] per-column gain.
 *   eps: finite, >= 0, added to the mean square (eps = 0 and an all-zero row
 *        give non-finite values in that row, as the formula does).
 *   Y (device, bf16) m x d output, leading dimension ldy >= d; may not alias X.
 *   scores (device, float) [d].
 *   d must be a multiple of 512 no larger than 8192 and X, w, Y rows 16-byte
 *   aligned (pointers and leading dimensions multiples of 8 elements), else
 *   RMM_ERR_UNSUPPORTED.
 *   ws: rmm_rmsnorm_scored_workspace_bytes(m, d) bytes (0: none), 256-byte aligned.
 */
size_t rmm_rmsnorm_scored_workspace_bytes(int64_t m, int64_t d);
rmm_status_t rmm_rmsnorm_scored(const void *X, int64_t ldx, const void *w, float eps, int64_t m, int64_t d,
                                void *Y, int64_t ldy, float *scores, void *ws, size_t ws_bytes,
                                rmm_stream_t stream);

/*
 * rmm_qk - feature-reduced attention scores for every query head (bf16 in,
 * float32 out).  Source: "Alcance de Aplicación" (reduce the feature dimension
 * of Q K^T).  For query head h with kv head g = floor(h*Hkv/Hq):
 *   s = column scores of Q_h over its Lq rows, I_h = top-k of s,
 *   S_h = Q_h[:, I_h] Kt_g[I_h, :]   (no softmax scale applied).
 *   Q (device, bf16)  element (t, h, j) at Q + t*q_tok_stride + h*q_head_stride + j.
 *   Kt (device, bf16) keys stored feature-major: element (g, j, u) at
 *                     Kt + g*kt_head_stride + j*ldkt + u, ldkt >= Lk.
 *   Hq >= 1, 1 <= Hkv <= Hq, Hq % Hkv == 0; 1 <= k <= dh.
 *   S (device, float) element (h, t, u) at S + h*s_head_stride + t*lds + u.
 *   idx (device, int32) [Hq][rmm_k_pad(k)], written as by rmm_topk.
 *   feat_scores (device, float, optional) [Hq][dh]: receives the column
 *   scores the selection used; NULL keeps them in the workspace.
 *   causal != 0: only the entries a causal softmax reads are promised, those
 *   with u <= t + (Lk - Lq).  S is written in 128 x 128 tiles; tiles lying
 *   wholly above that diagonal are not written at all (the memory keeps what
 *   it held), and tiles that cross it are written whole, so entries above the
 *   diagonal inside them hold the unmasked products.  causal == 0 writes all
 *   of S.  Q and K are only read.
 * Layouts the kernels cannot address (the feature rows of one key head
 * spanning 4 GiB or more) are rejected with RMM_ERR_UNSUPPORTED before
 * anything is enqueued, like every other rejection.
 */
size_t rmm_qk_workspace_bytes(int64_t Lq, int64_t Hq, int64_t dh, int64_t k);
rmm_status_t rmm_qk(const void *Q, int64_t Lq, int64_t Hq, int64_t dh, int64_t q_tok_stride,
                    int64_t q_head_stride, const void *Kt, int64_t Lk, int64_t Hkv,
                    int64_t kt_head_stride, int64_t ldkt, int64_t k, int causal, float *S,
                    int64_t s_head_stride, int64_t lds, int32_t *idx, float *feat_scores, void *ws,
                    size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_pv - token-reduced attention output for every query head (bf16).
 * Source: "Alcance de Aplicación" (optionally reduce the token dimension of
 * P V).  For query head h with kv head g = floor(h*Hkv/Hq):
 *   s = column scores of P_h over its Lq query rows, J_h = top-k tokens,
 *   O_h = P_h[:, J_h] V_g[J_h, :].
 *   causal != 0: P is a causal attention matrix: entries (t, u) with
 *   u > t + (Lk - Lq) are taken as zero, in the scores and the product
 *   alike.  Their values are never used (16-byte loads that straddle the
 *   diagonal may fetch them; they are discarded), and the tiles and row
 *   segments lying wholly above the diagonal are not read at all.
 *   causal == 0 reads all of P.
 *   P (device, bf16) element (h, t, u) at P + h*p_head_stride + t*ldp + u, ldp >= Lk.
 *   V (device, bf16) element (u, g, j) at V + u*v_tok_stride + g*v_head_stride + j.
 *   1 <= k <= Lk <= 524288 (RMM_ERR_UNSUPPORTED above).
 *   Layouts with 16-byte aligned rows (bases on 16-byte boundaries, strides
 *   multiples of 8) use 16-byte loads; others take a slower path with the
 *   same results.  256 rows of P (256*ldp elements) and the rows of one V
 *   head must each span less than 4 GiB (RMM_ERR_UNSUPPORTED otherwise).
 *   O (device, bf16) element (t, h, j) at O + t*o_tok_stride + h*o_head_stride + j.
 *   idx (device, int32) [Hq][rmm_k_pad(k)], written as by rmm_topk.
 *   tok_scores (device, float, optional) [Hq][Lk]: receives the token scores
 *   the selection used (column norms of P over the Lq rows, causal zeros
 *   included as zeros); NULL keeps them in the workspace.
 * The product reads P at 64-token tile granularity: tiles holding no kept
 * token are skipped, dropped tokens inside a kept tile are zeroed in both P
 * and V before the multiply, so the result equals the reduced product exactly
 * (float32 accumulation, bf16 output).
 */
size_t rmm_pv_workspace_bytes(int64_t Hq, int64_t Lq, int64_t Lk, int64_t k);
rmm_status_t rmm_pv(const void *P, int64_t Hq, int64_t Lq, int64_t Lk, int64_t p_head_stride,
                    int64_t ldp, const void *V, int64_t Hkv, int64_t dh, int64_t v_tok_stride,
                    int64_t v_head_stride, int64_t k, int causal, void *O, int64_t o_tok_stride,
                    int64_t o_head_stride, int32_t *idx, float *tok_scores, void *ws, size_t ws_bytes,
                    rmm_stream_t stream);

/*
 * rmm_attention - fused reduced attention of one layer (bf16 in and out):
 * the feature-reduced Q K^T, the softmax and the token-reduced P V without
 * writing the score or probability matrices.  Source: "Alcance de
 * Aplicación" (reduce the feature dimension of Q K^T and the token dimension
 * of P V) with "Estrategia de Selección" (scores are column norms).  For query
 * head h with kv head g = floor(h*Hkv/Hq):
 *   I_h = top-k_feat features of Q_h by column norm (as rmm_qk),
 *   S_h = Q_h[:, I_h] Kt_g[I_h, :],
 *   P_h = softmax of S_h / sqrt(dh) over each row, causal: key u is visible
 *         from query t when u <= t + (Lk - Lq); others are exact zeros,
 *   J_h = top-k_tok tokens by column norm of P_h (as rmm_pv, the scores taken
 *         from float32 probabilities),
 *   O_h = P_h[:, J_h] V_g[J_h, :]   (P rounded to bf16 as the MFMA operand,
 *         float32 accumulation, bf16 output).
 *   Q, Kt, V, O: layouts as in rmm_qk and rmm_pv.  dh must be 128 and
 *   1 <= k_feat <= 128, 1 <= k_tok <= Lk (RMM_ERR_UNSUPPORTED for other dh);
 *   causal != 0 needs Lq <= Lk (every query sees its diagonal key).
 *   idx_feat (device, int32) [Hq][rmm_k_pad(k_feat)], idx_tok [Hq][rmm_k_pad(k_tok)]:
 *   the selections, written as by rmm_topk.
 *   tok_scores (device, float, optional) [Hq][Lk]: the token scores; NULL keeps
 *   them in the workspace.
 *   o_scores (device, float, optional) [Hq][dh]: column scores of the bf16 O
 *   over the Lq tokens, o_scores[h][j] = ||O[:, h, j]||_2 - the selection
 *   scores of the projection that reads O as its [Lq][Hq*dh] input, formed
 *   while O is written (producer-fused scoring); NULL skips them.
 * S and P are recomputed tile by tile in three passes (row max and sum,
 * column sums of squares, output over the kept tokens); the workspace holds
 * the packed Q[:, I], K[:, I] and the kept keys and values
 * (rmm_attention_workspace_bytes).
 */
size_t rmm_attention_workspace_bytes(int64_t Lq, int64_t Lk, int64_t Hq, int64_t dh, int64_t k_feat,
                                     int64_t k_tok);
rmm_status_t rmm_attention(const void *Q, int64_t Lq, int64_t Hq, int64_t dh, int64_t q_tok_stride,
                           int64_t q_head_stride, const void *Kt, int64_t Lk, int64_t Hkv,
                           int64_t kt_head_stride, int64_t ldkt, const void *V, int64_t v_tok_stride,
                           int64_t v_head_stride, int64_t k_feat, int64_t k_tok, int causal, void *O,
                           int64_t o_tok_stride, int64_t o_head_stride, int32_t *idx_feat,
                           int32_t *idx_tok, float *tok_scores, float *o_scores, void *ws,
                           size_t ws_bytes, rmm_stream_t stream);

/*
 * rmm_attention_decode_batch - one decode step of nseq sequences, each with
 * its own KV cache: for every (sequence b, query head h) the reduced attention
 * of the sequence's one new token over its lens[b] cached tokens, as
 * rmm_attention computes it with Lq = 1 (causal: the new token is the last
 * position, so it sees the whole context).  Sources: "Alcance de Aplicación"
 * (feature reduction of Q K^T, token reduction of P V) and "Estrategia de
 * Selección" (column-norm scores, top-k); the pages state that the method
 * holds up in autoregressive generation.  With one row, the feature scores
 * are |q_f| and the token scores are the probabilities p_j.
 *   Q (device, bf16): element (b, h, f) at Q + b*q_seq_stride + h*q_head_stride + f.
 *   Kt (device, bf16): feature-major caches, element (b, g, f, j) at
 *        Kt + b*kt_seq_stride + g*kt_head_stride + f*ldkt + j, ldkt >= Lmax.
 *   V (device, bf16): element (b, j, g, d) at V + b*v_seq_stride + j*v_tok_stride
 *        + g*v_head_stride + d; 16-byte aligned rows (V and the three strides
 *        multiples of 8 elements), else RMM_ERR_UNSUPPORTED.
 *        Query head h reads kv head floor(h*Hkv/Hq).
 *   lens (device, int32) [nseq]: context length of each sequence (including
 *        the new token), clamped to [1, Lmax]; cache positions past it are
 *        never read for scores and never selected.
 *   k_tok (device, int32) [nseq]: tokens kept per sequence (the caller's
 *        ceil(rho * lens[b]), see rmm_k_from_rho), clamped to [1, min(lens[b], kt_max)].
 *   Lmax: longest context (cache capacity read); kt_max: the largest k_tok
 *        (1 <= kt_max <= Lmax), which sizes idx_tok rows.
 *   k_feat: features kept per (sequence, head), 1 <= k_feat <= dh; dh must be 128.
 *   O (device, bf16): element (b, h, d) at O + b*o_seq_stride + h*o_head_stride + d.
 *   idx_feat (device, int32) [nseq*Hq][rmm_k_pad(k_feat)], row b*Hq + h: kept
 *        features ascending, then -1.
 *   idx_tok (device, int32) [nseq*Hq][rmm_k_pad(kt_max)]: kept tokens of
 *        each row ascending, then -1 (ties to the lower index).
 *   tok_scores (device, float, optional) [nseq*Hq][Lmax]: token scores
 *        (-inf past lens[b]).
 *   ws: rmm_attention_decode_batch_workspace_bytes(nseq, Hq, dh, Lmax, kt_max)
 *        bytes, 256-byte aligned.
 * nseq * Hq must not exceed 65535.  Nothing is allocated; the call is
 * asynchronous on `stream` and can be captured in a HIP graph.
 */
size_t rmm_attention_decode_batch_workspace_bytes(int64_t nseq, int64_t Hq, int64_t dh, int64_t Lmax,
                                                  int64_t kt_max);
rmm_status_t rmm_attention_decode_batch(const void *Q, int64_t q_seq_stride, int64_t q_head_stride,
                                        const void *Kt, int64_t kt_seq_stride, int64_t kt_head_stride,
                                        int64_t ldkt, const void *V, int64_t v_seq_stride,
                                        int64_t v_tok_stride, int64_t v_head_stride, const int32_t *lens,
                                        const int32_t *k_tok, int64_t nseq, int64_t Hq, int64_t Hkv,
                                        int64_t dh, int64_t Lmax, int64_t k_feat, int64_t kt_max, void *O,
                                        int64_t o_seq_stride, int64_t o_head_stride, int32_t *idx_feat,
                                        int32_t *idx_tok, float *tok_scores, void *ws, size_t ws_bytes,
                                        rmm_stream_t stream);

/*
 * Per-kernel timing diagnostics (not part of the method; for measurement).
 * When enabled, each kernel the library enqueues is bracketed by two HIP
 * events recorded on its launch stream and filed under "<tag>/<kernel>"
 * (just "<kernel>" while the calling thread's tag is empty).
 *   rmm_timing_enable(on)     start (on != 0) or stop recording.
 *   rmm_timing_set_tag(tag)   label for later launches from this thread (host
 *                             string, copied; NULL or "" clears it).
 *   rmm_timing_collect()      wait for every recorded launch and add its
 *                             elapsed time to the totals (host-blocking).
 *   rmm_timing_count()        number of distinct "<tag>/<kernel>" totals.
 *   rmm_timing_entry(i, ...)  name (host buffer of name_len bytes), summed
 *                             milliseconds and launch count of total i.
 *   rmm_timing_reset()        clear the totals.
 * HIP events are created on first use and reused; no device memory is
 * allocated.  Recording adds two event records per launch.
 */
rmm_status_t rmm_timing_enable(int on);
rmm_status_t rmm_timing_set_tag(const char *tag);
rmm_status_t rmm_timing_collect(void);
int rmm_timing_count(void);
rmm_status_t rmm_timing_entry(int i, char *name, size_t name_len, double *total_ms,
                              int64_t *launches);
rmm_status_t rmm_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* RMM_H_ */

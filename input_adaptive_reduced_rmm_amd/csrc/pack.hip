// Gather of the kept activation columns, A_I = A[:, I] ("Mecanismo Central":
// the reduced product uses the slice A_{:,I}), into a dense K-contiguous buffer
// [batch][m][k_pad] whose tail columns k..k_pad-1 are zero, so the GEMM's K
// loop runs over whole 64-wide tiles.
//
// Each lane owns 16 bytes of one packed row (8 bf16 / 4 f32 consecutive kept
// columns).  Its column indices are loaded once and reused for every row the
// block walks; kept indices ascend, so neighbouring lanes read neighbouring
// addresses of the same source row and a wave's gathers fall in a few cache
// lines.  Stores are full 16-byte, fully coalesced.  The blocks of the first
// row block also write the cleaned index list (-1 for padding and for indices
// outside [0, d)) that the GEMM reads with 16-byte loads.
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
};

// grid: x = column block (kThreads*N packed columns), y = row block, z = batch.
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_kernel(const T *__restrict__ A, int64_t lda,
                                                        int64_t a_bs, const int32_t *__restrict__ idx,
                                                        int64_t idx_bs, int64_t m, int64_t d,
                                                        int64_t k, int64_t k_pad,
                                                        int64_t rows_per_block,
                                                        T *__restrict__ out,
                                                        int32_t *__restrict__ idx_clean) {
  constexpr int N = Vec16<T>::N;
  const int64_t t0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * N;
  if (t0 >= k_pad) return;
  const int64_t b = blockIdx.z;
  const int32_t *ib = idx + b * idx_bs;
  int64_t col[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    int64_t c = -1;
    if (t0 + e < k) {
      const int32_t v = ib[t0 + e];
      c = (v >= 0 && v < d) ? v : -1;
    }
    col[e] = c;
  }
  if (idx_clean && blockIdx.y == 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) idx_clean[b * k_pad + t0 + e] = (int32_t)col[e];
  }
  const T *Ab = A + b * a_bs;
  T *Ob = out + b * m * k_pad + t0;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(m, r0 + rows_per_block);
  for (int64_t r = r0; r < r1; ++r) {
    const T *row = Ab + r * lda;
    T v[N];
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = col[e] >= 0 ? row[col[e]] : T(0);
    if constexpr (N == 8) {
      uint4 w;
      w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
      w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
      w.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
      w.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4 *>(Ob + r * k_pad) = w;
    } else {
      *reinterpret_cast<float4 *>(Ob + r * k_pad) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace

hipError_t launch_pack(rmm_dtype_t dt, const void *A, int64_t lda, int64_t a_bs,
                       const int32_t *idx, int64_t idx_bs, int64_t batch, int64_t m, int64_t d,
                       int64_t k, int64_t k_pad, void *out, int32_t *idx_clean, hipStream_t st) {
  const int N = dt == RMM_BF16 ? 8 : 4;
  const int64_t col_blocks = ceil_div(k_pad, (int64_t)kThreads * N);
  // ~4096 blocks in total, at least 4 rows each.
  int64_t row_blocks = ceil_div(4096, col_blocks * batch);
  if (row_blocks > ceil_div(m, 4)) row_blocks = ceil_div(m, 4);
  if (row_blocks < 1) row_blocks = 1;
  if (row_blocks > 65535) row_blocks = 65535;
  const int64_t rpb = ceil_div(m, row_blocks);
  row_blocks = ceil_div(m, rpb);
  dim3 grid((unsigned)col_blocks, (unsigned)row_blocks, (unsigned)batch);
  KernelTimer timer("pack", st);
  if (dt == RMM_BF16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t *>(A), lda, a_bs, idx, idx_bs, m, d, k, k_pad,
                       rpb, static_cast<uint16_t *>(out), idx_clean);
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(kThreads), 0, st,
                       static_cast<const float *>(A), lda, a_bs, idx, idx_bs, m, d, k, k_pad, rpb,
                       static_cast<float *>(out), idx_clean);
  return hipGetLastError();
}

}  // namespace rmm

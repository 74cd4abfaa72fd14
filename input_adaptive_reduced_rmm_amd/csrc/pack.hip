// Gather of the kept activation columns, A_I = A[:, I] ("Mecanismo Central":
// the reduced product uses the slice A_{:,I}), into a dense K-contiguous buffer
// [batch][m][k_pad] whose tail columns k..k_pad-1 are zero, so the GEMM's K
// loop runs over whole 64-wide tiles.
//
// Each lane owns 16 bytes of one packed row (8 bf16 / 4 f32 consecutive kept
// columns).  Its column indices are loaded once and reused for every row the
// block walks; kept indices ascend, so neighbouring lanes read neighbouring
// addresses of the same source row and a wave's gathers fall in a few cache
// lines.  Narrow packed rows (head_dim features) are stacked several to a
// block so that no lane idles.  Stores are full 16-byte, fully coalesced.  The blocks of the first
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

// grid: x = column block, y = row block, z = batch.  A block row-slot covers
// `cpb` 16-byte chunks of a packed row; narrow rows (k_pad/N < kThreads) put
// `rpi` rows side by side in one block.  Each thread walks its rows kUnroll
// at a time so that kUnroll x N gathers are in flight before the stores.
constexpr int kUnroll = 4;
template <typename T>
__device__ __forceinline__ void store16(T *dst, const T *v) {
  if constexpr (sizeof(T) == 2) {
    uint4 w;
    w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    w.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    w.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    w.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4 *>(dst) = w;
  } else {
    *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// WIDE: one row per block at a time (rpi == 1), so the row is uniform and
// its address stays scalar.
template <typename T, bool WIDE>
__global__ __launch_bounds__(kThreads) void pack_kernel(const T *__restrict__ A, int64_t lda,
                                                        int64_t a_bs, const int32_t *__restrict__ idx,
                                                        int64_t idx_bs, int64_t m, int64_t d,
                                                        int64_t k, int64_t k_pad, int cpb, int rpi,
                                                        int64_t rows_per_block,
                                                        T *__restrict__ out,
                                                        int32_t *__restrict__ idx_clean) {
  constexpr int N = Vec16<T>::N;
  const int sub = WIDE ? 0 : (int)threadIdx.x / cpb;
  const int cl = WIDE ? (int)threadIdx.x : (int)threadIdx.x % cpb;
  if (!WIDE && sub >= rpi) return;
  const int64_t t0 = ((int64_t)blockIdx.x * cpb + cl) * N;
  if (t0 >= k_pad) return;
  const int64_t b = blockIdx.z;
  const int32_t *ib = idx + b * idx_bs;
  int32_t col[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    int32_t c = -1;
    if (t0 + e < k) {
      const int32_t v = ib[t0 + e];
      c = (v >= 0 && v < d) ? v : -1;
    }
    col[e] = c;
  }
  if (idx_clean && blockIdx.y == 0 && sub == 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) idx_clean[b * k_pad + t0 + e] = col[e];
  }
  const T *Ab = A + b * a_bs;
  T *Ob = out + b * m * k_pad + t0;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(m, r0 + rows_per_block);
  // Branch-free gathers: a dropped slot reads column 0 (always valid) and is
  // zeroed after the load.  All kUnroll x N gathers are issued before the
  // first store.
  int64_t cl64[N];
#pragma unroll
  for (int e = 0; e < N; ++e) cl64[e] = col[e] >= 0 ? col[e] : 0;
  const int step = WIDE ? 1 : rpi;
  int64_t r = r0 + sub;
  for (; r + (kUnroll - 1) * step < r1; r += kUnroll * step) {
    T v[kUnroll][N];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const T *__restrict__ row = Ab + (r + u * step) * lda;
#pragma unroll
      for (int e = 0; e < N; ++e) v[u][e] = row[cl64[e]];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int e = 0; e < N; ++e)
        if (col[e] < 0) v[u][e] = T(0);
      store16(Ob + (r + u * step) * k_pad, v[u]);
    }
  }
  for (; r < r1; r += step) {
    T v[N];
    const T *__restrict__ row = Ab + r * lda;
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = row[cl64[e]];
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (col[e] < 0) v[e] = T(0);
    store16(Ob + r * k_pad, v);
  }
}

}  // namespace

hipError_t launch_pack(rmm_dtype_t dt, const void *A, int64_t lda, int64_t a_bs,
                       const int32_t *idx, int64_t idx_bs, int64_t batch, int64_t m, int64_t d,
                       int64_t k, int64_t k_pad, void *out, int32_t *idx_clean, hipStream_t st) {
  const int N = dt == RMM_BF16 ? 8 : 4;
  const int64_t cpr = k_pad / N;                    // 16-byte chunks per packed row
  const int cpb = (int)(cpr < kThreads ? cpr : kThreads);
  const int rpi = kThreads / cpb;                   // rows side by side in a block
  const int64_t col_blocks = ceil_div(cpr, (int64_t)cpb);
  // ~4096 blocks in total, at least kUnroll row iterations each.
  int64_t row_blocks = ceil_div(4096, col_blocks * batch);
  if (row_blocks > ceil_div(m, (int64_t)rpi * kUnroll)) row_blocks = ceil_div(m, (int64_t)rpi * kUnroll);
  if (row_blocks < 1) row_blocks = 1;
  if (row_blocks > 65535) row_blocks = 65535;
  const int64_t rpb = ceil_div(m, row_blocks);
  row_blocks = ceil_div(m, rpb);
  dim3 grid((unsigned)col_blocks, (unsigned)row_blocks, (unsigned)batch);
  KernelTimer timer("pack", st);
  const bool wide = rpi == 1;
#define RMM_PACK(T, W)                                                                                   \
  hipLaunchKernelGGL((pack_kernel<T, W>), grid, dim3(kThreads), 0, st, static_cast<const T *>(A), lda, a_bs, \
                     idx, idx_bs, m, d, k, k_pad, cpb, rpi, rpb, static_cast<T *>(out), idx_clean)
  if (dt == RMM_BF16) {
    if (wide) RMM_PACK(uint16_t, true);
    else RMM_PACK(uint16_t, false);
  } else {
    if (wide) RMM_PACK(float, true);
    else RMM_PACK(float, false);
  }
#undef RMM_PACK
  return hipGetLastError();
}

}  // namespace rmm

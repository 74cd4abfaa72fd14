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
//
// Wide bf16 rows (the projections: d >= 512, one matrix) go through
// pack_rows_kernel instead: at the ratios the method uses nearly every
// 128-byte line of a source row holds a kept column, so the whole row is read
// with 16-byte direct-to-LDS loads (one load instruction per 16 bytes rather
// than per 2-byte element) and the kept columns are gathered from LDS.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

#define LDS_AS __attribute__((address_space(3)))

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
  for (int e = 0; e < N; ++e) col[e] = ib[t0 + e < k ? t0 + e : k - 1];   // all loads first
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int32_t v = col[e];
    col[e] = (t0 + e < k && v >= 0 && v < d) ? v : -1;
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

// One block walks `rows_per_block` rows through two LDS row buffers: while
// the kept columns of row r are gathered from one buffer and written, the
// whole of row r + 1 streams into the other (16-byte direct-to-LDS loads, one
// 1 KiB piece per wave instruction).  Every thread writes MAXC 16-byte chunks
// of each packed row (8 kept columns each; padding slots are zero) with
// buffer stores; chunks past the row go to an offset outside the row's
// resource and are dropped, so every wave issues exactly MAXC stores per row
// and the wait for row r + 1's loads can leave the MAXC stores of row r in
// flight (vmcnt counts loads and stores together, in issue order).
__device__ __forceinline__ void lds_row_load16(mg::rsrc_t r, void *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)lds, 16, voff, 0, 0, 0);
}

// Immediate of s_waitcnt vmcnt(n) with lgkmcnt and expcnt left alone.
constexpr int vm_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

template <int MAXC>
__global__ __launch_bounds__(kThreads) void pack_rows_kernel(const uint16_t *__restrict__ A, int64_t lda,
                                                             const int32_t *__restrict__ idx, int64_t m,
                                                             int64_t d, int64_t k, int64_t k_pad,
                                                             int64_t rows_per_block, int64_t row_bytes,
                                                             uint16_t *__restrict__ out,
                                                             int32_t *__restrict__ idx_clean) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char row_lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nchunk = k_pad / 8;
  // Kept columns of this thread's chunks.  Every load is issued before any
  // is used (slots past k read entry k - 1 and are then dropped), so the
  // block pays one memory latency here rather than one per index.
  int32_t col[MAXC][8];
#pragma unroll
  for (int u = 0; u < MAXC; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = (tid + (int64_t)kThreads * u) * 8 + e;
      col[u][e] = idx[t < k ? t : k - 1];
    }
#pragma unroll
  for (int u = 0; u < MAXC; ++u) {
    const int64_t c = tid + (int64_t)kThreads * u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int32_t x = col[u][e];
      col[u][e] = (c * 8 + e < k && x >= 0 && x < d) ? x : -1;
    }
    if (idx_clean && blockIdx.x == 0 && c < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) idx_clean[c * 8 + e] = col[u][e];
    }
  }
  const mg::rsrc_t ra = mg::make_rsrc(A, (uint64_t)((m - 1) * lda + d) * 2);
  const int nblk1k = (int)((d * 2 + 1023) / 1024);   // 1 KiB pieces of a row
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < m ? r0 + rows_per_block : m;
  auto issue_row = [&](int64_t r, unsigned char *buf) {
    for (int q = wave; q < nblk1k; q += kThreads / 64)
      lds_row_load16(ra, buf + q * 1024, (uint32_t)(r * lda * 2 + q * 1024 + lane * 16));
  };
  if (r0 < r1) issue_row(r0, row_lds);
  for (int64_t r = r0; r < r1; ++r) {
    const unsigned char *cur = row_lds + ((r - r0) & 1) * row_bytes;
    // Row r landed: after its loads this wave issued only the MAXC stores of
    // row r - 1.
    if (r == r0) __builtin_amdgcn_s_waitcnt(vm_imm(0));
    else __builtin_amdgcn_s_waitcnt(vm_imm(MAXC));
    // Every wave's pieces of row r are in, and row r - 1's buffer is no
    // longer read (its LDS reads were consumed before its stores were
    // issued).  A bare barrier: __syncthreads would also wait for this
    // wave's stores of row r - 1.
    __builtin_amdgcn_s_barrier();
    if (r + 1 < r1) issue_row(r + 1, row_lds + ((r + 1 - r0) & 1) * row_bytes);
    __builtin_amdgcn_sched_barrier(0);   // the stores below stay after these loads
    const uint16_t *row16 = reinterpret_cast<const uint16_t *>(cur);
    const mg::rsrc_t ro = mg::make_rsrc(out + r * k_pad, (uint64_t)k_pad * 2);
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
      const int64_t c = tid + (int64_t)kThreads * u;
      uint16_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = row16[col[u][e] >= 0 ? col[u][e] : 0];   // dropped slots read column 0
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col[u][e] < 0) v[e] = 0;
      typedef int v4i __attribute__((ext_vector_type(4)));
      const v4i w = {(int)((uint32_t)v[0] | ((uint32_t)v[1] << 16)), (int)((uint32_t)v[2] | ((uint32_t)v[3] << 16)),
                     (int)((uint32_t)v[4] | ((uint32_t)v[5] << 16)), (int)((uint32_t)v[6] | ((uint32_t)v[7] << 16))};
      __builtin_amdgcn_raw_buffer_store_b128(w, ro, c < nchunk ? (int)(c * 16) : (int)mg::kOOB, 0, 0);
    }
  }
}

}  // namespace

hipError_t launch_pack(rmm_dtype_t dt, const void *A, int64_t lda, int64_t a_bs,
                       const int32_t *idx, int64_t idx_bs, int64_t batch, int64_t m, int64_t d,
                       int64_t k, int64_t k_pad, void *out, int32_t *idx_clean, hipStream_t st) {
  const int N = dt == RMM_BF16 ? 8 : 4;
  const int64_t row_bytes = ceil_div(d * 2, 1024) * 1024;
  if (dt == RMM_BF16 && batch == 1 && d >= 512 && row_bytes <= 64 * 1024 && k_pad <= 8 * 8 * kThreads &&
      reinterpret_cast<uintptr_t>(A) % 16 == 0 && lda % 8 == 0 && (uint64_t)((m - 1) * lda + d) * 2 < mg::kMaxRecords) {
    const int64_t nchunk = k_pad / 8;
    const int64_t per_thread = ceil_div(nchunk, (int64_t)kThreads);
    // about 1024 blocks of at least one row, each with two row buffers
    int64_t rpb = ceil_div(m, 1024);
    const int64_t blocks = ceil_div(m, rpb);
    KernelTimer timer("pack", st);
#define RMM_PACK_ROWS(C)                                                                                      \
  hipLaunchKernelGGL(pack_rows_kernel<C>, dim3((unsigned)blocks), dim3(kThreads), (unsigned)(2 * row_bytes), st, \
                     static_cast<const uint16_t *>(A), lda, idx, m, d, k, k_pad, rpb, row_bytes,                  \
                     static_cast<uint16_t *>(out), idx_clean)
    if (per_thread <= 1) RMM_PACK_ROWS(1);
    else if (per_thread <= 2) RMM_PACK_ROWS(2);
    else if (per_thread <= 4) RMM_PACK_ROWS(4);
    else RMM_PACK_ROWS(8);
#undef RMM_PACK_ROWS
    return hipGetLastError();
  }
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

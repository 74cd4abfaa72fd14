// Column scores s_j = ||A[:, j]||_2 ("Estrategia de Selección": the importance of
// contraction index j is the Euclidean norm of activation column j).
//
// HBM-bound streaming reduction.  Each lane owns `VEC` adjacent columns and
// loads 16 bytes per row, so a wave reads 64 x 16 B = 1 KiB of contiguous row
// segment(s): for d >= 512 (bf16) a wave covers one row per step; for narrow
// matrices (head_dim 128) it covers 64/TPR rows at once and the lanes that
// share a column are folded with cross-lane xor shuffles at the end.  The
// four waves of a block then meet in LDS.  Rows are split into chunks over
// gridDim.y to put a few thousand blocks on the 256 CUs; per-chunk partial
// sums land in the workspace and a small second kernel adds them in chunk
// order and takes the square root, so the result is bitwise deterministic.
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;             // rows in flight per lane
constexpr int64_t kChunkRows = 1024;   // rows per block at most, where the grid allows
constexpr int kCausalTpr = 32;         // lanes across a row segment of a causal matrix (512 bytes)
constexpr int kWaves = kThreads / 64;

template <typename T, int VEC>
struct Loader;

// bf16, 8 per lane: one 16-byte load.  `d` is the row's column limit; with a
// separate matrix width `w` >= d (causal rows), a lane whose 8 columns stay
// inside the row still loads them as one vector and drops those >= d.
// NT: streaming (non-temporal) 16-byte loads, for matrices read once here
// and too large to stay in any cache (attention probabilities).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 load16(const void *p) {
  if constexpr (NT) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
  } else {
    return *reinterpret_cast<const uint4 *>(p);
  }
}

template <>
struct Loader<uint16_t, 8> {
  template <bool NT = false>
  __device__ static void load_sq(const uint16_t *p, int64_t c0, int64_t d, float *acc,
                                 int64_t w = -1) {
    if (c0 + 8 <= (w < 0 ? d : w) && c0 < d) {
      uint4 v = load16<NT>(p);
      float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                    bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = (c0 + e < d) ? x[e] : 0.f;
        acc[e] = fmaf(y, y, acc[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < d) {
          float x = bf16_to_f32(p[e]);
          acc[e] = fmaf(x, x, acc[e]);
        }
    }
  }
};

// f32, 4 per lane: one 16-byte load.
template <>
struct Loader<float, 4> {
  template <bool NT = false>
  __device__ static void load_sq(const float *p, int64_t c0, int64_t d, float *acc, int64_t = -1) {
    if (c0 + 4 <= d) {
      const uint4 u = load16<NT>(p);
      const float4 v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                                   __uint_as_float(u.w));
      acc[0] = fmaf(v.x, v.x, acc[0]);
      acc[1] = fmaf(v.y, v.y, acc[1]);
      acc[2] = fmaf(v.z, v.z, acc[2]);
      acc[3] = fmaf(v.w, v.w, acc[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c0 + e < d) acc[e] = fmaf(p[e], p[e], acc[e]);
    }
  }
};

// Scalar fallback for layouts that forbid 16-byte loads.
template <typename T>
struct Loader<T, 1> {
  template <bool NT = false>
  __device__ static void load_sq(const T *p, int64_t c0, int64_t d, float *acc, int64_t = -1) {
    if (c0 < d) {
      float x;
      if constexpr (sizeof(T) == 2) x = bf16_to_f32(*p);
      else x = *p;
      acc[0] = fmaf(x, x, acc[0]);
    }
  }
};

// grid: x = column tile (TPR*VEC columns), y = row chunk, z = batch.
// out: partial sums [chunk][batch][d] (or final scores when `final_sqrt`).
// CAUSAL: entry (i, j) is taken as zero and not read when j > i + coff (a
// causal attention matrix); rows that cannot reach a lane's columns are skipped.
template <typename T, int VEC, int TPR, bool CAUSAL, bool NT>
__global__ __launch_bounds__(kThreads) void colnorm_kernel(const T *__restrict__ A, int64_t m,
                                                           int64_t d, int64_t lda,
                                                           int64_t batch_stride,
                                                           int64_t rows_per_chunk,
                                                           float *__restrict__ out,
                                                           int final_sqrt, int64_t coff) {
  constexpr int RPW = 64 / TPR;       // rows one wave covers per step
  constexpr int RPB = kWaves * RPW;   // rows the block covers per step
  constexpr int CT = TPR * VEC;       // columns per block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / TPR;
  const int cl = lane % TPR;
  const int64_t col0 = (int64_t)blockIdx.x * CT;
  const int64_t c0 = col0 + (int64_t)cl * VEC;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r_end = min(m, r_begin + rows_per_chunk);
  const T *Ab = A + (int64_t)blockIdx.z * batch_stride + c0;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  if (c0 < d) {
    int64_t r = r_begin + wave * RPW + sub;
    if constexpr (CAUSAL) {
      // Rows i < col0 - coff reach no column of this tile; keep the lane's row phase.
      const int64_t first = col0 - coff;
      if (first > r_begin) r += ((first - r_begin) / RPB) * RPB;
      // Rows that cut through the tile's columns: per-element limits.  From
      // row col0 + CT - 1 - coff on, every column of the tile is kept and the
      // plain loop below takes over.
      int64_t band = col0 + CT - 1 - coff;
      if (band > r_end) band = r_end;
      for (; r + (kUnroll - 1) * RPB < band; r += kUnroll * RPB) {
        const T *p = Ab + r * lda;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          Loader<T, VEC>::template load_sq<NT>(p + u * RPB * lda, c0, min(d, r + u * RPB + coff + 1), acc, d);
      }
      for (; r < band; r += RPB) Loader<T, VEC>::template load_sq<NT>(Ab + r * lda, c0, min(d, r + coff + 1), acc, d);
    }
    // kUnroll rows in flight per lane
    for (; r + (kUnroll - 1) * RPB < r_end; r += kUnroll * RPB) {
      const T *p = Ab + r * lda;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) Loader<T, VEC>::template load_sq<NT>(p + u * RPB * lda, c0, d, acc);
    }
    for (; r < r_end; r += RPB) Loader<T, VEC>::template load_sq<NT>(Ab + r * lda, c0, d, acc);
  }

  // Fold the lanes that share a column (lane, lane^TPR, lane^2TPR, ...).
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }

  __shared__ float red[kWaves][CT];
  if (sub == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[wave][cl * VEC + e] = acc[e];
  }
  __syncthreads();
  float *o = out + ((int64_t)blockIdx.y * gridDim.z + blockIdx.z) * d;
  for (int c = threadIdx.x; c < CT; c += kThreads) {
    const int64_t col = col0 + c;
    if (col < d) {
      float s = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
      o[col] = final_sqrt ? __builtin_sqrtf(s) : s;
    }
  }
}

// scores[b][j] = sqrt(sum over chunks of part[c][b][j]) in a fixed order:
// 16 thread groups each add the chunks c = g, g + 16, ... (eight loads in
// flight per step), then the 16 group sums are added in group order.
constexpr int kFinCols = 64, kFinGroups = 16;
__global__ __launch_bounds__(kFinCols * kFinGroups) void colnorm_finish(const float *__restrict__ part,
                                                                      int64_t chunks, int64_t n,
                                                                      float *__restrict__ scores) {
  __shared__ float red[kFinGroups][kFinCols];
  const int col = threadIdx.x % kFinCols, grp = threadIdx.x / kFinCols;
  const int64_t i = (int64_t)blockIdx.x * kFinCols + col;
  float s = 0.f;
  if (i < n) {
    int64_t c = grp;
    for (; c + 7 * kFinGroups < chunks; c += 8 * kFinGroups) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(c + u * kFinGroups) * n + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < chunks; c += kFinGroups) s += part[c * n + i];
  }
  red[grp][col] = s;
  __syncthreads();
  if (grp == 0 && i < n) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < kFinGroups; ++q) t += red[q][col];
    scores[i] = __builtin_sqrtf(t);
  }
}

template <typename T, int VEC, bool CAUSAL, bool NT = false>
hipError_t dispatch_tpr(int tpr, dim3 grid, const T *A, int64_t m, int64_t d, int64_t lda,
                        int64_t bs, int64_t rpc, float *out, int fin, int64_t coff, hipStream_t st) {
  KernelTimer timer("colnorm", st);
  switch (tpr) {
#define RMM_CN(TP)                                                                                \
  case TP:                                                                                        \
    hipLaunchKernelGGL((colnorm_kernel<T, VEC, TP, CAUSAL, NT>), grid, dim3(kThreads), 0, st, A, m, \
                       d, lda, bs, rpc, out, fin, coff);                                          \
    break;
    RMM_CN(1) RMM_CN(2) RMM_CN(4) RMM_CN(8) RMM_CN(16) RMM_CN(32) RMM_CN(64)
#undef RMM_CN
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_colnorm_finish(const float *part, int64_t chunks, int64_t n, float *scores, hipStream_t st) {
  KernelTimer timer("colnorm_finish", st);
  hipLaunchKernelGGL(colnorm_finish, dim3((unsigned)ceil_div(n, kFinCols)), dim3(kFinCols * kFinGroups), 0, st, part,
                     chunks, n, scores);
  return hipGetLastError();
}

ColnormPlan colnorm_plan(rmm_dtype_t dt, int64_t m, int64_t d, int64_t batch, bool vec_ok, bool causal) {
  ColnormPlan p;
  const int esz = dt == RMM_BF16 ? 2 : 4;
  p.vec = vec_ok ? 16 / esz : 1;
  const int64_t lanes_needed = ceil_div(d, p.vec);
  // Causal: blocks on and above the diagonal carry less work or none, and a
  // grid of uneven blocks ends in a ragged last round; narrower column tiles
  // (32 lanes, 512-byte row segments) keep the tail short.  On 32 heads of
  // 16384 x 16384: 256-byte segments 1.44 ms, 512-byte 1.36 ms, 1 KiB 1.68 ms.
  const int max_tpr = causal ? kCausalTpr : 64;
  int tpr = 1;
  while (tpr < max_tpr && tpr < lanes_needed) tpr <<= 1;
  p.tpr = tpr;
  p.col_tiles = ceil_div(d, (int64_t)tpr * p.vec);
  const int64_t rpb = (int64_t)kWaves * (64 / tpr);
  // Aim for ~4096 blocks of at most ~1024 rows, but give each block at least
  // 8 steps of rows.
  const int64_t tiles = p.col_tiles * batch;
  int64_t want_chunks = ceil_div(4096, tiles);
  if (want_chunks < ceil_div(m, kChunkRows)) want_chunks = ceil_div(m, kChunkRows);
  if (want_chunks > 256) want_chunks = 256;
  int64_t max_chunks = ceil_div(m, rpb * 8);
  int64_t chunks = want_chunks < max_chunks ? want_chunks : max_chunks;
  if (chunks < 1) chunks = 1;
  if (chunks > 65535) chunks = 65535;
  int64_t rpc = ceil_div(ceil_div(m, chunks), rpb) * rpb;
  p.rows_per_chunk = rpc;
  p.chunks = ceil_div(m, rpc);
  return p;
}

size_t colnorm_ws_bytes(const ColnormPlan &p, int64_t d, int64_t batch) {
  return p.chunks > 1 ? (size_t)p.chunks * (size_t)batch * (size_t)d * sizeof(float) : 0;
}

hipError_t launch_colnorm(rmm_dtype_t dt, const void *A, int64_t m, int64_t d, int64_t lda,
                          int64_t batch, int64_t batch_stride, float *scores, void *ws,
                          const ColnormPlan &p, hipStream_t st, bool causal, int64_t coff, bool stream) {
  const bool single = p.chunks == 1;
  float *out = single ? scores : static_cast<float *>(ws);
  dim3 grid((unsigned)p.col_tiles, (unsigned)p.chunks, (unsigned)batch);
  const int64_t bs = batch_stride, rpc = p.rows_per_chunk;
  hipError_t e;
  if (dt == RMM_BF16) {
    const uint16_t *a = static_cast<const uint16_t *>(A);
    if (p.vec != 8)
      e = causal ? dispatch_tpr<uint16_t, 1, true>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, coff, st)
                 : dispatch_tpr<uint16_t, 1, false>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, 0, st);
    else if (causal)
      e = stream ? dispatch_tpr<uint16_t, 8, true, true>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, coff, st)
                 : dispatch_tpr<uint16_t, 8, true>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, coff, st);
    else
      e = stream ? dispatch_tpr<uint16_t, 8, false, true>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, 0, st)
                 : dispatch_tpr<uint16_t, 8, false>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, 0, st);
  } else {
    const float *a = static_cast<const float *>(A);
    e = p.vec == 4 ? dispatch_tpr<float, 4, false>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, 0, st)
                   : dispatch_tpr<float, 1, false>(p.tpr, grid, a, m, d, lda, bs, rpc, out, single, 0, st);
  }
  if (e != hipSuccess || single) return e;
  const int64_t n = batch * d;
  KernelTimer timer("colnorm_finish", st);
  hipLaunchKernelGGL(colnorm_finish, dim3((unsigned)ceil_div(n, kFinCols)), dim3(kFinCols * kFinGroups), 0, st,
                     static_cast<const float *>(ws), p.chunks, n, scores);
  return hipGetLastError();
}

}  // namespace rmm

// Producer-fused column scores: the kernel that writes an activation also
// accumulates the sums of squares of its columns, so the next reduced product
// can select its indices without reading the activation again ("Estrategia de
// Selección": the score of index j is the norm of column j of A; the pages
// call it a lightweight vector operation beside the product).
//
// swiglu_scored_kernel writes the gated MLP activation H = silu(G) * U (the
// input of the down projection of a LLaMA-style layer), rounded to bf16, and
// adds the squares of exactly those bf16 values per column.  A wave covers 512
// contiguous columns of a row (16 bytes per lane); the four waves of a block
// take interleaved rows of its row chunk, four rows in flight per lane, and
// meet in LDS at the end; chunk partials are added in a fixed order by
// colnorm_finish, so the scores are bitwise deterministic.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kWaves = 4;
constexpr int kCols = 64 * 8;   // columns per block (8 bf16 per lane)
constexpr int kUnroll = 4;      // rows in flight per lane

__device__ __forceinline__ float silu(float x) {
  // x * sigmoid(x) = x / (1 + 2^(-x log2 e))
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

__global__ __launch_bounds__(64 * kWaves) void swiglu_scored_kernel(const uint16_t *__restrict__ G, int64_t ldg,
                                                                    const uint16_t *__restrict__ U, int64_t ldu,
                                                                    int64_t m, int64_t n, uint16_t *__restrict__ H,
                                                                    int64_t ldh, int64_t rows_per_chunk,
                                                                    float *__restrict__ out, int final_sqrt) {
  __shared__ float red[kWaves][kCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kCols + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < m ? r0 + rows_per_chunk : m;
  const bool col_ok = c0 < n;   // n % 8 == 0: a chunk is all in or all out
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (col_ok) {
    for (int64_t rb = r0 + wave; rb < r1; rb += kWaves * kUnroll) {
      uint4 gv[kUnroll], uv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = rb + (int64_t)u * kWaves;
        if (r < r1) {
          gv[u] = *reinterpret_cast<const uint4 *>(G + r * ldg + c0);
          uv[u] = *reinterpret_cast<const uint4 *>(U + r * ldu + c0);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t r = rb + (int64_t)u * kWaves;
        if (r < r1) {
          uint32_t hw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t gw = mg::u4get(gv[u], q), uw = mg::u4get(uv[u], q);
            const float h0 = silu(bf16_lo(gw)) * bf16_lo(uw);
            const float h1 = silu(bf16_hi(gw)) * bf16_hi(uw);
            hw[q] = pack_bf16x2(h0, h1);
            // the scores are of the bf16 values the next product reads
            const float b0 = bf16_lo(hw[q]), b1 = bf16_hi(hw[q]);
            acc[2 * q] = fmaf(b0, b0, acc[2 * q]);
            acc[2 * q + 1] = fmaf(b1, b1, acc[2 * q + 1]);
          }
          *reinterpret_cast<uint4 *>(H + r * ldh + c0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  // 256 threads finish 512 columns: two each, waves added in order
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + h * 64 * kWaves;
    const int64_t col = (int64_t)blockIdx.x * kCols + c;
    if (col < n) {
      const float s = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
      out[(int64_t)blockIdx.y * n * (1 - final_sqrt) + col] = final_sqrt ? __builtin_sqrtf(s) : s;
    }
  }
}

// rmsnorm_scored_kernel writes Y = bf16(x * w / sqrt(mean(x^2) + eps)) per
// row (the normalised input of the q, k, v and up, gate projections of a
// LLaMA-style layer) and adds the squares of the bf16 Y per column.  A
// workgroup has one thread per 8 columns (d / 8 threads, 1 to 16 waves), so
// each column belongs to one thread and its sum needs no reduction across
// threads.  kRmsRows rows are in flight per thread; their sums of squares meet
// through a double-buffered LDS array (one barrier per kRmsRows rows, the
// waves' parts added in wave order).
constexpr int kRmsRows = 4;

__global__ __launch_bounds__(1024) void rmsnorm_scored_kernel(const uint16_t *__restrict__ X, int64_t ldx,
                                                               const uint16_t *__restrict__ w, float eps, int64_t m,
                                                               int64_t d, uint16_t *__restrict__ Y, int64_t ldy,
                                                               int64_t rows_per_chunk, float *__restrict__ out,
                                                               int final_sqrt) {
  __shared__ float red[2][kRmsRows][16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  const int64_t col = (int64_t)t * 8;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < m ? r0 + rows_per_chunk : m;
  const float inv_d = 1.f / (float)d;
  const uint4 wv = *reinterpret_cast<const uint4 *>(w + col);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  int buf = 0;
  for (int64_t rb = r0; rb < r1; rb += kRmsRows) {
    uint4 xv[kRmsRows];
#pragma unroll
    for (int u = 0; u < kRmsRows; ++u)
      xv[u] = rb + u < r1 ? *reinterpret_cast<const uint4 *>(X + (rb + u) * ldx + col) : make_uint4(0, 0, 0, 0);
    float ss[kRmsRows];
#pragma unroll
    for (int u = 0; u < kRmsRows; ++u) {
      ss[u] = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t xw = mg::u4get(xv[u], q);
        const float a = bf16_lo(xw), b = bf16_hi(xw);
        ss[u] = fmaf(a, a, ss[u]);
        ss[u] = fmaf(b, b, ss[u]);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss[u] += __shfl_xor(ss[u], o, 64);
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kRmsRows; ++u) red[buf][u][wave] = ss[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kRmsRows; ++u) {
      const int64_t r = rb + u;
      if (r < r1) {
        float tot = 0.f;
        for (int v = 0; v < nw; ++v) tot += red[buf][u][v];
        const float inv = 1.f / __builtin_sqrtf(tot * inv_d + eps);
        uint32_t yw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t xw = mg::u4get(xv[u], q), ww = mg::u4get(wv, q);
          yw[q] = pack_bf16x2(bf16_lo(xw) * inv * bf16_lo(ww), bf16_hi(xw) * inv * bf16_hi(ww));
          const float y0 = bf16_lo(yw[q]), y1 = bf16_hi(yw[q]);
          acc[2 * q] = fmaf(y0, y0, acc[2 * q]);
          acc[2 * q + 1] = fmaf(y1, y1, acc[2 * q + 1]);
        }
        *reinterpret_cast<uint4 *>(Y + r * ldy + col) = make_uint4(yw[0], yw[1], yw[2], yw[3]);
      }
    }
    buf ^= 1;
  }
  float *o = out + (int64_t)blockIdx.x * d * (1 - final_sqrt) + col;
  if (final_sqrt) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_sqrtf(acc[e]);
  }
  if ((reinterpret_cast<uintptr_t>(out) & 15) == 0) {   // partials always; scores when 16-byte aligned
    *reinterpret_cast<float4 *>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4 *>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[e];
  }
}

struct SwigluPlan {
  int64_t col_tiles, rows_per_chunk, chunks;
};

SwigluPlan swiglu_plan(int64_t m, int64_t n) {
  SwigluPlan p;
  p.col_tiles = ceil_div(n, kCols);
  // About 4096 blocks, each with at least 64 rows, at most 256 chunks.
  int64_t chunks = ceil_div(4096, p.col_tiles);
  const int64_t max_chunks = ceil_div(m, 64);
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks > 256) chunks = 256;
  if (chunks < 1) chunks = 1;
  const int64_t step = kWaves * kUnroll;
  p.rows_per_chunk = ceil_div(ceil_div(m, chunks), step) * step;
  p.chunks = ceil_div(m, p.rows_per_chunk);
  return p;
}

// About 512 workgroups, each a whole number of row groups.
constexpr int64_t kRmsBlocks = 512;
int64_t rmsnorm_rows_per_chunk(int64_t m) { return ceil_div(ceil_div(m, kRmsBlocks), kRmsRows) * kRmsRows; }

}  // namespace

bool rmsnorm_ok(const void *X, int64_t ldx, const void *w, const void *Y, int64_t ldy, int64_t d) {
  auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return al(X) && al(w) && al(Y) && ldx % 8 == 0 && ldy % 8 == 0 && d % kCols == 0 && d / kCols >= 1 &&
         d / kCols <= 16;
}

size_t rmsnorm_part_bytes(int64_t m, int64_t d) {
  const int64_t chunks = ceil_div(m, rmsnorm_rows_per_chunk(m));
  return chunks > 1 ? (size_t)chunks * (size_t)d * 4 : 0;
}

hipError_t launch_rmsnorm_scored(const void *X, int64_t ldx, const void *w, float eps, int64_t m, int64_t d, void *Y,
                                 int64_t ldy, float *scores, float *part, hipStream_t st) {
  const int64_t rpc = rmsnorm_rows_per_chunk(m), chunks = ceil_div(m, rpc);
  const bool single = chunks == 1;
  {
    KernelTimer timer("rmsnorm_scored", st);
    const uint16_t *x = static_cast<const uint16_t *>(X), *wp = static_cast<const uint16_t *>(w);
    uint16_t *y = static_cast<uint16_t *>(Y);
    float *o = single ? scores : part;
    const dim3 grid((unsigned)chunks), blk((unsigned)(d / 8));
    hipLaunchKernelGGL(rmsnorm_scored_kernel, grid, blk, 0, st, x, ldx, wp, eps, m, d, y, ldy, rpc, o, single);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || single) return e;
  }
  return launch_colnorm_finish(part, chunks, d, scores, st);
}

bool swiglu_ok(const void *G, int64_t ldg, const void *U, int64_t ldu, const void *H, int64_t ldh, int64_t n) {
  auto al = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return al(G) && al(U) && al(H) && ldg % 8 == 0 && ldu % 8 == 0 && ldh % 8 == 0 && n % 8 == 0;
}

size_t swiglu_part_bytes(int64_t m, int64_t n) {
  const SwigluPlan p = swiglu_plan(m, n);
  return p.chunks > 1 ? (size_t)p.chunks * (size_t)n * 4 : 0;
}

hipError_t launch_swiglu_scored(const void *G, int64_t ldg, const void *U, int64_t ldu, int64_t m, int64_t n,
                                void *H, int64_t ldh, float *scores, float *part, hipStream_t st) {
  const SwigluPlan p = swiglu_plan(m, n);
  const bool single = p.chunks == 1;
  {
    KernelTimer timer("swiglu_scored", st);
    hipLaunchKernelGGL(swiglu_scored_kernel, dim3((unsigned)p.col_tiles, (unsigned)p.chunks), dim3(64 * kWaves), 0,
                       st, static_cast<const uint16_t *>(G), ldg, static_cast<const uint16_t *>(U), ldu, m, n,
                       static_cast<uint16_t *>(H), ldh, p.rows_per_chunk, single ? scores : part, single ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || single) return e;
  }
  return launch_colnorm_finish(part, p.chunks, n, scores, st);
}

}  // namespace rmm

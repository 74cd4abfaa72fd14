// Top-k selection of column scores ("Estrategia de Selección": keep the k
// indices with the highest scores), ties to the lower index, output ascending.
//
// One workgroup per batch row (1024 threads; 256 for rows of at most 4096).
// Scores are mapped to order-preserving unsigned keys and (for d up to
// kLdsKeys) parked in LDS; the exact radix select and the ascending emission
// are sel::block_select.  All integer work: the result is exact.
#include "rmm_internal.h"
#include "select.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kLdsKeys = 32768;  // 128 KiB of keys; beyond that, keys are re-read from global

// NT threads per workgroup: 1024 for long rows, 256 for short ones (fewer
// waves meet at each of the select's barriers).
// k_rows (optional): row b keeps k_rows[b / k_div] indices instead of k,
// clamped to [1, min(k, d, len)] (ragged batches: one count per sequence,
// shared by its heads; k is then the largest count, which sizes the output
// rows).  len_rows (optional, with k_rows): the row's valid length
// len_rows[b / k_div], itself clamped to [1, d]; scores past it are never
// kept, so no more than len indices are.
template <bool IN_LDS, int NT>
__global__ __launch_bounds__(NT) void topk_kernel(const float *__restrict__ scores, int64_t d,
                                                        int64_t k, int64_t k_pad,
                                                        int32_t *__restrict__ idx,
                                                        const int32_t *__restrict__ k_rows,
                                                        const int32_t *__restrict__ len_rows, int k_div) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[IN_LDS ? (NT == 256 ? 4096 : kLdsKeys) : 1];
  __shared__ sel::BlockShared<NT> sh;

  const int tid = threadIdx.x;
  if (k_rows) {
    int64_t kmax = k < d ? k : d;
    if (len_rows) {
      const int64_t L = len_rows[blockIdx.x / k_div];
      const int64_t Lc = L < 1 ? 1 : (L > d ? d : L);
      if (Lc < kmax) kmax = Lc;
    }
    const int64_t kr = k_rows[blockIdx.x / k_div];
    k = kr < 1 ? 1 : (kr > kmax ? kmax : kr);
  }
  const float *s = scores + (int64_t)blockIdx.x * d;
  int32_t *out = idx + (int64_t)blockIdx.x * k_pad;

  // Load keys (into LDS when they fit); OR/AND over this thread's keys.
  // Eight loads per thread are issued before any is used, so the pass costs
  // about one memory latency per eight loads instead of one per load.  Rows
  // of 16-byte aligned scores are read four keys per load (a quarter of the
  // load instructions, whose issue otherwise bounds this pass).
  uint32_t kor = 0u, kand = 0xFFFFFFFFu;
  if (IN_LDS && d % 4 == 0 && reinterpret_cast<uintptr_t>(s) % 16 == 0) {
    const float4 *s4 = reinterpret_cast<const float4 *>(s);
    const int64_t d4 = d / 4;
    for (int64_t t0 = tid; t0 < d4; t0 += 8 * NT) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t t = t0 + (int64_t)u * NT;
        v[u] = t < d4 ? s4[t] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t t = t0 + (int64_t)u * NT;
        if (t < d4) {
          const uint4 key = make_uint4(sel::score_key(v[u].x), sel::score_key(v[u].y), sel::score_key(v[u].z),
                                       sel::score_key(v[u].w));
          if constexpr (IN_LDS) *reinterpret_cast<uint4 *>(&keys[4 * t]) = key;
          kor |= key.x | key.y | key.z | key.w;
          kand &= key.x & key.y & key.z & key.w;
        }
      }
    }
  } else {
    for (int64_t j0 = tid; j0 < d; j0 += 8 * NT) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * NT;
        v[u] = j < d ? s[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * NT;
        if (j < d) {
          const uint32_t key = sel::score_key(v[u]);
          if constexpr (IN_LDS) keys[j] = key;
          kor |= key;
          kand &= key;
        }
      }
    }
  }
  if constexpr (IN_LDS)
    sel::block_select<NT>([&](int64_t j) -> uint32_t { return keys[j]; }, d, kor, kand, k, k_pad, out, sh);
  else
    sel::block_select<NT>([&](int64_t j) -> uint32_t { return sel::score_key(s[j]); }, d, kor, kand, k, k_pad,
                          out, sh);
}

// k == d: every index is kept.
__global__ __launch_bounds__(256) void iota_kernel(int64_t d, int64_t k_pad, int32_t *idx) {
  int32_t *out = idx + (int64_t)blockIdx.y * k_pad;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < k_pad; t += (int64_t)gridDim.x * 256)
    out[t] = t < d ? (int32_t)t : -1;
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t batch, int64_t d, int64_t k, int64_t k_pad,
                       int32_t *idx, hipStream_t st, const int32_t *k_rows, int k_div, const int32_t *len_rows) {
  KernelTimer timer("topk", st);
  if (k == d && !k_rows) {
    unsigned gx = (unsigned)ceil_div(k_pad, 256);
    if (gx > 1024) gx = 1024;
    hipLaunchKernelGGL(iota_kernel, dim3(gx, (unsigned)batch), dim3(256), 0, st, d, k_pad, idx);
    return hipGetLastError();
  }
  if (k_div < 1) k_div = 1;
  if (d <= 4096)
    hipLaunchKernelGGL((topk_kernel<true, 256>), dim3((unsigned)batch), dim3(256), 0, st, scores, d, k, k_pad, idx,
                       k_rows, len_rows, k_div);
  else if (d <= kLdsKeys)
    hipLaunchKernelGGL((topk_kernel<true, kMaxThreads>), dim3((unsigned)batch), dim3(kMaxThreads), 0, st, scores,
                       d, k, k_pad, idx, k_rows, len_rows, k_div);
  else
    hipLaunchKernelGGL((topk_kernel<false, kMaxThreads>), dim3((unsigned)batch), dim3(kMaxThreads), 0, st, scores,
                       d, k, k_pad, idx, k_rows, len_rows, k_div);
  return hipGetLastError();
}

}  // namespace rmm

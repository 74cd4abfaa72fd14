// Top-k selection of column scores ("Estrategia de Selección": keep the k
// indices with the highest scores), ties to the lower index, output ascending.
//
// One 1024-thread workgroup per batch row.  Scores are mapped to order-
// preserving unsigned keys and (for d up to kLdsKeys) parked in LDS.  The exact
// k-th largest key T is found by MSD radix select: the bits every key shares
// are skipped (found with a block OR/AND reduction), then <= 8-bit digits are
// histogrammed in LDS and a single wave locates the digit that holds the k-th
// key.  Emission is one ordered pass: each thread owns a contiguous index
// segment, counts its keys > T and == T, and two block-wide exclusive scans
// give every thread its output offset and how many of its == T keys it may
// take (the lowest-index ones win).  All integer work: the result is exact.
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsKeys = 32768;  // 128 KiB of keys; beyond that, keys are re-read from global

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix sum of one uint32 per thread; returns the block total in *total.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      uint32_t y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < kWaves) wsum[kWaves + lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  const uint32_t before = wave ? wsum[kWaves + wave - 1] : 0u;
  *total = wsum[2 * kWaves - 1];
  const uint32_t r = before + x - v;
  __syncthreads();
  return r;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float *__restrict__ scores, int64_t d,
                                                        int64_t k, int64_t k_pad,
                                                        int32_t *__restrict__ idx) {
  __shared__ uint32_t keys[IN_LDS ? kLdsKeys : 1];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[2 * kWaves];
  __shared__ uint32_t red_or[kWaves], red_and[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *s = scores + (int64_t)blockIdx.x * d;
  int32_t *out = idx + (int64_t)blockIdx.x * k_pad;
  auto key_at = [&](int64_t j) -> uint32_t {
    if constexpr (IN_LDS) return keys[j];
    else return score_key(s[j]);
  };

  // Load keys; OR/AND over all keys gives the bits every key shares.
  uint32_t kor = 0u, kand = 0xFFFFFFFFu;
  for (int64_t j = tid; j < d; j += kThreads) {
    const uint32_t key = score_key(s[j]);
    if constexpr (IN_LDS) keys[j] = key;
    kor |= key;
    kand &= key;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kor |= __shfl_xor(kor, off, 64);
    kand &= __shfl_xor(kand, off, 64);
  }
  if (lane == 0) {
    red_or[wave] = kor;
    red_and[wave] = kand;
  }
  __syncthreads();
  kor = 0u;
  kand = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kor |= red_or[w];
    kand &= red_and[w];
  }
  const uint32_t diff = kor ^ kand;
  // Bits at positions >= lo are known (equal to `prefix`) for the k-th key.
  int lo = diff ? 32 - __clz(diff) : 0;
  uint32_t prefix = lo >= 32 ? 0u : (kand & (0xFFFFFFFFu << lo));
  uint32_t krem = (uint32_t)k;  // rank of the wanted key among keys matching `prefix` above lo

  while (lo > 0) {
    const int width = lo < 8 ? lo : 8;
    const int shift = lo - width;
    const uint32_t hmask = lo >= 32 ? 0u : (0xFFFFFFFFu << lo);
    const uint32_t dmask = (1u << width) - 1u;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int64_t j = tid; j < d; j += kThreads) {
      const uint32_t key = key_at(j);
      if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l..4l+3; count keys in strictly higher bins.
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const uint32_t mine = h0 + h1 + h2 + h3;
      uint32_t suf = mine;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t y = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += y;
      }
      uint32_t above = suf - mine;  // keys in bins of higher lanes
      const uint32_t hb[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (above < krem && krem <= above + hb[q]) {
          sel_digit = (uint32_t)(4 * lane + q);
          sel_above = above;
        }
        above += hb[q];
      }
    }
    __syncthreads();
    krem -= sel_above;
    prefix |= sel_digit << shift;
    lo = shift;
    __syncthreads();
  }

  // prefix is now the k-th largest key T; krem of the keys equal to T are kept.
  const uint32_t T = prefix;
  const int64_t seg = (d + kThreads - 1) / kThreads;
  const int64_t j0 = (int64_t)tid * seg;
  const int64_t j1 = j0 + seg < d ? j0 + seg : d;
  uint32_t gt = 0u, eq = 0u;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan(eq, wsum, &tot);
  const uint32_t take_eq =
      krem > eq_before ? ((krem - eq_before) < eq ? (krem - eq_before) : eq) : 0u;
  const uint32_t pos0 = block_excl_scan(gt + take_eq, wsum, &tot);
  uint32_t pos = pos0, taken = 0u;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t key = key_at(j);
    if (key > T || (key == T && taken < take_eq)) {
      out[pos++] = (int32_t)j;
      taken += key == T;
    }
  }
  for (int64_t t = k + tid; t < k_pad; t += kThreads) out[t] = -1;
}

// k == d: every index is kept.
__global__ __launch_bounds__(256) void iota_kernel(int64_t d, int64_t k_pad, int32_t *idx) {
  int32_t *out = idx + (int64_t)blockIdx.y * k_pad;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < k_pad; t += (int64_t)gridDim.x * 256)
    out[t] = t < d ? (int32_t)t : -1;
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t batch, int64_t d, int64_t k, int64_t k_pad,
                       int32_t *idx, hipStream_t st) {
  KernelTimer timer("topk", st);
  if (k == d) {
    unsigned gx = (unsigned)ceil_div(k_pad, 256);
    if (gx > 1024) gx = 1024;
    hipLaunchKernelGGL(iota_kernel, dim3(gx, (unsigned)batch), dim3(256), 0, st, d, k_pad, idx);
    return hipGetLastError();
  }
  if (d <= kLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)batch), dim3(kThreads), 0, st, scores, d,
                       k, k_pad, idx);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)batch), dim3(kThreads), 0, st, scores,
                       d, k, k_pad, idx);
  return hipGetLastError();
}

}  // namespace rmm

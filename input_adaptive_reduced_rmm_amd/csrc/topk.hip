// Top-k selection of column scores ("Estrategia de Selección": keep the k
// indices with the highest scores), ties to the lower index, output ascending.
//
// One workgroup per batch row (1024 threads; 256 for rows of at most 4096).
// Scores are mapped to order-preserving unsigned keys and (for d up to
// kLdsKeys) parked in LDS.  The exact k-th largest key T is found by MSD
// radix select: the bits every key shares are skipped (found with a block
// OR/AND reduction), then <= 8-bit digits are histogrammed in LDS and a
// single wave locates the digit that holds the k-th key.  Two histograms
// alternate, so while that wave scans one the others clear the other, and a
// pass costs two barriers.  The select stops early when the digit's bin is
// needed whole (every key in it ranks within k): T is then the bin's lowest
// possible key and every key >= T is kept.  Emission walks the keys in index
// order, one contiguous run per wave: keys > T are kept, and of the keys == T
// the lowest-index ones up to the count still needed.  All integer work: the
// result is exact.
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kLdsKeys = 32768;  // 128 KiB of keys; beyond that, keys are re-read from global

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Set bits of a wave mask in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

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
  __shared__ uint32_t keys[IN_LDS ? (NT == 256 ? 4096 : kLdsKeys) : 1];
  // Long rows: kRep copies of the histogram, lane l adding to copy l % kRep
  // (padded to 257 words so the copies' bins sit in different banks): scores
  // that crowd into a few digits then collide kRep times less.
  constexpr int kRep = NT == 1024 ? 4 : 1;
  constexpr int kHist = kRep == 1 ? 256 : kRep * 257;
  __shared__ uint32_t hist[2][kHist];
  constexpr int kThreads = NT, kWaves = NT / 64;
  __shared__ uint32_t red_or[kWaves], red_and[kWaves];
  __shared__ uint32_t sel_digit, sel_above, sel_count;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  auto key_at = [&](int64_t j) -> uint32_t {
    if constexpr (IN_LDS) return keys[j];
    else return score_key(s[j]);
  };

  // Load keys; OR/AND over all keys gives the bits every key shares.
  // Eight loads per thread are issued before any is used, so the pass costs
  // about one memory latency per eight keys instead of one per key.
  uint32_t kor = 0u, kand = 0xFFFFFFFFu;
  for (int64_t j0 = tid; j0 < d; j0 += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + (int64_t)u * kThreads;
      v[u] = j < d ? s[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + (int64_t)u * kThreads;
      if (j < d) {
        const uint32_t key = score_key(v[u]);
        if constexpr (IN_LDS) keys[j] = key;
        kor |= key;
        kand &= key;
      }
    }
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
  for (int i = tid; i < kHist; i += kThreads) hist[0][i] = 0u;
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
  int hb_cur = 0;

  while (lo > 0) {
    const int width = lo < 8 ? lo : 8;
    const int shift = lo - width;
    const uint32_t hmask = lo >= 32 ? 0u : (0xFFFFFFFFu << lo);
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t *hist_c = hist[hb_cur];
    for (int64_t j0 = tid; j0 < d; j0 += 8 * kThreads) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * kThreads;
        kk[u] = j < d ? key_at(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * kThreads;
        if (j < d && (kk[u] & hmask) == prefix)
          atomicAdd(&hist_c[(kRep == 1 ? 0 : (lane % kRep) * 257) + ((kk[u] >> shift) & dmask)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l..4l+3; count keys in strictly higher bins.
      uint32_t h0 = 0u, h1 = 0u, h2 = 0u, h3 = 0u;
#pragma unroll
      for (int c = 0; c < kRep; ++c) {
        const uint32_t *hc = hist_c + (kRep == 1 ? 0 : c * 257);
        h0 += hc[4 * lane];
        h1 += hc[4 * lane + 1];
        h2 += hc[4 * lane + 2];
        h3 += hc[4 * lane + 3];
      }
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
          sel_count = hb[q];
        }
        above += hb[q];
      }
    } else {
      // the next pass's histogram, last read before this pass's first barrier
      uint32_t *hist_n = hist[hb_cur ^ 1];
      for (int i = tid - 64; i < kHist; i += kThreads - 64) hist_n[i] = 0u;
    }
    __syncthreads();
    // sel_* are written again only after two more barriers: no third one here
    krem -= sel_above;
    prefix |= sel_digit << shift;
    lo = shift;
    hb_cur ^= 1;
    if (krem == sel_count) {
      // every key of the bin ranks within k: keep all keys >= prefix
      krem = 0xFFFFFFFFu;
      break;
    }
  }

  // prefix is now T, the k-th largest key (or after an early stop the lowest
  // key of its bin); krem of the keys equal to T are kept (all after an early
  // stop).
  // Emission: each wave owns a contiguous run of indices and walks it 64 keys
  // at a time (lane = key, conflict-free LDS reads).  A counting walk gives
  // each wave its kept keys; the waves' output offsets and shares of the keys
  // equal to T follow in index order; a second walk writes every kept index
  // at its slot (ballot + lane prefix count), so the output is ascending.
  const uint32_t T = prefix;
  const int64_t per_wave = ((d + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t w0 = (int64_t)wave * per_wave;
  const int64_t w1 = w0 + per_wave < d ? w0 + per_wave : d;
  // Both walks read eight 64-key chunks before using any (one LDS latency per
  // eight chunks instead of one per chunk).
  constexpr int U = 8;
  uint32_t gt = 0u, eq = 0u;
  for (int64_t c0 = w0; c0 < w1; c0 += 64 * U) {
    uint32_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = c0 + 64 * u + lane;
      kk[u] = j < w1 ? key_at(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = c0 + 64 * u + lane < w1;
      gt += valid && kk[u] > T;
      eq += valid && kk[u] == T;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off, 64);
    eq += __shfl_xor(eq, off, 64);
  }
  __syncthreads();   // the wave arrays (last read before the first pass) are reused below
  if (lane == 0) {
    red_or[wave] = gt;
    red_and[wave] = eq;
  }
  __syncthreads();
  uint32_t my_take = 0u, my_pos = 0u;
  {
    uint32_t eq_acc = 0u, pos_acc = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t g_w = red_or[w], e_w = red_and[w];
      const uint32_t take = krem > eq_acc ? ((krem - eq_acc) < e_w ? (krem - eq_acc) : e_w) : 0u;
      if (w == wave) {
        my_take = take;
        my_pos = pos_acc;
      }
      eq_acc += e_w;
      pos_acc += g_w + take;
    }
  }
  uint32_t eq_seen = 0u, kept_seen = 0u;
  for (int64_t c0 = w0; c0 < w1; c0 += 64 * U) {
    uint32_t kk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = c0 + 64 * u + lane;
      kk[u] = j < w1 ? key_at(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = c0 + 64 * u + lane;
      const bool valid = j < w1;
      const bool is_eq = valid && kk[u] == T;
      const uint64_t eqm = __ballot(is_eq);
      const uint32_t eq_rank = eq_seen + lanes_below(eqm);
      const bool keep = valid && (kk[u] > T || (is_eq && eq_rank < my_take));
      const uint64_t km = __ballot(keep);
      if (keep) out[my_pos + kept_seen + lanes_below(km)] = (int32_t)j;
      eq_seen += (uint32_t)__popcll(eqm);
      kept_seen += (uint32_t)__popcll(km);
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

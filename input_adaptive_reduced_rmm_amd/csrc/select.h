// Exact top-k selection on order-preserving integer keys ("Estrategia de
// Selección": keep the k indices with the highest scores), ties to the lower
// index, kept indices written in ascending order.  Shared by the top-k kernel
// and by kernels that compute their scores and select in the same launch.
//
// block_select: one workgroup, any row length.  The k-th largest key T is
// found by MSD radix select: the bits every key shares are skipped (from a
// block OR/AND reduction), then <= 8-bit digits are histogrammed in LDS and
// one wave locates the digit that holds the k-th key.  Two histograms
// alternate, so while that wave scans one the others clear the other, and a
// pass costs two barriers.  The select stops early when the digit's bin is
// needed whole (every key in it ranks within k): T is then the bin's lowest
// possible key and every key >= T is kept.  Emission walks the keys in index
// order, one contiguous run per wave: keys > T are kept, and of the keys == T
// the lowest-index ones up to the count still needed.
//
// wave_select128: one wave, 128 keys (two per lane), for head-dimension
// feature sets: T by a bitwise search on ballot counts, then the same
// emission rule.  All integer work: both results are exact.
#pragma once

#include "rmm_internal.h"

namespace rmm {
namespace sel {

// Order-preserving key of a float score (-0.0 ranks as +0.0).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Set bits of a wave mask in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// LDS of block_select for NT threads.  Long rows: kRep copies of each
// histogram, lane l adding to copy l % kRep (padded to 257 words so the
// copies' bins sit in different banks): scores that crowd into a few digits
// then collide kRep times less.
template <int NT>
struct BlockShared {
  static constexpr int kRep = NT == 1024 ? 4 : 1;
  static constexpr int kHist = kRep == 1 ? 256 : kRep * 257;
  static constexpr int kWaves = NT / 64;
  uint32_t hist[2][kHist];
  uint32_t red_or[kWaves], red_and[kWaves];
  uint32_t sel_digit, sel_above, sel_count;
};

// Top-k of the row's d keys, key_at(j) giving key j; writes the k kept
// indices ascending to out[0, k) and -1 to out[k, k_pad).  kor / kand: this
// thread's OR and AND over the keys it produced (any split of the row over
// the threads).  Every thread of the workgroup calls it; a barrier at its
// start publishes what the caller wrote to LDS before the call.
template <int NT, typename KeyAt>
__device__ __forceinline__ void block_select(KeyAt key_at, int64_t d, uint32_t kor, uint32_t kand, int64_t k,
                                             int64_t k_pad, int32_t *__restrict__ out, BlockShared<NT> &sh) {
  constexpr int kRep = BlockShared<NT>::kRep, kHist = BlockShared<NT>::kHist, kWaves = BlockShared<NT>::kWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kor |= __shfl_xor(kor, off, 64);
    kand &= __shfl_xor(kand, off, 64);
  }
  if (lane == 0) {
    sh.red_or[wave] = kor;
    sh.red_and[wave] = kand;
  }
  for (int i = tid; i < kHist; i += NT) sh.hist[0][i] = 0u;
  __syncthreads();
  kor = 0u;
  kand = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kor |= sh.red_or[w];
    kand &= sh.red_and[w];
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
    uint32_t *hist_c = sh.hist[hb_cur];
    uint32_t *hist_l = hist_c + (kRep == 1 ? 0 : (lane % kRep) * 257);
    // eight keys read before any is used
    for (int64_t j0 = tid; j0 < d; j0 += 8 * NT) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * NT;
        kk[u] = j < d ? key_at(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + (int64_t)u * NT;
        if (j < d && (kk[u] & hmask) == prefix) atomicAdd(&hist_l[(kk[u] >> shift) & dmask], 1u);
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
          sh.sel_digit = (uint32_t)(4 * lane + q);
          sh.sel_above = above;
          sh.sel_count = hb[q];
        }
        above += hb[q];
      }
    } else {
      // the next pass's histogram, last read before this pass's first barrier
      uint32_t *hist_n = sh.hist[hb_cur ^ 1];
      for (int i = tid - 64; i < kHist; i += NT - 64) hist_n[i] = 0u;
    }
    __syncthreads();
    // sel_* are written again only after two more barriers: no third one here
    krem -= sh.sel_above;
    prefix |= sh.sel_digit << shift;
    lo = shift;
    hb_cur ^= 1;
    if (krem == sh.sel_count) {
      // every key of the bin ranks within k: keep all keys >= prefix
      krem = 0xFFFFFFFFu;
      break;
    }
  }

  // prefix is now T, the k-th largest key (or after an early stop the lowest
  // key of its bin); krem of the keys equal to T are kept (all after an early
  // stop).  Each wave owns a contiguous run of indices and walks it 64 keys
  // at a time (lane = key): a counting walk gives each wave its kept keys;
  // the waves' output offsets and shares of the keys equal to T follow in
  // index order; a second walk writes every kept index at its slot (ballot +
  // lane prefix count), so the output is ascending.
  const uint32_t T = prefix;
  const int64_t per_wave = ((d + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t w0 = (int64_t)wave * per_wave;
  const int64_t w1 = w0 + per_wave < d ? w0 + per_wave : d;
  // Both walks read eight 64-key chunks before using any.
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
    sh.red_or[wave] = gt;
    sh.red_and[wave] = eq;
  }
  __syncthreads();
  uint32_t my_take = 0u, my_pos = 0u;
  {
    uint32_t eq_acc = 0u, pos_acc = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t g_w = sh.red_or[w], e_w = sh.red_and[w];
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
  for (int64_t t = k + tid; t < k_pad; t += NT) out[t] = -1;
}

// Top-k of 128 keys held by one wave, lane l holding keys l (k0) and l + 64
// (k1); 1 <= k <= 128.  Writes the kept indices ascending to out[0, k) and -1
// to out[k, k_pad) (k_pad <= 128).  T = the largest value with at least k
// keys >= it, found bit by bit from the top.
__device__ __forceinline__ void wave_select128(uint32_t k0, uint32_t k1, int k, int k_pad, int32_t *out) {
  const int lane = threadIdx.x & 63;
  uint32_t T = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = T | (1u << b);
    const int c = __popcll(__ballot(k0 >= t)) + __popcll(__ballot(k1 >= t));
    if (c >= k) T = t;
  }
  const int gt = __popcll(__ballot(k0 > T)) + __popcll(__ballot(k1 > T));
  const int take = k - gt;   // keys equal to T kept, lowest index first
  const uint64_t e0 = __ballot(k0 == T), e1 = __ballot(k1 == T);
  const int r0 = (int)lanes_below(e0), r1 = __popcll(e0) + (int)lanes_below(e1);
  const bool keep0 = k0 > T || (k0 == T && r0 < take);
  const bool keep1 = k1 > T || (k1 == T && r1 < take);
  const uint64_t m0 = __ballot(keep0), m1 = __ballot(keep1);
  if (keep0) out[lanes_below(m0)] = lane;
  if (keep1) out[__popcll(m0) + (int)lanes_below(m1)] = 64 + lane;
  if (k + lane < k_pad) out[k + lane] = -1;
  if (k + 64 + lane < k_pad) out[k + 64 + lane] = -1;
}

}  // namespace sel
}  // namespace rmm

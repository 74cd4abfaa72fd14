// Token-reduced attention output O_h = P_h[:, J_h] V_g[J_h, :] ("Alcance de
// Aplicación": optionally reduce the token dimension of P V).
//
// P V is bound by reading P from HBM, and P's rows are token-contiguous.  On
// this layout a column gather cannot save bytes at cache-line granularity
// (a 128-byte line holds 64 tokens), so the product works at that granularity
// instead of packing: a small plan kernel turns each head's kept-token list
// into the ascending list of 64-token tiles that hold at least one kept token,
// each with a 64-bit keep mask.  The MFMA core (mfma_gemm.h, kMaskedTiles)
// then streams, for its block of query rows, only those tiles of P, zeroes
// the dropped tokens in both P and V while staging, and multiplies.  Dropped
// tokens contribute exact zeros and tiles without a kept token are never
// read: the result is exactly the reduced product, with P read once at line
// granularity and no packed copy written.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kMaxTiles = 8192;  // 64-bit masks in LDS: Lk <= 524288

// One block per head: keep masks of every 64-token tile, then the ascending
// list of tiles with a nonzero mask.
__global__ __launch_bounds__(kPlanThreads) void pv_plan_kernel(const int32_t *__restrict__ idx,
                                                               int64_t idx_stride, int64_t k,
                                                               int64_t Lk, int64_t ntiles,
                                                               int32_t *__restrict__ tiles,
                                                               uint64_t *__restrict__ masks,
                                                               int32_t *__restrict__ counts) {
  __shared__ unsigned long long m[kMaxTiles];
  __shared__ uint32_t wsum[2 * kPlanWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t h = blockIdx.x;
  const int32_t *ib = idx + h * idx_stride;
  for (int64_t t = tid; t < ntiles; t += kPlanThreads) m[t] = 0ull;
  __syncthreads();
  for (int64_t t = tid; t < k; t += kPlanThreads) {
    const int32_t j = ib[t];
    if (j >= 0 && j < Lk) atomicOr(&m[j >> 6], 1ull << (j & 63));
  }
  __syncthreads();
  const int64_t seg = (ntiles + kPlanThreads - 1) / kPlanThreads;
  const int64_t t0 = tid * seg, t1 = t0 + seg < ntiles ? t0 + seg : ntiles;
  uint32_t cnt = 0;
  for (int64_t t = t0; t < t1; ++t) cnt += m[t] != 0ull;
  // block exclusive scan of cnt
  uint32_t x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kPlanWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kPlanWaves; off <<= 1) {
      uint32_t y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < kPlanWaves) wsum[kPlanWaves + lane] = w;
  }
  __syncthreads();
  uint32_t pos = (wave ? wsum[kPlanWaves + wave - 1] : 0u) + x - cnt;
  int32_t *tb = tiles + h * ntiles;
  uint64_t *mb = masks + h * ntiles;
  for (int64_t t = t0; t < t1; ++t) {
    if (m[t] != 0ull) {
      tb[pos] = (int32_t)t;
      mb[pos] = m[t];
      ++pos;
    }
  }
  if (tid == 0) counts[h] = (int32_t)wsum[2 * kPlanWaves - 1];
}

}  // namespace

int64_t pv_max_tokens() { return (int64_t)kMaxTiles * 64; }

size_t pv_plan_bytes(int64_t hq, int64_t Lk) {
  const int64_t nt = ceil_div(Lk, 64);
  return align_up((size_t)hq * nt * 4, 256) + align_up((size_t)hq * nt * 8, 256) + align_up((size_t)hq * 4, 256);
}

hipError_t launch_pv(const void *P, int64_t ldp, int64_t p_hs, const void *V, int64_t v_ts,
                     int64_t v_hs, void *O, int64_t o_ts, int64_t o_hs, const int32_t *idx,
                     int64_t idx_stride, int64_t k, int64_t hq, int64_t hkv, int64_t Lq, int64_t Lk,
                     int64_t dh, bool causal, void *plan_ws, hipStream_t st) {
  const int64_t nt = ceil_div(Lk, 64);
  char *w = static_cast<char *>(plan_ws);
  int32_t *tiles = reinterpret_cast<int32_t *>(w);
  uint64_t *masks = reinterpret_cast<uint64_t *>(w + align_up((size_t)hq * nt * 4, 256));
  int32_t *counts = reinterpret_cast<int32_t *>(w + align_up((size_t)hq * nt * 4, 256) +
                                                align_up((size_t)hq * nt * 8, 256));
  {
    KernelTimer timer("pv_plan", st);
    hipLaunchKernelGGL(pv_plan_kernel, dim3((unsigned)hq), dim3(kPlanThreads), 0, st, idx, idx_stride,
                       k, Lk, nt, tiles, masks, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#ifndef RMM_PV_BM
#define RMM_PV_BM 128
#endif
#ifndef RMM_PV_STAGES
#define RMM_PV_STAGES 2
#endif
  constexpr int BM = RMM_PV_BM, BN = 128, STG = RMM_PV_STAGES;
  mg::Args a{};
  a.A = static_cast<const uint16_t *>(P);
  a.lda = ldp;
  a.a_bs = p_hs;
  a.a_cols = Lk;
  a.B = static_cast<const uint16_t *>(V);
  a.ldb = v_ts;
  a.b_bs = v_hs;
  a.tiles = tiles;
  a.masks = masks;
  a.counts = counts;
  a.ntiles = nt;
  a.Y = O;
  a.ldy = o_ts;
  a.y_bs = o_hs;
  a.batch = hq;
  a.hq = hq;
  a.hkv = hkv;
  a.m = Lq;
  a.n = dh;
  a.d = Lk;
  a.tiles_m = ceil_div(Lq, BM);
  a.tiles_n = ceil_div(dh, BN);
  a.causal = causal ? 1 : 0;
  a.causal_off = Lk - Lq;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)hq);
  KernelTimer timer("pv_gemm", st);
  const bool avec = reinterpret_cast<uintptr_t>(P) % 16 == 0 && ldp % 8 == 0 && p_hs % 8 == 0;
  const bool bvec = reinterpret_cast<uintptr_t>(V) % 16 == 0 && v_ts % 8 == 0 && v_hs % 8 == 0;
  if (avec && bvec)
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, mg::kMaskedTiles, uint16_t, STG, true, true>), grid, dim3(256), 0,
                       st, a);
  else if (avec)
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, mg::kMaskedTiles, uint16_t, STG, true, false>), grid, dim3(256), 0,
                       st, a);
  else if (bvec)
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, mg::kMaskedTiles, uint16_t, STG, false, true>), grid, dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, mg::kMaskedTiles, uint16_t, STG, false, false>), grid, dim3(256),
                       0, st, a);
  return hipGetLastError();
}

bool pv_layout_ok(const void *, int64_t ldp, int64_t, const void *, int64_t v_ts, int64_t,
                  int64_t Lk, int64_t dh) {
  return (uint64_t)(255 * ldp + Lk) * 2 < mg::kMaxRecords &&
         (uint64_t)((Lk - 1) * v_ts + dh) * 2 < mg::kMaxRecords;
}

}  // namespace rmm

// Token-reduced attention output O_h = P_h[:, J_h] V_g[J_h, :] ("Alcance de
// Aplicación": optionally reduce the token dimension of P V).
//
// P V is bound by reading P from HBM, and P's rows are token-contiguous.  On
// this layout a column gather cannot save bytes at cache-line granularity
// (a 128-byte line holds 64 tokens), so the product works at that granularity
// instead of packing: a small plan kernel turns each head's kept-token list
// into the ascending list of 64-token tiles that hold at least one kept token,
// each with a 64-bit keep mask.  The MFMA kernel below then streams, for its
// block of query rows, only those tiles of P, zeroes the dropped tokens in
// both P and V while staging, and multiplies.  Dropped
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


struct PvArgs {
  const uint16_t *P;       // [hq] x [Lq rows of ldp]
  int64_t ldp, p_hs;
  const uint16_t *V;       // [Lk tokens of v_ts] x [hkv of v_hs]
  int64_t v_ts, v_hs;
  uint16_t *O;             // [Lq tokens of o_ts] x [hq of o_hs]
  int64_t o_ts, o_hs;
  const int32_t *tiles;    // [hq][ntiles] ascending 64-token tiles with a kept token
  const uint64_t *masks;   // keep mask of each listed tile
  const int32_t *counts;   // listed tiles per head
  int64_t ntiles, hq, hkv, Lq, Lk, dh;
  int64_t tiles_m, tiles_n;
  int causal;
  int64_t coff;            // causal: token j is visible from query row i when j <= i + coff
};

constexpr int kBN = 128;     // output columns per block (head_dim 128 in one tile)
constexpr int kEpiPitch = kBN + 8;

// Reduced P V for one (row block, column block, head).  The 64-token tiles of
// the head's list are streamed PD ahead of the MFMA: the registers hold the
// loads of tiles q+1 .. q+PD while tile q is multiplied from LDS, so each
// block keeps PD tiles of P (PD x BM x 128 B) in flight.  Dropped tokens are zeroed
// in both the P tile and the V rows (their V rows are not even loaded), and
// on tiles that straddle the causal diagonal the entries above it are zeroed
// per row, so the values stored there are never used.
// Calls f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>) in order.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void template_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    template_for<N, I + 1>(f);
  }
}

template <int BM, int PD, bool AVEC, bool BVEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void pv_kernel(PvArgs g) {
  constexpr int WTM = BM / 2;                 // wave tile rows (2 x 2 waves)
  constexpr int TM = WTM / 32, TN = 2;        // 32 x 32 MFMA tiles per wave
  constexpr int A_CH = BM / 32;               // 16-byte P chunks per thread per tile
  constexpr int KB = 4;                       // V rows per thread per tile (x 8 columns)
  constexpr int NB = kBN / 8;                 // threads across a V row
  constexpr int kStage = (BM + kBN) * mg::kBK;
  static_assert(BM * kEpiPitch <= 2 * kStage, "epilogue staging must fit the operand buffers");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Block order: rounds of one row block over every (head, column block); in
  // causal mode the heaviest row blocks (the most tiles) come first across all
  // heads, so the lightest ones fill the tail.  Within a round, workgroups are
  // dealt round-robin to the 8 XCDs: give each XCD a contiguous run of heads,
  // i.e. whole KV groups, so its L2 holds the V rows of few groups.
  const int64_t per_round = g.hq * g.tiles_n;
  const int64_t rnd = (int64_t)blockIdx.x / per_round, w = (int64_t)blockIdx.x % per_round;
  const int64_t hw = per_round % 8 == 0 ? (w % 8) * (per_round / 8) + w / 8 : w;
  const int64_t h = hw / g.tiles_n, tn = hw % g.tiles_n;
  const int64_t tm = g.causal ? g.tiles_m - 1 - rnd : rnd;
  const int64_t m0 = tm * BM, n0 = tn * kBN;
  const int64_t grp = (h * g.hkv) / g.hq;
  const int64_t rows = g.Lq - m0 < BM ? g.Lq - m0 : BM;

  const uint16_t *Pb = g.P + h * g.p_hs + m0 * g.ldp;
  const mg::rsrc_t rp = mg::make_rsrc(Pb, ((uint64_t)(rows - 1) * g.ldp + g.Lk) * 2);
  const uint16_t *Vb = g.V + grp * g.v_hs + n0;
  const mg::rsrc_t rv = mg::make_rsrc(Vb, ((uint64_t)(g.Lk - 1) * g.v_ts + (g.dh - n0)) * 2);

  const int akc = tid & 7;                    // P chunk column within a tile
  const int bnb = tid % NB, bkb = tid / NB;   // V block: tokens bkb*KB.., columns bnb*8..
  const int32_t *tl = g.tiles + h * g.ntiles;
  const uint64_t *ml = g.masks + h * g.ntiles;
  int nk = g.counts[h];
  if (g.causal) {
    // keep the listed tiles that start at or before the block's last visible column
    const int64_t last_col = m0 + rows - 1 + g.coff;
    int lo = 0, hi = nk;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)tl[mid] * mg::kBK <= last_col) lo = mid + 1;
      else hi = mid;
    }
    nk = lo;
  }

  uint4 ra[PD][A_CH], rb[PD][KB];
  uint64_t mk[PD];
  int64_t cc[PD];

  // Loads of listed tile q into register slot S (no use of the data here).
  auto issue = [&](auto slot, int q) {
    constexpr int S = decltype(slot)::value;
    const uint64_t m = ml[q];
    const int64_t c0 = (int64_t)tl[q] * mg::kBK;
    mk[S] = m;
    cc[S] = c0;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      ra[S][i] = mg::load_chunk<AVEC, mg::kCached>(rp, (uint32_t)(((int64_t)row * g.ldp + c0 + akc * 8) * 2));
    }
#pragma unroll
    for (int r = 0; r < KB; ++r) {
      const int t = bkb * KB + r;
      const uint32_t off = ((m >> t) & 1ull) ? (uint32_t)(((c0 + t) * g.v_ts + bnb * 8) * 2) : mg::kOOB;
      rb[S][r] = mg::load_chunk<BVEC>(rv, off);
    }
  };

  // Mask register slot S and write it into LDS buffer S.
  auto stage = [&](auto slot, auto buf) {
    constexpr int S = decltype(slot)::value;
    uint16_t *As = smem + decltype(buf)::value * kStage;
    uint16_t *Bs = As + BM * mg::kBK;
    const uint64_t m = mk[S];
    const int64_t c0 = cc[S];
    const bool diag = g.causal && c0 + mg::kBK - 1 > m0 + g.coff;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      uint32_t bits = (uint32_t)(m >> (akc * 8)) & 0xFFu;
      if (diag) {
        // columns c0 + akc*8 + e are visible only while <= m0 + row + coff
        const int64_t allow = m0 + row + g.coff - (c0 + akc * 8) + 1;
        bits &= allow >= 8 ? 0xFFu : allow <= 0 ? 0u : ((1u << allow) - 1u);
      }
      *reinterpret_cast<uint4 *>(&As[mg::swz(row, akc)]) = mg::mask8(ra[S][i], bits);
    }
    // 4 tokens x 8 columns per thread -> each column gets an 8-byte half K-run.
    const int kc = bkb >> 1, half = (bkb & 1) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = mg::u4get(rb[S][r], q);
      const uint2 ev = make_uint2((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16));
      const uint2 od = make_uint2((w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u));
      const int n_ev = bnb * 8 + 2 * q;
      *reinterpret_cast<uint2 *>(&Bs[mg::swz(n_ev, kc) + half]) = ev;
      *reinterpret_cast<uint2 *>(&Bs[mg::swz(n_ev + 1, kc) + half]) = od;
    }
  };

  mg::f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lk = lane >> 5;
  auto mma = [&](auto buf) {
    const uint16_t *As = smem + decltype(buf)::value * kStage;
    const uint16_t *Bs = As + BM * mg::kBK;
#pragma unroll
    for (int ks = 0; ks < mg::kBK / 16; ++ks) {
      mg::bf16x8_t av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        av[i] = __builtin_bit_cast(mg::bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                      &As[mg::swz(wm * WTM + i * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = __builtin_bit_cast(mg::bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                      &Bs[mg::swz(wn * 64 + j * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };

  // Tile q sits in LDS buffer q % 2; register slots (q + 1) % PD .. (q + PD - 1) % PD
  // hold tiles q + 1 .. q + PD - 1 in flight, and slot q % PD is free.  The
  // loop is unrolled by 2 PD so that every slot and buffer index is static.
  auto step = [&](auto qm, int q) {
    constexpr int QM = decltype(qm)::value;
    using Free = std::integral_constant<int, QM % PD>;
    using Next = std::integral_constant<int, (QM + 1) % PD>;
    using Buf = std::integral_constant<int, QM % 2>;
    using NBuf = std::integral_constant<int, (QM + 1) % 2>;
    if (q + PD < nk) issue(Free{}, q + PD);
    mma(Buf{});
    if (q + 1 < nk) stage(Next{}, NBuf{});
    __syncthreads();
  };
  template_for<PD>([&](auto p) {
    if (decltype(p)::value < nk) issue(p, decltype(p)::value);
  });
  if (nk > 0) {
    stage(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    __syncthreads();
  }
  for (int q = 0; q < nk; q += 2 * PD) {
    template_for<2 * PD>([&](auto qm) {
      if (q + decltype(qm)::value < nk) step(qm, q + decltype(qm)::value);
    });
  }

  // Epilogue: bf16 tile through LDS (the operand buffers are free after the
  // loop's last barrier), then 16-byte row segments.  D of a 32x32 tile:
  // lane l holds column l%32; register r holds row 8*(r/4) + 4*(l/32) + r%4.
  uint16_t *E = smem;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        E[row * kEpiPitch + wn * 64 + j * 32 + lrow] = f32_to_bf16(acc[i][j][r]);
      }
  __syncthreads();
  uint16_t *Oh = g.O + h * g.o_hs;
  const int cch = tid & 15;                  // 16-byte chunk of a 128-column row
  const int64_t col = n0 + cch * 8;
  const bool vec = col + 8 <= g.dh && g.o_ts % 8 == 0 && g.o_hs % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(g.O) % 16 == 0;
#pragma unroll
  for (int it = 0; it < BM / 16; ++it) {
    const int row = it * 16 + (tid >> 4);
    if (row >= rows) break;
    const uint16_t *src = &E[row * kEpiPitch + cch * 8];
    uint16_t *dst = Oh + (m0 + row) * g.o_ts + col;
    if (vec) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < g.dh) dst[e] = src[e];
    }
  }
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
  constexpr int BM = 128, PD = 2;
  PvArgs a{};
  a.P = static_cast<const uint16_t *>(P);
  a.ldp = ldp;
  a.p_hs = p_hs;
  a.V = static_cast<const uint16_t *>(V);
  a.v_ts = v_ts;
  a.v_hs = v_hs;
  a.O = static_cast<uint16_t *>(O);
  a.o_ts = o_ts;
  a.o_hs = o_hs;
  a.tiles = tiles;
  a.masks = masks;
  a.counts = counts;
  a.ntiles = nt;
  a.hq = hq;
  a.hkv = hkv;
  a.Lq = Lq;
  a.Lk = Lk;
  a.dh = dh;
  a.tiles_m = ceil_div(Lq, BM);
  a.tiles_n = ceil_div(dh, kBN);
  a.causal = causal ? 1 : 0;
  a.coff = Lk - Lq;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n * hq));
  KernelTimer timer("pv_gemm", st);
  const bool avec = reinterpret_cast<uintptr_t>(P) % 16 == 0 && ldp % 8 == 0 && p_hs % 8 == 0;
  const bool bvec = reinterpret_cast<uintptr_t>(V) % 16 == 0 && v_ts % 8 == 0 && v_hs % 8 == 0;
  if (avec && bvec)
    hipLaunchKernelGGL((pv_kernel<BM, PD, true, true>), grid, dim3(256), 0, st, a);
  else if (avec)
    hipLaunchKernelGGL((pv_kernel<BM, PD, true, false>), grid, dim3(256), 0, st, a);
  else if (bvec)
    hipLaunchKernelGGL((pv_kernel<BM, PD, false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((pv_kernel<BM, PD, false, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

bool pv_layout_ok(const void *, int64_t ldp, int64_t, const void *, int64_t v_ts, int64_t,
                  int64_t Lk, int64_t dh) {
  return (uint64_t)(255 * ldp + Lk) * 2 < mg::kMaxRecords &&
         (uint64_t)((Lk - 1) * v_ts + dh) * 2 < mg::kMaxRecords;
}

}  // namespace rmm

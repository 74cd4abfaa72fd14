// Feature-reduced attention scores S_h = Q_h[:, I_h] Kt_g[I_h, :] ("Alcance de
// Aplicación": reduce the feature dimension of Q K^T), float32 output.
//
// The product is bound by writing S (Lq x Lk floats per head) to HBM; its K
// depth is only k_pad <= 128 (one or two 64-wide tiles).  A 128 x 128 output
// tile is little work next to its 64 KiB of stores, so one workgroup per tile
// makes the launch limited by workgroup dispatch.  This kernel is persistent
// instead: a grid of a few workgroups per CU walks the list of output tiles,
// and in causal mode the list holds only the tiles that reach the lower
// triangle (u <= t + Lk - Lq), enumerated in closed form, so the skipped half
// costs nothing.  Per tile: the packed Q_I rows and the kept rows Kt[I, :]
// are loaded with range-checked buffer loads, Kt rows are transposed in
// registers into K-contiguous LDS runs, v_mfma_f32_32x32x16_bf16 multiplies,
// and the fp32 tile is written with non-temporal stores.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

using mg::bf16x8_t;
using mg::f32x16_t;
using mg::rsrc_t;

constexpr int kT = 128;  // output tile (rows and columns)

struct QkArgs {
  const uint16_t *A;      // packed Q_I [Hq][Lq][k_pad]
  const int32_t *idx;     // cleaned [Hq][k_pad]
  const uint16_t *Kt;     // [Hkv] x [dh rows of ldkt]
  int64_t kt_hs, ldkt;
  float *S;
  int64_t s_hs, lds;
  int64_t hq, hkv, Lq, Lk, dh, k_pad;
  int64_t tiles_m, tiles_n;
  int64_t c0;             // tiles in row r: clamp(r + c0, 0, tiles_n)
  int64_t per_head;       // tiles per head
  int64_t total;          // per_head * hq
};

// Number of tiles in rows [0, x): sum of clamp(r + c0, 0, T).
__host__ __device__ __forceinline__ int64_t tiles_before(int64_t x, int64_t c0, int64_t T) {
  const int64_t a0 = 1 - c0 > 0 ? 1 - c0 : 0;      // rows below a0 hold no tile
  const int64_t a1 = T - c0 > a0 ? T - c0 : a0;    // rows from a1 on hold T tiles
  int64_t s = 0;
  const int64_t q = x < a1 ? x : a1;
  if (q > a0) s += (q - a0) * (a0 + q - 1) / 2 + (q - a0) * c0;
  if (x > a1) s += (x - a1) * T;
  return s;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kPitch = 68;                                  // staging row pitch (floats)
constexpr int kOperandBytes = 2 * kT * mg::kBK * 2;        // A and B tiles
constexpr int kStageBytes = 4 * 32 * kPitch * 4;           // 4 waves x 32 rows
constexpr int kSmemBytes = kOperandBytes > kStageBytes ? kOperandBytes : kStageBytes;

// Resident workgroups per CU (four waves each; the register count allows two).
constexpr int kQkBlocksPerCu = 2;

// BSTORE: S is written with buffer stores whose resource drops rows past Lq
// and whose offsets drop columns past Lk, so every tile issues the same number
// of stores on every path (no branch around them).  The next tile's loads go
// out before them, and the wait for those loads then leaves this tile's stores
// in flight (one counter tracks loads and stores in issue order) instead of
// draining them before the next tile's product.  Needs 32 rows of S within one
// resource (4 GiB), 16-byte aligned rows and Lk % 4 == 0.
template <bool BVEC, bool BSTORE>
__global__ __launch_bounds__(256) void qk_persistent(QkArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
  uint16_t *As = reinterpret_cast<uint16_t *>(smem);
  uint16_t *Bs = As + kT * mg::kBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: store resources stay scalar
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, lk = lane >> 5;
  const int akc = tid & 7;
  const int bnb = tid & 15, bkb = tid >> 4;   // B block: k rows bkb*4.., columns bnb*8..
  const int nk = (int)(g.k_pad / mg::kBK);

  struct Tile {
    int64_t h, m0, n0, grp, rows;
  };
  auto tile_at = [&](int64_t t) -> Tile {
    Tile ti;
    ti.h = t / g.per_head;
    const int64_t loc = t - ti.h * g.per_head;
    // row of tiles holding `loc`: largest tm with tiles_before(tm) <= loc
    int64_t lo = 0, hi = g.tiles_m - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (tiles_before(mid, g.c0, g.tiles_n) <= loc) lo = mid;
      else hi = mid - 1;
    }
    ti.m0 = lo * kT;
    ti.n0 = (loc - tiles_before(lo, g.c0, g.tiles_n)) * kT;
    ti.grp = (ti.h * g.hkv) / g.hq;
    ti.rows = g.Lq - ti.m0 < kT ? g.Lq - ti.m0 : kT;
    return ti;
  };

  uint4 ra4[4], rb4[4];
  // Issue the loads of K tile q of output tile `ti` into ra4/rb4.
  auto issue = [&](const Tile &ti, int q) {
    const int64_t c0 = (int64_t)q * mg::kBK;
    const rsrc_t ra = mg::make_rsrc(g.A + (ti.h * g.Lq + ti.m0) * g.k_pad, (uint64_t)ti.rows * g.k_pad * 2);
    const rsrc_t rb = mg::make_rsrc(g.Kt + ti.grp * g.kt_hs + ti.n0,
                                    ((uint64_t)(g.dh - 1) * g.ldkt + (g.Lk - ti.n0)) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      ra4[i] = mg::bload16(ra, (uint32_t)(((int64_t)row * g.k_pad + c0 + akc * 8) * 2));
    }
    const int4 src = *reinterpret_cast<const int4 *>(g.idx + ti.h * g.k_pad + c0 + bkb * 4);
    const int32_t s4[4] = {src.x, src.y, src.z, src.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t off = s4[r] >= 0 ? (uint32_t)(((int64_t)s4[r] * g.ldkt + bnb * 8) * 2) : mg::kOOB;
      rb4[r] = mg::load_chunk<BVEC>(rb, off);
    }
  };

  // Workgroups are dealt round-robin to the 8 XCDs.  The grid walks the tile
  // list in rounds of gridDim.x consecutive tiles; within a round, give each
  // XCD a contiguous run (gridDim.x / 8 tiles of mostly one row) so that its
  // L2 serves the Q_I rows and kept K rows those tiles share.
  const int64_t t_step = gridDim.x, t_end = g.total;
  int64_t t = blockIdx.x;
  if (gridDim.x % 8 == 0) t = (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  Tile cur = tile_at(t < t_end ? t : 0);
  if (t < t_end) {
    issue(cur, 0);
    if constexpr (BSTORE) {
      // Dropped stores (empty resource): the loop is entered with the same
      // count of stores behind the first loads as every later tile, so the
      // wait at its top is for the loads only.
      const rsrc_t none = mg::make_rsrc(g.S, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) __builtin_amdgcn_raw_buffer_store_b32(0, none, (int)mg::kOOB - 64 * q, 0, 0);
    }
  }
  for (; t < t_end; t += t_step) {
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int q = 0; q < nk; ++q) {
      if (q > 0) issue(cur, q);
      __syncthreads();   // previous users of the LDS (operands or staging) are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        *reinterpret_cast<uint4 *>(&As[mg::swz(row, akc)]) = ra4[i];
      }
      {
        const int kc = bkb >> 1, half = (bkb & 1) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = mg::u4get(rb4[r], e);
          const uint2 ev = make_uint2((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16));
          const uint2 od = make_uint2((w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u));
          const int n_ev = bnb * 8 + 2 * e;
          *reinterpret_cast<uint2 *>(&Bs[mg::swz(n_ev, kc) + half]) = ev;
          *reinterpret_cast<uint2 *>(&Bs[mg::swz(n_ev + 1, kc) + half]) = od;
        }
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < mg::kBK / 16; ++ks) {
        bf16x8_t av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          av[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                    &As[mg::swz(wm * 64 + i * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bv[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                    &Bs[mg::swz(wn * 64 + j * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    // Prefetch the next output tile's first K tile before this tile's stores:
    // on this architecture one counter tracks loads and stores in issue order,
    // so loads issued after the stores would also wait for them.
    const Tile ti = cur;
    const bool more = t + t_step < t_end;
    if (more) cur = tile_at(t + t_step);
    if (more) issue(cur, 0);
    __syncthreads();   // every wave is done reading the operand tiles

    // Epilogue through LDS: each wave parks 32 x 64 floats of its tile at a
    // time (row pitch 68 floats keeps the column-strided writes and the
    // row-wise reads on distinct banks), then writes them back as 16-byte
    // row segments: one store instruction covers 4 rows x 256 bytes.
    float *Sh = g.S + ti.h * g.s_hs;
    float *stage = reinterpret_cast<float *>(smem) + wave * (32 * kPitch);
    const bool full_cols = ti.n0 + kT <= g.Lk && (g.lds % 4 == 0) &&
                           (reinterpret_cast<uintptr_t>(Sh) % 16 == 0);
    // lane part of a store offset: row lane/16 of a 4-row group, 4 columns
    const uint32_t vo = (uint32_t)(((lane >> 4) * g.lds + (lane & 15) * 4) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stage[(8 * (r >> 2) + 4 * lk + (r & 3)) * kPitch + j * 32 + lrow] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      const int64_t rbase = ti.m0 + wm * 64 + i * 32;
      const int64_t cbase = ti.n0 + wn * 64;
      if constexpr (BSTORE) {
        // Resource over this wave's 32 x 64 block: rows past Lq and, in the
        // last row, columns past Lk fall outside it; a 4-column group past Lk
        // in other rows gets an offset outside it (Lk % 4 == 0 here).
        const int64_t rows = g.Lq - rbase < 32 ? g.Lq - rbase : 32;
        const int64_t ncols = g.Lk - cbase < 64 ? g.Lk - cbase : 64;
        const rsrc_t rs = mg::make_rsrc(Sh + rbase * g.lds + cbase,
                                        rows > 0 && ncols > 0 ? ((uint64_t)(rows - 1) * g.lds + ncols) * 4 : 0);
        const bool col_ok = (lane & 15) * 4 < ncols;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t *>(&stage[(it * 4 + (lane >> 4)) * kPitch +
                                                                       (lane & 15) * 4]);
          const uint32_t off = col_ok ? vo + (uint32_t)(it * 4 * g.lds * 4) : mg::kOOB;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), rs, (int)off, 0, 2 /* nt */);
        }
        __builtin_amdgcn_wave_barrier();
        continue;
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rr = it * 4 + (lane >> 4);
        const int cc = (lane & 15) * 4;
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(&stage[rr * kPitch + cc]);
        const int64_t row = rbase + rr;
        if (row < g.Lq) {
          float *dst = Sh + row * g.lds + cbase + cc;
          if (full_cols) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(dst));
          } else {
            const float e4[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (cbase + cc + q < g.Lk) dst[q] = e4[q];
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace

bool qk_layout_ok(int64_t Lq, int64_t dh, int64_t ldkt, int64_t Lk, int64_t k_pad) {
  return (uint64_t)kT * k_pad * 2 < mg::kMaxRecords &&
         (uint64_t)((dh - 1) * ldkt + Lk) * 2 < mg::kMaxRecords && Lq > 0;
}

namespace {
// The tile list of one head: tiles_m rows of 128-query tiles, row r holding
// column tiles 0 .. clamp(r + c0, 0, tiles_n) - 1, per_head tiles in all.
struct QkTiles {
  int64_t tiles_m, tiles_n, c0, per_head;
  bool ok;   // the closed form agrees with the direct sum
};
QkTiles qk_tiles(int64_t Lq, int64_t Lk, bool causal) {
  QkTiles t;
  t.tiles_m = ceil_div(Lq, kT);
  t.tiles_n = ceil_div(Lk, kT);
  if (causal) {
    // row r of tiles spans rows r*128 .. r*128+127; it needs columns up to
    // r*128 + 127 + (Lk - Lq), i.e. tiles 0 .. r + floor((127 + off) / 128).
    const int64_t off = Lk - Lq;
    const int64_t num = kT - 1 + off;
    const int64_t fl = num >= 0 ? num / kT : -((-num + kT - 1) / kT);
    t.c0 = 1 + fl;
  } else {
    t.c0 = t.tiles_n;  // every row holds all tiles
  }
  // The kernel locates tiles with the closed form; cross-check it against the
  // direct sum.
  int64_t direct = 0;
  for (int64_t r = 0; r < t.tiles_m; ++r) {
    const int64_t c = r + t.c0;
    direct += c < 0 ? 0 : (c > t.tiles_n ? t.tiles_n : c);
  }
  t.per_head = tiles_before(t.tiles_m, t.c0, t.tiles_n);
  t.ok = t.per_head == direct;
  return t;
}
}  // namespace

bool qk_tiles_ok(int64_t Lq, int64_t Lk, bool causal) { return Lq > 0 && Lk > 0 && qk_tiles(Lq, Lk, causal).ok; }

hipError_t launch_qk(const void *Apacked, const int32_t *idx_clean, const void *Kt, int64_t kt_hs,
                     int64_t ldkt, float *S, int64_t s_hs, int64_t lds, int64_t hq, int64_t hkv,
                     int64_t Lq, int64_t Lk, int64_t dh, int64_t k_pad, bool causal, hipStream_t st) {
  QkArgs g;
  g.A = static_cast<const uint16_t *>(Apacked);
  g.idx = idx_clean;
  g.Kt = static_cast<const uint16_t *>(Kt);
  g.kt_hs = kt_hs;
  g.ldkt = ldkt;
  g.S = S;
  g.s_hs = s_hs;
  g.lds = lds;
  g.hq = hq;
  g.hkv = hkv;
  g.Lq = Lq;
  g.Lk = Lk;
  g.dh = dh;
  g.k_pad = k_pad;
  const QkTiles t = qk_tiles(Lq, Lk, causal);   // rmm_qk has checked t.ok before any launch
  g.tiles_m = t.tiles_m;
  g.tiles_n = t.tiles_n;
  g.c0 = t.c0;
  g.per_head = t.per_head;
  g.total = g.per_head * hq;
  if (g.total == 0) return hipSuccess;
  const bool bvec = reinterpret_cast<uintptr_t>(Kt) % 16 == 0 && ldkt % 8 == 0 && kt_hs % 8 == 0;
  // Stores left in flight pay off when a tile has two K tiles (k_pad = 128:
  // 4.10 -> 3.80 ms for 32 heads x 16384^2 causal); with one K tile, letting
  // them drain at the next tile's first wait measured faster (3.02 against
  // 3.29 ms at k_pad = 64).
  const bool bstore = k_pad > mg::kBK && reinterpret_cast<uintptr_t>(S) % 16 == 0 && lds % 4 == 0 &&
                      s_hs % 4 == 0 && Lk % 4 == 0 && (uint64_t)32 * lds * 4 < mg::kMaxRecords;
  int64_t grid = 256 * kQkBlocksPerCu;
  if (grid > g.total) grid = g.total;
  KernelTimer timer("qk_gemm", st);
  const dim3 gr((unsigned)grid), blk(256);
  if (bvec && bstore) hipLaunchKernelGGL((qk_persistent<true, true>), gr, blk, 0, st, g);
  else if (bvec) hipLaunchKernelGGL((qk_persistent<true, false>), gr, blk, 0, st, g);
  else if (bstore) hipLaunchKernelGGL((qk_persistent<false, true>), gr, blk, 0, st, g);
  else hipLaunchKernelGGL((qk_persistent<false, false>), gr, blk, 0, st, g);
  return hipGetLastError();
}

}  // namespace rmm

// Reduced projection GEMM for many rows: Y = A_I B_I with both operands packed
// K-contiguous ("Mecanismo Central": A_{:,I} B_{I,:}).
//
// When m is large the product is MFMA-bound and the weight slice B_I is
// re-read by every row tile, so it pays to lay it out once for the matrix
// cores: `bt_pack` writes B_I^T[n][t] = B[idx[t], n] (zero for padding
// slots) into the workspace, the same way A_I is packed.  The weights
// themselves are only read.  Both operand tiles then come straight from
// memory into LDS with `buffer_load_dwordx4 ... lds` (no staging registers,
// no in-loop transposes), which leaves the register file to the accumulators
// and to double-buffered MFMA fragments.
//
// Block tile 256 x 256 x 64, eight waves of 128 x 64 (two per SIMD), two LDS
// stages (128 KiB).  LDS rows hold 64 bf16 with the 16-byte chunk index
// XOR-swizzled by the row; since one direct load writes 64 consecutive
// 16-byte LDS chunks, each lane fetches the global chunk that the swizzle maps
// onto its LDS slot.  The MFMA takes the B fragment as its first operand so
// each lane ends up with four consecutive output columns of one row.  The
// epilogue passes the tile through the remaining 32 KiB of LDS, 64 rows at a
// time, and writes whole 512-byte rows with 16-byte stores.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

#define LDS_AS __attribute__((address_space(3)))

namespace rmm {
namespace {

using mg::bf16x8_t;
using mg::f32x16_t;
using mg::rsrc_t;

constexpr int kBK = 64;   // slot granularity of the packed operands

// ---------------------------------------------------------------- B_I^T pack
// grid: x = 256-wide column block of B, y = 64-wide block of kept slots.
// Each thread loads an 8 (slots) x 8 (columns) block, transposes it in
// registers into eight 16-byte K-runs, parks them in LDS as [n][64], and the
// block then writes 256 rows of 128 contiguous bytes.
// grid.z = batch entry b (several packs in one launch): it reads B group
// floor(b * hkv / hq) (group stride b_gs), index row b and writes BT entry b.
struct BtBatch {
  int64_t hq, hkv, b_gs, idx_bs, bt_bs;
};
template <bool BVEC>
__global__ __launch_bounds__(256) void bt_pack_kernel(const uint16_t *__restrict__ B, int64_t ldb,
                                                      int64_t d, int64_t n,
                                                      const int32_t *__restrict__ idx_clean,
                                                      int64_t k_pad, uint16_t *__restrict__ BT, BtBatch bb) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[256 * kBK];
  const int tid = threadIdx.x;
  {
    const int64_t b = blockIdx.z;
    B += (b * bb.hkv / bb.hq) * bb.b_gs;
    idx_clean += b * bb.idx_bs;
    BT += b * bb.bt_bs;
  }
  const int64_t n0 = (int64_t)blockIdx.x * 256;
  const int64_t t0 = (int64_t)blockIdx.y * kBK;
  const int nb = tid & 31, tb = tid >> 5;          // columns nb*8.., slots tb*8..
  const rsrc_t rb = mg::make_rsrc(B + n0, ((uint64_t)(d - 1) * ldb + (n - n0)) * 2);
  const int4 s0 = *reinterpret_cast<const int4 *>(idx_clean + t0 + tb * 8);
  const int4 s1 = *reinterpret_cast<const int4 *>(idx_clean + t0 + tb * 8 + 4);
  const int32_t src[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint4 r[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t off = src[q] >= 0 ? (uint32_t)(((int64_t)src[q] * ldb + nb * 8) * 2) : mg::kOOB;
    r[q] = mg::load_chunk<BVEC>(rb, off);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = mg::u4get(r[q], e);
    const uint4 ev = make_uint4((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16),
                                (w[4] & 0xFFFFu) | (w[5] << 16), (w[6] & 0xFFFFu) | (w[7] << 16));
    const uint4 od = make_uint4((w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u),
                                (w[4] >> 16) | (w[5] & 0xFFFF0000u), (w[6] >> 16) | (w[7] & 0xFFFF0000u));
    const int nr = nb * 8 + 2 * e;
    *reinterpret_cast<uint4 *>(&tile[mg::swz(nr, tb)]) = ev;
    *reinterpret_cast<uint4 *>(&tile[mg::swz(nr + 1, tb)]) = od;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, kc = c & 7;
    if (n0 + row < n)
      *reinterpret_cast<uint4 *>(BT + (n0 + row) * k_pad + t0 + kc * 8) =
          *reinterpret_cast<const uint4 *>(&tile[mg::swz(row, kc)]);
  }
}

// ---------------------------------------------------------------- GEMM
struct NtArgs {
  const uint16_t *A;   // [m][k_pad]
  const uint16_t *BT;  // [n][k_pad]
  uint16_t *Y;
  int64_t ldy, m, n, k_pad, tiles_m, tiles_n;
  float *ypart;        // optional [2 tiles_m][n]: column sums of squares of the bf16 Y per 128-row slab
  int y_stream;        // Y larger than the memory-side cache: non-temporal stores
};

// LDS operand tiles are [256 rows][64] bf16: 8 16-byte chunks per row, the
// chunk index XOR-swizzled by (row ^ row/8) & 7 so that the 32 consecutive
// rows an MFMA fragment read touches spread over the banks.

// 16 bytes per lane from the buffer straight into LDS: the wave's 64 lanes
// fill the 1 KiB at `lds` in lane order.  (A plain function, so that the
// kernel templates stay instantiable in the host compilation pass.)
__device__ __forceinline__ void lds_load16(rsrc_t r, unsigned char *lds, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)lds, 16, voff, soff, 0, 0);
}

// Immediate of s_waitcnt vmcnt(n) with lgkmcnt and expcnt left alone:
// vmcnt[3:0] | vmcnt[5:4] << 14.
constexpr int vm_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

// 256 x 256 x 64 tiles, two LDS stages, persistent: one workgroup per CU
// walks its XCD's tile range.  After the last K-step's barrier (every wave is
// done reading LDS) it issues the first two K-tiles of its next output tile,
// and only then converts and stores the finished accumulators, so the next
// tile's loads fly while the epilogue runs and the pipeline never drains
// between tiles.  The stores come after those loads in issue order, so
// waiting for the loads does not wait for them.
//
// Epilogue.  Straight from the accumulators, one store instruction would put
// 16 bytes into each of 32 rows: every CU finishing a tile at about the same
// time then sends millions of small writes to L2, and the next tile's second
// K-step waits behind them (about 10 us per round of tiles).  Instead, for
// each of the four 32-row groups of every wave, the eight waves write their
// 32 x 64 pieces (rows of both 128-row slabs) into a 64 x 256 staging area in
// the LDS left over by the operand stages, and the workgroup writes the area
// out as whole 512-byte rows: 16 stores per wave, each covering two rows.
// A Y larger than the memory-side cache is stored non-temporally: the kernel
// that reads it next could not find it there anyway.
//
// Register budget: the accumulators take half the register file, so the rest
// must hold only fragments and a few addresses.  The LDS fragment addresses
// are built by hand: with the XOR swizzle, the byte offset of fragment (i, ks)
// of a lane is rowbase + 4096 i + 16 (e ^ c), with e a per-lane constant and
// c = 2 ks ^ 4 (i & 1) one of four compile-time values, plus the stage offset.
// Eight base registers thus address every fragment read through ds_read's
// immediate offset; they pass through an empty asm each step so the compiler
// cannot hoist one register per (fragment, stage) out of the loop.
//
// WGN: waves across the tile's columns (2: four waves of 128 x 128, one per
// SIMD; 4: eight waves of 128 x 64, two per SIMD, so that one wave's MFMAs
// run while the other waits on LDS or on the barrier: about 10 % faster).
// SCORED: also write the per-slab column sums of squares of Y (g.ypart).
template <int WGN, bool SCORED>
__global__ __launch_bounds__(128 * WGN) __attribute__((amdgpu_waves_per_eu(WGN / 2))) void gemm_nt_persistent(
    NtArgs g) {
  constexpr int BM = 256, BN = 256, BK = 64, NST = 2;
  constexpr int NWAVE = 2 * WGN;
  constexpr int WTN = BN / WGN;                      // wave tile columns (rows: 128)
  constexpr int TI = 4, TJ = WTN / 32;
  constexpr int TILE = 256 * BK * 2;                 // one operand tile, 32 KiB
  constexpr int LPW = 32 / NWAVE;                    // direct loads per wave per operand
  constexpr int KS = BK / 16;
  constexpr int EPI = 64 * BN * 2;                   // epilogue staging: 64 rows of the tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NST * TILE + EPI];   // [A0 | A1 | B0 | B1 | E]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lrow = lane & 31, lk = lane >> 5;
  const int64_t total = g.tiles_m * g.tiles_n;
  const int nk = (int)(g.k_pad / BK);

  // Direct load i of this wave writes the 1 KiB LDS block q = NWAVE i + wave:
  // rows 8 q + lane/8, slot lane%8, holding logical chunk slot ^ f(row) with
  // f(row) = (row ^ row/8) & 7 = (lane/8) ^ ((NWAVE i + wave) & 7).  The lane
  // part of the byte offset depends on i at most through i & 1; the rest
  // (8 NWAVE i rows and the K offset) is uniform and goes in the scalar offset.
  uint32_t vbase[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int logical = (lane & 7) ^ (lane >> 3) ^ ((wave + NWAVE * p) & 7);
    vbase[p] = (uint32_t)((((int64_t)wave * 8 + (lane >> 3)) * g.k_pad + logical * 8) * 2);
  }
  const uint32_t srow = (uint32_t)(8 * NWAVE * g.k_pad * 2);   // bytes of 8 NWAVE rows

  // Fragment read bases (see above): row lrow of the wave's row slab, chunk
  // e ^ c for c = 0, 2, 4, 6.
  const int e = lk ^ (lrow & 7) ^ (lrow >> 3);
  uint32_t fa[4], fb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t off = (uint32_t)(lrow * 128 + ((e ^ (2 * c)) << 4));
    fa[c] = off + (uint32_t)(wm * 128 * 128);
    fb[c] = off + (uint32_t)(NST * TILE + wn * WTN * 128);
  }

  struct Ctx {
    int64_t m0, n0;
    rsrc_t ra, rb;
  };
  auto ctx_of = [&](int64_t w) __attribute__((always_inline)) {
    uint32_t tm, tn;
    mg::tile_of32((uint32_t)w, (uint32_t)g.tiles_m, (uint32_t)g.tiles_n, tm, tn);
    Ctx c;
    c.m0 = (int64_t)tm * BM;
    c.n0 = (int64_t)tn * BN;
    const int64_t rows = g.m - c.m0 < BM ? g.m - c.m0 : BM;
    const int64_t cols = g.n - c.n0 < BN ? g.n - c.n0 : BN;
    c.ra = mg::make_rsrc(g.A + c.m0 * g.k_pad, (uint64_t)rows * g.k_pad * 2);
    c.rb = mg::make_rsrc(g.BT + c.n0 * g.k_pad, (uint64_t)cols * g.k_pad * 2);
    return c;
  };
  auto issue = [&](const Ctx &c, int kt, int stage) __attribute__((always_inline)) {
    unsigned char *sa = smem + stage * TILE;
    unsigned char *sb = smem + (NST + stage) * TILE;
    const uint32_t koff = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      lds_load16(c.ra, sa + (NWAVE * i + wave) * 1024, vbase[i & 1], i * srow + koff);
      lds_load16(c.rb, sb + (NWAVE * i + wave) * 1024, vbase[i & 1], i * srow + koff);
    }
  };
  auto prologue = [&](const Ctx &c) __attribute__((always_inline)) {
    issue(c, 0, 0);
    if (nk > 1) issue(c, 1, 1);
  };

  f32x16_t acc[TJ][TI];
  bf16x8_t av[2][TI], bv[2][TJ];
  // Fragments of K-slice ks of the tile at LDS byte offset `so` (its stage)
  // into register slot `slot`.
  auto frags = [&](uint32_t so, int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int c = ((2 * ks) ^ (4 * (i & 1))) >> 1;
      av[slot][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                     smem + (fa[c] + so) + i * 4096));
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int c = ((2 * ks) ^ (4 * (j & 1))) >> 1;
      bv[slot][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                     smem + (fb[c] + so) + j * 4096));
    }
  };
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int i = 0; i < TI; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[slot][j], av[slot][i], acc[j][i], 0, 0, 0);
  };

  int64_t w = blockIdx.x;
  if (w >= total) return;
  Ctx cur = ctx_of(w);
  prologue(cur);
  // Stores this wave issued after the current tile's first two K-tiles (the
  // previous tile's epilogue): kStLds on the staged path, kStReg on the
  // register path of a partial column tile; on the element path the waits
  // below count none.  vmcnt holds at most 63.
  constexpr int kStLds = 4 * TI, kStReg = TI * TJ * 4;
  static_assert(2 * LPW + kStReg <= 63, "store count exceeds vmcnt");
  int nstores = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
    // K-tile 0 landed: K-tile 1 (if any) and then the previous tile's stores
    // were issued after it.
    if (nk > 1) {
      if (nstores == kStLds) __builtin_amdgcn_s_waitcnt(vm_imm(2 * LPW + kStLds));
      else if (nstores == kStReg) __builtin_amdgcn_s_waitcnt(vm_imm(2 * LPW + kStReg));
      else __builtin_amdgcn_s_waitcnt(vm_imm(2 * LPW));
    } else {
      if (nstores == kStLds) __builtin_amdgcn_s_waitcnt(vm_imm(kStLds));
      else if (nstores == kStReg) __builtin_amdgcn_s_waitcnt(vm_imm(kStReg));
      else __builtin_amdgcn_s_waitcnt(vm_imm(0));
    }
    // A bare barrier: every wave's part of K-tile 0 is in LDS.  (__syncthreads
    // would also make each wave wait for its previous tile's stores.)
    __builtin_amdgcn_s_barrier();
    frags(0, 0, 0);

    // One K-step on K-tile kt (stage kt & 1).  ISSUE: refill this stage with
    // K-tile kt+2 after the barrier.  LAST: no next K-tile to wait for.
    auto step = [&](int kt, auto issue_flag, auto last_flag) __attribute__((always_inline)) {
      constexpr bool ISSUE = decltype(issue_flag)::value;
      constexpr bool LAST = decltype(last_flag)::value;
#pragma unroll
      for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(fa[c]), "+v"(fb[c]));
      const uint32_t so = (uint32_t)(kt & 1) * TILE;
      __builtin_amdgcn_iglp_opt(1);   // interleave fragment reads with the MFMAs
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
        frags(so, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1);
      }
      if constexpr (!LAST) {
        // K-tile kt+1 landed.  On the first step only the previous tile's
        // stores can follow it.
        if (kt == 0 && nstores == kStLds) __builtin_amdgcn_s_waitcnt(vm_imm(kStLds));
        else if (kt == 0 && nstores == kStReg) __builtin_amdgcn_s_waitcnt(vm_imm(kStReg));
        else __builtin_amdgcn_s_waitcnt(vm_imm(0));
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this tile's fragment reads are done
      __builtin_amdgcn_s_barrier();
      if constexpr (ISSUE) {
        issue(cur, kt + NST, kt & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!LAST) frags(TILE - so, 0, 0);
      mfmas((KS - 1) & 1);
    };
    int kt = 0;
    for (; kt + NST < nk; ++kt) step(kt, std::true_type{}, std::false_type{});
    for (; kt + 1 < nk; ++kt) step(kt, std::false_type{}, std::false_type{});
    step(kt, std::false_type{}, std::true_type{});

    // Next tile's first K-tiles go out before this tile's stores.
    const int64_t dm0 = cur.m0, dn0 = cur.n0;
    w += gridDim.x;
    const bool more = w < total;
    if (more) {
      cur = ctx_of(w);
      prologue(cur);
    }

    // Producer-fused column scores of Y (optional): the squares of the bf16
    // values this wave stores, summed over its 128 rows (its four rows per
    // lane, then the 32 lanes of each half in a fixed butterfly), one partial
    // per (128-row slab, column); colnorm_finish adds the slabs in order.
    // Rows past m were multiplied from zero rows of A and add nothing.
    if constexpr (SCORED) {
      float cs[TJ][16];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = 0.f;
#pragma unroll
          for (int i = 0; i < TI; ++i) {
            const float v = __uint_as_float((uint32_t)f32_to_bf16(acc[j][i][r]) << 16);
            t = fmaf(v, v, t);
          }
          cs[j][r] = t;
        }
#pragma unroll
      for (int off = 1; off < 32; off <<= 1)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) cs[j][r] += __shfl_xor(cs[j][r], off, 64);
      if ((lane & 31) == 0) {
        float *pr = g.ypart + (dm0 / 128 + wm) * g.n;
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t col = dn0 + wn * WTN + j * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
            if (col < g.n) pr[col] = cs[j][r];
          }
      }
    }

    // Epilogue: lane l of acc[j][i] holds four consecutive columns
    // j*32 + 8*(r/4) + 4*(l/32) of row i*32 + l%32 of the wave's 128-row slab.
    const int64_t rbase = dm0 + wm * 128, cbase = dn0 + wn * WTN;
    // Opaque copies of the lane's row and half: keeps the per-store address
    // arithmetic below inside the loop (folded into immediate offsets)
    // instead of 64 hoisted registers.
    int er = lrow, ek = lk;
    asm volatile("" : "+v"(er), "+v"(ek));
    nstores = 0;
    // Staged path, for tiles whose 256 columns all lie inside Y (the same
    // for every wave of the workgroup, which meets at the barriers below).
    // Staging row s = 32 wm + l%32 holds row wm*128 + i*32 + l%32 of the
    // tile; its 16-byte chunk c sits at slot c ^ (s % 32), so the 32 rows a
    // write instruction touches and the 32 chunks of a row a read touches
    // spread over the banks.  Rows past m fall outside the store resource
    // and are dropped.
    const bool staged = dn0 + BN <= g.n && g.ldy % 8 == 0 && reinterpret_cast<uintptr_t>(g.Y) % 16 == 0 &&
                        (uint64_t)BM * g.ldy * 2 < mg::kMaxRecords;
    // Register path (partial column tiles): 8-byte buffer stores, one lane
    // offset, the column step in the immediate and the 32-row step in the
    // scalar offset.
    const bool vec = (g.ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(g.Y) % 8 == 0) && cbase + WTN <= g.n &&
                     (uint64_t)128 * g.ldy * 2 < mg::kMaxRecords;
    if (staged) {
      typedef int v4i __attribute__((ext_vector_type(4)));
      unsigned char *E = smem + 2 * NST * TILE;
      const int64_t rows_valid = g.m - dm0 < BM ? g.m - dm0 : BM;
      const rsrc_t ry = mg::make_rsrc(g.Y + dm0 * g.ldy + dn0, (uint64_t)((rows_valid - 1) * g.ldy + BN) * 2);
      // LDS byte addresses of the staging area.  Its writes and reads are
      // issued from assembly: the compiler cannot tell them apart from the
      // next tile's direct loads into the operand stages (still in flight)
      // and would otherwise wait for those loads first.  The writes are
      // complete at the lgkmcnt(0) before the barrier; the reads wait for
      // their data inside the same assembly block.
      const uint32_t ebase = (uint32_t)(uintptr_t)(LDS_AS unsigned char *)E;
      const uint32_t wrow = ebase + (uint32_t)((wm * 32 + er) * (BN * 2));
      constexpr int RQ = 64 * BN / 8 / (64 * NWAVE);   // 16-byte chunks each thread copies out per row group
      static_assert(RQ == 4, "the read-out below issues four reads");
      uint32_t raddr[RQ];
      int rtrow[RQ], rch[RQ];
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        const int c = tid + 64 * NWAVE * q;
        const int sr = c / (BN / 8), ch = c % (BN / 8);
        raddr[q] = ebase + (uint32_t)(sr * (BN * 2) + ((ch ^ (sr & 31)) << 4));
        rtrow[q] = (sr >> 5) * 128 + (sr & 31);
        rch[q] = ch;
      }
      typedef unsigned v2u __attribute__((ext_vector_type(2)));
      typedef unsigned v4u __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const uint32_t lo = pack_bf16x2(acc[j][i][4 * gq + 0], acc[j][i][4 * gq + 1]);
            const uint32_t hi = pack_bf16x2(acc[j][i][4 * gq + 2], acc[j][i][4 * gq + 3]);
            const int c = wn * (WTN / 8) + j * 4 + gq;
            const uint32_t a = wrow + (uint32_t)((c ^ er) << 4) + 8u * (uint32_t)ek;
            asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v2u{lo, hi}) : "memory");
          }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's part is in LDS
        __builtin_amdgcn_s_barrier();
        v4u v[RQ];
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %5\n\t"
            "ds_read_b128 %2, %6\n\t"
            "ds_read_b128 %3, %7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
            : "v"(raddr[0]), "v"(raddr[1]), "v"(raddr[2]), "v"(raddr[3])
            : "memory");
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          const int trow = rtrow[q] + i * 32;
          const int off = (int)(((int64_t)trow * g.ldy + rch[q] * 8) * 2);
          if (g.y_stream) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v[q]), ry, off, 0, 2);
          else __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v[q]), ry, off, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's reads of the area are done
        __builtin_amdgcn_s_barrier();
      }
      nstores = kStLds;
    } else if (vec) {
      const int64_t rows_left = g.m - rbase;
      if (rows_left > 0) {
        const rsrc_t ry = mg::make_rsrc(g.Y + rbase * g.ldy + cbase,
                                        (uint64_t)((rows_left < 128 ? rows_left : 128) - 1) * g.ldy * 2 + WTN * 2);
        const uint32_t vo = (uint32_t)((er * g.ldy + 4 * ek) * 2);
        const uint32_t s32 = (uint32_t)(32 * g.ldy * 2);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const uint32_t lo = pack_bf16x2(acc[j][i][4 * gq + 0], acc[j][i][4 * gq + 1]);
              const uint32_t hi = pack_bf16x2(acc[j][i][4 * gq + 2], acc[j][i][4 * gq + 3]);
              typedef int v2i __attribute__((ext_vector_type(2)));
              __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)lo, (int)hi}, ry, (int)(vo + (j * 32 + 8 * gq) * 2),
                                                    (int)(i * s32), 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        nstores = kStReg;
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t row = rbase + i * 32 + er;
        uint16_t *yr = g.Y + row * g.ldy;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int64_t col = cbase + j * 32 + 8 * gq + 4 * ek;
            const uint32_t lo = pack_bf16x2(acc[j][i][4 * gq + 0], acc[j][i][4 * gq + 1]);
            const uint32_t hi = pack_bf16x2(acc[j][i][4 * gq + 2], acc[j][i][4 * gq + 3]);
            const uint16_t ev[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
            if (row < g.m) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (col + q < g.n) yr[col + q] = ev[q];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (!more) break;
  }
}


constexpr int kWGN = 4;

}  // namespace

size_t gemm_nt_bt_bytes(int64_t n, int64_t k_pad) { return align_up((size_t)n * k_pad * 2, 256); }

bool gemm_nt_ok(int64_t m, int64_t n, int64_t d, int64_t ldb, int64_t k_pad) {
  return m >= 1024 && (uint64_t)256 * k_pad * 2 < mg::kMaxRecords &&
         (uint64_t)((d - 1) * ldb + n) * 2 < mg::kMaxRecords;
}

hipError_t launch_bt_pack(const void *B, int64_t ldb, int64_t d, int64_t n, const int32_t *idx_clean,
                          int64_t k_pad, void *BT, int64_t batch, int64_t hq, int64_t hkv, int64_t b_gs,
                          int64_t idx_bs, int64_t bt_bs, hipStream_t st) {
  const bool bvec = reinterpret_cast<uintptr_t>(B) % 16 == 0 && ldb % 8 == 0 && b_gs % 8 == 0;
  dim3 grid((unsigned)ceil_div(n, 256), (unsigned)(k_pad / kBK), (unsigned)batch);
  const BtBatch bb{hq, hkv, b_gs, idx_bs, bt_bs};
  if (bvec)
    hipLaunchKernelGGL(bt_pack_kernel<true>, grid, dim3(256), 0, st, static_cast<const uint16_t *>(B), ldb, d, n,
                       idx_clean, k_pad, static_cast<uint16_t *>(BT), bb);
  else
    hipLaunchKernelGGL(bt_pack_kernel<false>, grid, dim3(256), 0, st, static_cast<const uint16_t *>(B), ldb, d, n,
                       idx_clean, k_pad, static_cast<uint16_t *>(BT), bb);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const void *A_packed, const int32_t *idx_clean, const void *B, int64_t ldb,
                          int64_t d, void *BT_ws, void *Y, int64_t ldy, int64_t m, int64_t n,
                          int64_t k_pad, hipStream_t st, float *y_scores, float *ypart) {
  {
    KernelTimer timer("bt_pack", st);
    hipError_t e = launch_bt_pack(B, ldb, d, n, idx_clean, k_pad, BT_ws, 1, 1, 1, 0, 0, 0, st);
    if (e != hipSuccess) return e;
  }
  NtArgs g;
  g.A = static_cast<const uint16_t *>(A_packed);
  g.BT = static_cast<const uint16_t *>(BT_ws);
  g.Y = static_cast<uint16_t *>(Y);
  g.ldy = ldy;
  g.m = m;
  g.n = n;
  g.k_pad = k_pad;
  g.tiles_m = ceil_div(m, 256);
  g.tiles_n = ceil_div(n, 256);
  g.ypart = y_scores ? ypart : nullptr;
  g.y_stream = (double)m * (double)n * 2.0 > kStreamBytes;
  {
    KernelTimer timer("gemm_nt", st);
    const int64_t tiles = g.tiles_m * g.tiles_n;
    const int64_t grid = tiles < 256 ? tiles : 256;
    if (g.ypart)
      hipLaunchKernelGGL((gemm_nt_persistent<kWGN, true>), dim3((unsigned)grid), dim3(128 * kWGN), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_nt_persistent<kWGN, false>), dim3((unsigned)grid), dim3(128 * kWGN), 0, st, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !y_scores) return e;
  }
  return launch_colnorm_finish(ypart, 2 * g.tiles_m, n, y_scores, st);
}

size_t gemm_nt_ypart_bytes(int64_t m, int64_t n) { return align_up((size_t)2 * ceil_div(m, 256) * n * 4, 256); }

}  // namespace rmm

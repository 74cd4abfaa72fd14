// Shared bf16 MFMA GEMM core for the reduced products, and the buffer-load,
// swizzle and masking helpers the other MFMA kernels use.
//
// Y[b] = A_b[:, I] * B_g(b)[I, :], float32 accumulation, on
// v_mfma_f32_32x32x16_bf16.  A is the packed kept-column slice [m][k_pad]
// (K-contiguous); K-tile q covers packed columns 64q..64q+63, and B row t of
// the tile is B[idx[t], :] with idx a cleaned index list (-1 = contributes
// zero).
//
// Memory access: every global load is a raw buffer load whose resource covers
// exactly the bytes the block may touch, so rows past the matrix end and the
// "contributes zero" rows (offset pushed past the range) read as zero with no
// branch.  The loop issues the next K-tile's loads, multiplies the current
// tile from LDS, then transposes/masks the loaded registers into the other
// LDS stage: the only waits on global loads are right before that store.  B
// is row-major (N-contiguous) in memory and must be K-contiguous per lane for
// the MFMA, so each thread loads an (BN/32) x 8 block and transposes it in
// registers before writing K-runs to LDS.  LDS rows are 64 bf16 (128 B) with
// the 16-byte chunk index XOR-swizzled by the row so that the row-strided
// MFMA operand reads spread over the banks.
#pragma once

#include <type_traits>

#include "rmm_internal.h"

namespace rmm {
namespace mg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBK = 64;
constexpr uint32_t kOOB = 0xFFFFFFF0u;       // offset that always falls outside a resource
constexpr uint64_t kMaxRecords = 0xFFFFFF00ull;

struct Args {
  const uint16_t *A;
  int64_t lda, a_bs;            // A row stride, batch stride (elements)
  const uint16_t *B;
  int64_t ldb, b_bs;            // B row stride, kv-group stride
  const int32_t *idx;           // cleaned [batch][k_pad]
  int64_t idx_bs;
  void *Y;
  int64_t ldy, y_bs;
  int64_t batch, hq, hkv;       // batch entry b reads B group floor(b*hkv/hq)
  int64_t m, n, d;              // d = rows of B
  int64_t k_pad;
  int64_t tiles_m, tiles_n;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint64_t bytes) {
  const uint32_t nr = (uint32_t)(bytes < kMaxRecords ? bytes : kMaxRecords);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nr, 0x00020000);
}

// Cache policy of a buffer load: kNonTemporal streams data that is read once
// and is far larger than the caches.
constexpr int kCached = 0, kNonTemporal = 2;

template <int POL = kCached>
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL));
}

// Eight 2-byte loads assembled into one 16-byte chunk (layouts whose rows are
// not 16-byte aligned); each element is range-checked like the wide load.
template <int POL = kCached>
__device__ __forceinline__ uint4 bload16_e(rsrc_t r, uint32_t off) {
  uint32_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    e[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)(off + 2u * q), 0, POL);
  return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

template <bool VEC, int POL = kCached>
__device__ __forceinline__ uint4 load_chunk(rsrc_t r, uint32_t off) {
  if constexpr (VEC) return bload16<POL>(r, off);
  else return bload16_e<POL>(r, off);
}

__device__ __forceinline__ int swz(int row, int c) {
  return row * kBK + ((c ^ ((row ^ (row >> 3)) & 7)) << 3);
}

// Zero the bf16 lanes of a 16-byte chunk whose bit in `bits` (8 used) is clear.
__device__ __forceinline__ uint4 mask8(uint4 v, uint32_t bits) {
  const uint32_t m0 = ((bits & 1u) ? 0xFFFFu : 0u) | ((bits & 2u) ? 0xFFFF0000u : 0u);
  const uint32_t m1 = ((bits & 4u) ? 0xFFFFu : 0u) | ((bits & 8u) ? 0xFFFF0000u : 0u);
  const uint32_t m2 = ((bits & 16u) ? 0xFFFFu : 0u) | ((bits & 32u) ? 0xFFFF0000u : 0u);
  const uint32_t m3 = ((bits & 64u) ? 0xFFFFu : 0u) | ((bits & 128u) ? 0xFFFF0000u : 0u);
  return make_uint4(v.x & m0, v.y & m1, v.z & m2, v.w & m3);
}

__device__ __forceinline__ uint32_t u4get(const uint4 &v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

template <typename OUT>
__device__ __forceinline__ void store_out(OUT *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) {
  __builtin_nontemporal_store(v, p);
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) {
  *p = f32_to_bf16(v);
}

// Logical tile for this workgroup: workgroups are dealt round-robin over the
// 8 XCDs, so give each XCD a contiguous range of tiles and walk it in groups
// of kGroupM tile rows (blocks sharing an L2 then share A and B panels).
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of(int64_t w, int64_t tiles_m, int64_t tiles_n, int64_t &tm,
                                        int64_t &tn) {
  const int64_t ntiles = tiles_m * tiles_n;
  int64_t lt = w;
  if ((ntiles & 7) == 0) lt = (w & 7) * (ntiles >> 3) + (w >> 3);
  const int64_t span = (int64_t)kGroupM * tiles_n;
  const int64_t first_m = (lt / span) * kGroupM;
  const int64_t gsz = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  tm = first_m + (lt % span) % gsz;
  tn = (lt % span) / gsz;
}

// The same mapping in 32-bit arithmetic (tile counts below 2^31): 64-bit
// division is a long VALU sequence, too costly inside a persistent loop.
__device__ __forceinline__ void tile_of32(uint32_t w, uint32_t tiles_m, uint32_t tiles_n, uint32_t &tm,
                                          uint32_t &tn) {
  const uint32_t ntiles = tiles_m * tiles_n;
  uint32_t lt = w;
  if ((ntiles & 7) == 0) lt = (w & 7) * (ntiles >> 3) + (w >> 3);
  const uint32_t span = kGroupM * tiles_n;
  const uint32_t first_m = (lt / span) * kGroupM;
  const uint32_t gsz = tiles_m - first_m < (uint32_t)kGroupM ? tiles_m - first_m : (uint32_t)kGroupM;
  tm = first_m + (lt % span) % gsz;
  tn = (lt % span) / gsz;
}

// AVEC / BVEC: 16-byte loads for A / B (rows 16-byte aligned), else 2-byte loads.
template <int BM, int BN, typename OUT, int STAGES, bool AVEC, bool BVEC>
__global__ __launch_bounds__(256) void mfma_gemm(Args g) {
  constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile (2 x 2 waves)
  constexpr int TM = WTM / 32, TN = WTN / 32; // MFMA tiles per wave
  constexpr int A_CH = BM / 32;               // 16-byte A chunks per thread
  constexpr int KB = BN / 32;                 // B rows per thread (x 8 columns)
  constexpr int NB = BN / 8;                  // threads across a B row
  static_assert(KB == 4 || KB == 8, "BN must be 128 or 256");
  __shared__ __attribute__((aligned(16))) uint16_t As[STAGES][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[STAGES][BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int64_t tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t b = blockIdx.z;
  const int64_t grp = (b * g.hkv) / g.hq;
  const int64_t rows = g.m - m0 < BM ? g.m - m0 : BM;

  // Resources: the block's A rows and its B column panel.
  const uint16_t *Ab = g.A + b * g.a_bs + m0 * g.lda;
  const rsrc_t ra_r = make_rsrc(Ab, (uint64_t)rows * g.lda * 2);
  const uint16_t *Bb = g.B + grp * g.b_bs + n0;
  const rsrc_t rb_r = make_rsrc(Bb, ((uint64_t)(g.d - 1) * g.ldb + (g.n - n0)) * 2);

  const int akc = tid & 7;                    // A chunk column
  const int bnb = tid % NB, bkb = tid / NB;   // B block: rows bkb*KB.., columns bnb*8..

  const int32_t *idxb = g.idx + b * g.idx_bs;
  const int nk = (int)(g.k_pad / kBK);

  uint4 ra[A_CH], rb[KB];
  int32_t inext[KB];          // source rows of the next tile to load

  auto load_idx = [&](int q, int32_t *dst) {
    const int4 *p = reinterpret_cast<const int4 *>(idxb + (int64_t)q * kBK + bkb * KB);
#pragma unroll
    for (int v = 0; v < KB / 4; ++v) {
      const int4 x = p[v];
      dst[4 * v] = x.x;
      dst[4 * v + 1] = x.y;
      dst[4 * v + 2] = x.z;
      dst[4 * v + 3] = x.w;
    }
  };

  // Issue the loads of K-tile q (registers only; no use of the data here).
  auto load_tile = [&](int q, const int32_t *src_rows) {
    const int64_t c0 = (int64_t)q * kBK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      ra[i] = load_chunk<AVEC>(ra_r, (uint32_t)(((int64_t)row * g.lda + c0 + akc * 8) * 2));
    }
#pragma unroll
    for (int r = 0; r < KB; ++r) {
      const int32_t s = src_rows[r];
      const uint32_t off = s >= 0 ? (uint32_t)(((int64_t)s * g.ldb + bnb * 8) * 2) : kOOB;
      rb[r] = load_chunk<BVEC>(rb_r, off);
    }
  };

  // Write the loaded registers of a tile into LDS stage `buf`.
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4 *>(&As[buf][swz(row, akc)]) = ra[i];
    }
    if constexpr (KB == 8) {
      // 8 x 8 block -> column e gets one full 16-byte K-run (r0[e] .. r7[e]).
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = u4get(rb[r], q);
        const uint4 ev = make_uint4((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16),
                                    (w[4] & 0xFFFFu) | (w[5] << 16), (w[6] & 0xFFFFu) | (w[7] << 16));
        const uint4 od = make_uint4((w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u),
                                    (w[4] >> 16) | (w[5] & 0xFFFF0000u), (w[6] >> 16) | (w[7] & 0xFFFF0000u));
        const int n_ev = bnb * 8 + 2 * q;
        *reinterpret_cast<uint4 *>(&Bs[buf][swz(n_ev, bkb)]) = ev;
        *reinterpret_cast<uint4 *>(&Bs[buf][swz(n_ev + 1, bkb)]) = od;
      }
    } else {
      // 4 x 8 block -> column e gets an 8-byte half K-run.
      const int kc = bkb >> 1, half = (bkb & 1) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = u4get(rb[r], q);
        const uint2 ev = make_uint2((w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16));
        const uint2 od = make_uint2((w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u));
        const int n_ev = bnb * 8 + 2 * q;
        *reinterpret_cast<uint2 *>(&Bs[buf][swz(n_ev, kc) + half]) = ev;
        *reinterpret_cast<uint2 *>(&Bs[buf][swz(n_ev + 1, kc) + half]) = od;
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Prologue: tile 0 into stage 0; indices of tile 1 in flight.
  if (nk > 0) {
    int32_t i0[KB];
    load_idx(0, i0);
    load_tile(0, i0);
    if (nk > 1) load_idx(1, inext);
    store_tile(0);
    __syncthreads();
  }

  const int lrow = lane & 31, lk = lane >> 5;
  for (int q = 0; q < nk; ++q) {
    const int buf = STAGES == 2 ? (q & 1) : 0;
    const bool more = q + 1 < nk;
    if (more) {
      load_tile(q + 1, inext);
      if (q + 2 < nk) load_idx(q + 2, inext);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        av[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                  &As[buf][swz(wm * WTM + i * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                  &Bs[buf][swz(wn * WTN + j * 32 + lrow, ks * 2 + lk)]));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      if constexpr (STAGES == 1) __syncthreads();
      store_tile(STAGES == 2 ? (buf ^ 1) : 0);
    }
    __syncthreads();
  }

  // D of a 32x32 tile: lane l holds column l%32; register r holds row
  // 8*(r/4) + 4*(l/32) + r%4.
  OUT *Y = static_cast<OUT *>(g.Y) + b * g.y_bs;
  if constexpr (std::is_same<OUT, uint16_t>::value) {
    // bf16 tiles whose columns all lie inside Y go out through LDS (free
    // after the loop's last barrier) as 16-byte row segments, PR rows per
    // pass; stored from the accumulators, every instruction would write 64
    // bytes into each of two rows.  Chunk c of staged row r sits at slot
    // c ^ (r % CPR): the two rows one write instruction touches differ in
    // bit 2 of r and so land on different banks.
    constexpr int CPR = BN / 8;                        // 16-byte chunks per row
    constexpr int PR = STAGES * BM * kBK / BN;         // rows per pass
    static_assert(PR == WTM || PR == BM, "a pass holds one or both wave rows of the tile");
    if (n0 + BN <= g.n && g.ldy % 8 == 0 && reinterpret_cast<uintptr_t>(Y) % 16 == 0) {
      uint16_t *E = &As[0][0];
#pragma unroll
      for (int p = 0; p < BM / PR; ++p) {
        if (PR == BM || wm == p) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int col = wn * WTN + j * 32 + lrow;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = (PR == BM ? wm * WTM : 0) + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
                E[row * BN + (((col >> 3) ^ (row % CPR)) << 3) + (col & 7)] = f32_to_bf16(acc[i][j][r]);
              }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PR * CPR / 256; ++q) {
          const int c = tid + 256 * q;
          const int row = c / CPR, ch = c % CPR;
          const int64_t grow = m0 + p * PR + row;
          const uint4 v = *reinterpret_cast<const uint4 *>(&E[row * BN + ((ch ^ (row % CPR)) << 3)]);
          if (grow < g.m) *reinterpret_cast<uint4 *>(Y + grow * g.ldy + n0 + ch * 8) = v;
        }
        if (p + 1 < BM / PR) __syncthreads();
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * WTN + j * 32 + lrow;
      if (col >= g.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        if (row < g.m) store_out<OUT>(Y + row * g.ldy + col, acc[i][j][r]);
      }
    }
}

}  // namespace mg
}  // namespace rmm

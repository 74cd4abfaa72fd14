// Index-gathered GEMM: Y = A_I B[I, :] ("Mecanismo Central": the reduced
// product A_{:,I} B_{I,:} replaces A B), float32 accumulation.
//
// The bf16 products run on the shared MFMA core (mfma_gemm.h) whenever B's
// base and strides allow 16-byte loads; the kernel below is the fallback for
// other layouts (same math, plain loads).
//
// bf16 fallback (MFMA v_mfma_f32_32x32x16_bf16, gfx950):
//   block tile BM x BN x 64, 4 waves in a 2 x 2 grid, each wave BM/2 x BN/2 as
//   (BM/64) x (BN/64) MFMA tiles of 32 x 32.  A_I arrives packed and
//   K-contiguous, so its tile is copied to LDS as 16-byte chunks.  B is read
//   as it lies in memory: for each kept index t the contiguous row
//   B[idx[t], n0 : n0+BN] is streamed; every thread loads a 4 (k) x 8 (n)
//   block with four 16-byte loads, transposes it in registers and writes eight
//   8-byte K-runs into the K-contiguous B tile in LDS, which is the operand
//   layout the MFMA wants (each lane holds 8 consecutive k of one column).
//   LDS tiles use an XOR swizzle of the 16-byte chunk index so the wave-wide
//   row-strided accesses spread over the banks.  Two LDS stages: the next
//   tile's global loads are in flight while the current tile is multiplied.
//
// f32 path (MFMA v_mfma_f32_16x16x4f32): 64 x 64 x 16 tiles, one element per
// lane per operand, so no transposition is needed.
#include <type_traits>

#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;          // K tile (== kKTile)
constexpr int kChunks = kBK / 8; // 16-byte chunks per LDS row

// Swizzled offset (in bf16 elements) of 16-byte chunk `c` of LDS row `row`.
__device__ __forceinline__ int swz(int row, int c) {
  return row * kBK + ((c ^ ((row ^ (row >> 3)) & 7)) << 3);
}

template <typename OUT>
__device__ __forceinline__ void store_out(OUT *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float v) { *p = f32_to_bf16(v); }

template <int BM, int BN, typename OUT, bool BVEC>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  static_assert(BN == 128, "B loader assumes BN == 128");
  constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32; // MFMA tiles per wave
  constexpr int A_CH = BM * kChunks / 256;    // A chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (g.n + BN - 1) / BN;
  const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t b = blockIdx.z;

  const uint16_t *A = static_cast<const uint16_t *>(g.A) + b * g.m * g.k_pad;
  const int32_t *idx = g.idx + b * g.idx_stride;
  const uint16_t *B = static_cast<const uint16_t *>(g.B) + ((b * g.hkv) / g.hq) * g.b_batch_stride;
  OUT *Y = static_cast<OUT *>(g.Y) + b * g.y_batch_stride;

  // B loader coordinates: 4 k-rows x 8 n-columns per thread.
  const int bnb = tid & 15, bkb = tid >> 4;   // n-block 0..15, k-block 0..15
  const int64_t bcol = n0 + bnb * 8;

  uint4 ra[A_CH];
  uint4 rb[4];

  auto load_global = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      const int64_t gr = m0 + row;
      ra[i] = gr < g.m ? *reinterpret_cast<const uint4 *>(A + gr * g.k_pad + k0 + kc * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = k0 + bkb * 4 + r;
      int64_t src = -1;
      if (t < g.k) {
        const int32_t v = idx[t];
        src = (v >= 0 && v < g.d) ? v : -1;
      }
      uint4 val = make_uint4(0, 0, 0, 0);
      if (src >= 0) {
        const uint16_t *p = B + src * g.ldb + bcol;
        if (BVEC && bcol + 8 <= g.n) {
          val = *reinterpret_cast<const uint4 *>(p);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = (bcol + q < g.n) ? p[q] : (uint16_t)0;
          val.x = e[0] | ((uint32_t)e[1] << 16);
          val.y = e[2] | ((uint32_t)e[3] << 16);
          val.z = e[4] | ((uint32_t)e[5] << 16);
          val.w = e[6] | ((uint32_t)e[7] << 16);
        }
      }
      rb[r] = val;
    }
  };

  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4 *>(&As[buf][swz(row, kc)]) = ra[i];
    }
    // Transpose the 4 x 8 block: column e gets (r0[e], r1[e], r2[e], r3[e]).
    const uint32_t w0[4] = {rb[0].x, rb[0].y, rb[0].z, rb[0].w};
    const uint32_t w1[4] = {rb[1].x, rb[1].y, rb[1].z, rb[1].w};
    const uint32_t w2[4] = {rb[2].x, rb[2].y, rb[2].z, rb[2].w};
    const uint32_t w3[4] = {rb[3].x, rb[3].y, rb[3].z, rb[3].w};
    const int kc = bkb >> 1, half = (bkb & 1) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // even column 2q: low halves; odd column 2q+1: high halves
      const uint2 ev = make_uint2((w0[q] & 0xFFFFu) | (w1[q] << 16), (w2[q] & 0xFFFFu) | (w3[q] << 16));
      const uint2 od = make_uint2((w0[q] >> 16) | (w1[q] & 0xFFFF0000u),
                                  (w2[q] >> 16) | (w3[q] & 0xFFFF0000u));
      const int n_ev = bnb * 8 + 2 * q, n_od = n_ev + 1;
      *reinterpret_cast<uint2 *>(&Bs[buf][swz(n_ev, kc) + half]) = ev;
      *reinterpret_cast<uint2 *>(&Bs[buf][swz(n_od, kc) + half]) = od;
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (int)(g.k_pad / kBK);
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global((int64_t)(kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8_t av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + i * 32 + lrow;
        uint4 v = *reinterpret_cast<const uint4 *>(&As[buf][swz(row, ks * 2 + lk)]);
        av[i] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WTN + j * 32 + lrow;
        uint4 v = *reinterpret_cast<const uint4 *>(&Bs[buf][swz(row, ks * 2 + lk)]);
        bv[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // D[i][j] of a 32x32 tile: lane l holds column l%32, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4.
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

// ---------------------------------------------------------------- f32 path
// TB x TB output tiles (64, or 32 when 64 x 64 tiles would leave most CUs
// idle: fp32 MFMA runs at a sixteenth of the bf16 rate, so a small product
// needs the whole chip), 64-deep K-steps: each step's A and B values are
// loaded into registers while the previous step is multiplied from LDS, so
// a product of a few K-steps pays about one memory latency instead of one
// per step.  Four waves of (TB/2) x (TB/2), v_mfma_f32_16x16x4f32.
constexpr int kFBK = 64;

template <int TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int TW = TB / 32;            // 16 x 16 MFMA tiles per wave side
  constexpr int TPA = 256 / TB;          // threads per A row
  constexpr int FA = kFBK / TPA;         // A values per thread and step (multiple of 4)
  constexpr int FB = TB / 4;             // B values per thread and step (4 threads per kept row)
  static_assert(FA % 4 == 0 && (TB == 32 || TB == 64), "tile");
  __shared__ float As[TB][kFBK + 1];     // row pitch 65: the 16 rows of a fragment read hit distinct banks
  __shared__ float Bs[kFBK][TB + 4];     // row pitch TB + 4: the 4 rows of a fragment read hit distinct banks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (g.n + TB - 1) / TB;
  const int64_t m0 = (blockIdx.x / tiles_n) * TB, n0 = (blockIdx.x % tiles_n) * TB;
  const int64_t b = blockIdx.z;
  const float *A = static_cast<const float *>(g.A) + b * g.m * g.k_pad;
  const int32_t *idx = g.idx + b * g.idx_stride;
  const float *B = static_cast<const float *>(g.B) + ((b * g.hkv) / g.hq) * g.b_batch_stride;
  float *Y = static_cast<float *>(g.Y) + b * g.y_batch_stride;

  f32x4_t acc[TW][TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Per thread and K-step: FA consecutive K values of A row ar, and FB
  // consecutive columns of kept row br of B.
  const int ar = tid / TPA, ac = (tid % TPA) * FA;
  const int br = tid >> 2, bc = (tid & 3) * FB;
  float4 ra[FA / 4];
  float rb[FB];
  auto load = [&](int64_t k0) {
    const int64_t gr = m0 + ar;
#pragma unroll
    for (int q = 0; q < FA / 4; ++q)
      ra[q] = gr < g.m ? *reinterpret_cast<const float4 *>(A + gr * g.k_pad + k0 + ac + 4 * q)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t t = k0 + br;
    int64_t src = -1;
    if (t < g.k) {
      const int32_t v = idx[t];
      src = (v >= 0 && v < g.d) ? v : -1;
    }
#pragma unroll
    for (int q = 0; q < FB; ++q) {
      const int64_t col = n0 + bc + q;
      rb[q] = (src >= 0 && col < g.n) ? B[src * g.ldb + col] : 0.f;
    }
  };

  load(0);
  for (int64_t k0 = 0; k0 < g.k_pad; k0 += kFBK) {
#pragma unroll
    for (int q = 0; q < FA / 4; ++q) {
      As[ar][ac + 4 * q + 0] = ra[q].x;
      As[ar][ac + 4 * q + 1] = ra[q].y;
      As[ar][ac + 4 * q + 2] = ra[q].z;
      As[ar][ac + 4 * q + 3] = ra[q].w;
    }
#pragma unroll
    for (int q = 0; q < FB; ++q) Bs[br][bc + q] = rb[q];
    __syncthreads();
    if (k0 + kFBK < g.k_pad) load(k0 + kFBK);   // next step's loads fly during this product
#pragma unroll
    for (int kk = 0; kk < kFBK; kk += 4) {
      float av[TW], bv[TW];
#pragma unroll
      for (int i = 0; i < TW; ++i) av[i] = As[wm * (TB / 2) + i * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < TW; ++j) bv[j] = Bs[kk + (lane >> 4)][wn * (TB / 2) + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D of a 16x16 tile: lane l holds column l%16, register r holds row 4*(l/16) + r.
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int64_t col = n0 + wn * (TB / 2) + j * 16 + (lane & 15);
      if (col >= g.n) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * (TB / 2) + i * 16 + 4 * (lane >> 4) + r;
        if (row < g.m) Y[row * g.ldy + col] = acc[i][j][r];
      }
    }
}

template <int BM, typename OUT>
hipError_t launch_bm(const GemmArgs &g, bool bvec, hipStream_t st) {
  constexpr int BN = 128;
  const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  dim3 grid((unsigned)tiles, 1, (unsigned)g.batch);
  KernelTimer timer(std::is_same<OUT, float>::value ? "gemm_bf16_f32out" : "gemm_bf16", st);
  if (bvec)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, OUT, true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, OUT, false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int BM, int BN, typename OUT, int STAGES>
hipError_t launch_core(const GemmArgs &g, const char *name, hipStream_t st) {
  const bool bvec = (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && (g.ldb % 8 == 0) &&
                    (g.b_batch_stride % 8 == 0);
  mg::Args a{};
  a.A = static_cast<const uint16_t *>(g.A);
  a.lda = g.k_pad;
  a.a_bs = g.m * g.k_pad;
  a.B = static_cast<const uint16_t *>(g.B);
  a.ldb = g.ldb;
  a.b_bs = g.b_batch_stride;
  a.idx = g.idx;
  a.idx_bs = g.idx_stride;
  a.Y = g.Y;
  a.ldy = g.ldy;
  a.y_bs = g.y_batch_stride;
  a.batch = g.batch;
  a.hq = g.hq;
  a.hkv = g.hkv;
  a.m = g.m;
  a.n = g.n;
  a.d = g.d;
  a.k_pad = g.k_pad;
  a.tiles_m = (g.m + BM - 1) / BM;
  a.tiles_n = (g.n + BN - 1) / BN;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)g.batch);
  KernelTimer timer(name, st);
  if (bvec)
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, OUT, STAGES, true, true>), grid, dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL((mg::mfma_gemm<BM, BN, OUT, STAGES, true, false>), grid, dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_core_ok(const GemmArgs &g) {
  const bool aligned16 = (reinterpret_cast<uintptr_t>(g.B) % 2 == 0) &&
                         (reinterpret_cast<uintptr_t>(g.idx) % 16 == 0) && (g.idx_stride % 4 == 0);
  const bool fits = (uint64_t)((g.d - 1) * g.ldb + g.n) * 2 < mg::kMaxRecords &&
                    (uint64_t)256 * g.k_pad * 2 < mg::kMaxRecords;
  return aligned16 && fits;
}

// `g.idx` must be the cleaned index list (k_pad entries per batch, -1 where a
// row contributes zero) when the core path is taken.
hipError_t launch_gemm_bf16(const GemmArgs &g, OutType out, hipStream_t st) {
  if (gemm_core_ok(g)) {
    const int64_t nk = g.k_pad / kBK;
    if (out == OutType::F32) {
      if (nk == 1) return launch_core<128, 128, float, 1>(g, "gemm_f32out", st);
      return launch_core<128, 128, float, 2>(g, "gemm_f32out", st);
    }
    const int64_t t256 = ((g.m + 255) / 256) * ((g.n + 255) / 256) * g.batch;
    if (t256 >= 200) return launch_core<256, 256, uint16_t, 2>(g, "gemm_256", st);
    return launch_core<128, 128, uint16_t, 2>(g, "gemm_128", st);
  }
  const bool bvec = (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && (g.ldb % 8 == 0) &&
                    (g.b_batch_stride % 8 == 0);
  if (out == OutType::F32) return launch_bm<128, float>(g, bvec, st);
  return launch_bm<128, uint16_t>(g, bvec, st);
}

hipError_t launch_gemm_f32(const GemmArgs &g, hipStream_t st) {
  const int64_t tiles64 = ((g.m + 63) / 64) * ((g.n + 63) / 64) * g.batch;
  KernelTimer timer("gemm_f32", st);
  if (tiles64 >= 128) {
    hipLaunchKernelGGL(gemm_f32_kernel<64>, dim3((unsigned)(tiles64 / g.batch), 1, (unsigned)g.batch), dim3(256), 0,
                       st, g);
  } else {
    const int64_t tiles32 = ((g.m + 31) / 32) * ((g.n + 31) / 32);
    hipLaunchKernelGGL(gemm_f32_kernel<32>, dim3((unsigned)tiles32, 1, (unsigned)g.batch), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace rmm

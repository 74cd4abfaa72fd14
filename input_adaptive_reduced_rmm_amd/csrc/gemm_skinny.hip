// Reduced GEMM for a few rows (decode batches, m <= 32): Y = A_I B[I, :]
// ("Mecanismo Central": the reduced product A_{:,I} B_{I,:} replaces A B),
// with B in bf16 or in int8 with one float scale per output column (the
// pages state that the method works unchanged on INT8 weights).
//
// At m <= 32 the product is bound by reading the kept rows of B (k x n
// elements) once; the flops are small.  The kernel therefore spreads those
// rows over many workgroups: a workgroup owns a 128-column panel (bf16 or
// int8; a 256-column int8 panel ran 17-23 % slower on the largest 70B decode
// product) and a contiguous range of K-tiles (split over K),
// and writes fp32 partial sums that a second kernel adds in a fixed order
// (deterministic).  With a single split the first kernel writes Y directly.
//
// Per K-tile of 64 kept rows each thread loads one 16-byte chunk from each of
// its rows (the row offsets come from the cleaned index list staged in LDS;
// -1 rows read as zero through the buffer range).  The loads are
// non-temporal: a decode step reads each weight row once, and a load that
// does not allocate in the caches neither evicts other data nor has to wait
// for the dirty lines an allocation would evict to be written back.  Each
// thread converts int8 to bf16 (exact: |q| <= 128 needs 8 significant bits),
// transposes its block in registers into K-runs and writes them to a
// swizzled K-contiguous LDS tile.
// The packed A_I rows of the K-tile (32 rows, rows >= m read zero) go into
// the same LDS stage, one 16-byte chunk per thread: the register slots then
// hold almost only weight bytes, which lets more K-tiles be in flight.
// Waves multiply with v_mfma_f32_32x32x16_bf16: A_I fragments are the first
// operand, the B^T fragments the second, so each lane ends with one output
// column and 16 rows.  The int8 column scale multiplies the fp32 sum once, at
// the end.
#include <type_traits>

#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

using mg::bf16x8_t;
using mg::f32x16_t;
using mg::rsrc_t;

constexpr int kBK = 64;
// s_waitcnt immediate: vmcnt = n, expcnt and lgkmcnt not waited on
constexpr int vm_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
constexpr int kMaxTilesPerSplit = 32;   // cleaned indices of a split staged in LDS (8 KiB)

// Calls f(integral_constant<I>) for I = B .. E-1 (compile-time slot indices).
template <int B, int E>
struct Unroll {
  template <class F>
  __device__ __forceinline__ static void run(F &&f) {
    f(std::integral_constant<int, B>{});
    Unroll<B + 1, E>::run(f);
  }
};
template <int E>
struct Unroll<E, E> {
  template <class F>
  __device__ __forceinline__ static void run(F &&) {}
};

struct SkinnyArgs {
  const uint16_t *A;     // packed A_I [m][k_pad] bf16
  const void *B;         // [d][ldb] bf16 or int8
  int64_t ldb;           // elements
  const float *scale;    // [n] for int8 B
  const int32_t *idx;    // cleaned [k_pad]
  uint16_t *Y;
  int64_t ldy;
  float *part;           // [splits][m][n] (splits > 1)
  int64_t m, n, d, k_pad;
  int tiles_n, splits, tiles_per_split;
};

__device__ __forceinline__ uint32_t i8_to_bf16_bits(uint32_t w, int byte) {
  const int v = (int)(w << (24 - 8 * byte)) >> 24;
  return __float_as_uint((float)v) >> 16;
}

constexpr int kW8BN = 128;
constexpr int kPdBf16 = 4, kPdW8 = 4;

template <bool W8>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyArgs g) {
  constexpr int BN = W8 ? kW8BN : 128;     // columns per workgroup
  constexpr int TN = BN / 128;             // 32-column MFMA tiles per wave
  constexpr int CPC = W8 ? 16 : 8;         // columns per 16-byte chunk
  constexpr int NBT = BN / CPC;            // threads across the panel
  constexpr int RPT = kBK * NBT / 256;     // rows per thread per K-tile
  static_assert(RPT == (W8 ? 2 : 4), "loader assumes 4 bf16 or 2 int8 rows per thread");
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t As[2][32 * kBK];
  __shared__ int32_t sidx[kMaxTilesPerSplit * kBK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tn = (int)(blockIdx.x % (unsigned)g.tiles_n), split = (int)(blockIdx.x / (unsigned)g.tiles_n);
  const int64_t n0 = (int64_t)tn * BN;
  const int nk = (int)(g.k_pad / kBK);
  const int q0 = split * g.tiles_per_split;
  const int q1 = q0 + g.tiles_per_split < nk ? q0 + g.tiles_per_split : nk;
  const int ntile = q1 - q0;

  constexpr int E = W8 ? 1 : 2;   // bytes per B element
  const char *Bp = static_cast<const char *>(g.B) + n0 * E;
  const rsrc_t rb_r = mg::make_rsrc(Bp, (uint64_t)((g.d - 1) * g.ldb + (g.n - n0)) * E);
  const rsrc_t ra_r = mg::make_rsrc(g.A, (uint64_t)g.m * g.k_pad * 2);

  // This split's kept rows, staged once.
  for (int i = tid; i < ntile * kBK; i += 256) sidx[i] = g.idx[(int64_t)q0 * kBK + i];
  __syncthreads();

  const int bnb = tid % NBT, bkb = tid / NBT;   // chunk column, row group (rows RPT*bkb..)
  const int lrow = lane & 31, lk = lane >> 5;
  const int arow = tid >> 3, achk = tid & 7;    // this thread's A_I chunk of a K-tile
  // PD register slots: the loads of the next PD K-tiles are in flight while
  // the current one is multiplied from LDS (at this few rows the kernel is
  // bound by how many bytes each CU keeps in flight).
  constexpr int PD = W8 ? kPdW8 : kPdBf16;
  uint4 rb[PD][RPT], ra[PD];

  auto issue = [&](int slot, int q) {   // q: tile index within the split
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int32_t s = sidx[q * kBK + bkb * RPT + r];
      const uint32_t off = s >= 0 ? (uint32_t)(((int64_t)s * g.ldb) * E + bnb * 16) : mg::kOOB;
      rb[slot][r] = mg::bload16<mg::kNonTemporal>(rb_r, off);
    }
    ra[slot] = mg::bload16(ra_r, (uint32_t)(((int64_t)arow * g.k_pad + (int64_t)(q0 + q) * kBK + achk * 8) * 2));
  };

  // Registers of one K-tile -> K-contiguous LDS stage `buf`.
  auto store = [&](int slot, int buf) {
    *reinterpret_cast<uint4 *>(&As[buf][mg::swz(arow, achk)]) = ra[slot];
    // rows RPT*bkb .. RPT*bkb+RPT-1 -> K-chunk kc, elements half .. half+RPT-1
    const int kc = (RPT * bkb) >> 3, half = (RPT * bkb) & 7;
    if constexpr (!W8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = mg::u4get(rb[slot][0], q), w1 = mg::u4get(rb[slot][1], q),
                       w2 = mg::u4get(rb[slot][2], q), w3 = mg::u4get(rb[slot][3], q);
        const uint2 ev = make_uint2((w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16));
        const uint2 od = make_uint2((w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u));
        const int n_ev = bnb * CPC + 2 * q;
        *reinterpret_cast<uint2 *>(&Bs[buf][mg::swz(n_ev, kc) + half]) = ev;
        *reinterpret_cast<uint2 *>(&Bs[buf][mg::swz(n_ev + 1, kc) + half]) = od;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int q = c >> 2, byte = c & 3;
        const uint32_t b0 = i8_to_bf16_bits(mg::u4get(rb[slot][0], q), byte);
        const uint32_t b1 = i8_to_bf16_bits(mg::u4get(rb[slot][1], q), byte);
        *reinterpret_cast<uint32_t *>(&Bs[buf][mg::swz(bnb * CPC + c, kc) + half]) = b0 | (b1 << 16);
      }
    }
  };

  f32x16_t acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  constexpr int LOADS = RPT + 1;   // vector loads per issue
  // Wait until at most n issues (n * LOADS loads) are outstanding.
  auto wait_issues = [&](int n) __attribute__((always_inline)) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(vm_imm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(vm_imm(LOADS)); break;
      case 2: __builtin_amdgcn_s_waitcnt(vm_imm(2 * LOADS)); break;
      case 3: __builtin_amdgcn_s_waitcnt(vm_imm(3 * LOADS)); break;
      case 4: __builtin_amdgcn_s_waitcnt(vm_imm(4 * LOADS)); break;
      case 5: __builtin_amdgcn_s_waitcnt(vm_imm(5 * LOADS)); break;
      default: __builtin_amdgcn_s_waitcnt(vm_imm(6 * LOADS)); break;
    }
  };
  static_assert(PD >= 2 && PD <= 7 && 6 * LOADS <= 63, "prefetch depth");
  // One K-tile q: LDS stage q&1 holds it (A_I and B), and slot S = q % PD,
  // whose registers it came from, is free; tiles q+1 .. q+PD-1 are in flight.
  // Refill slot S with tile q + PD, multiply, then convert tile q + 1 into
  // the other stage.
  auto step = [&](auto s_c, int q) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value, SN = (S + 1) % PD;
    const int buf = q & 1;
    if (q + PD < ntile) issue(S, q + PD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8_t a8 = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4 *>(&As[buf][mg::swz(lrow, ks * 2 + lk)]));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const bf16x8_t b8 = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4 *>(&Bs[buf][mg::swz(wave * 32 * TN + j * 32 + lrow, ks * 2 + lk)]));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, acc[j], 0, 0, 0);
      }
    }
    if (q + 1 < ntile) {
      // issued after tile q+1: tiles q+2 .. min(q+PD, ntile-1)
      const int later = (q + PD < ntile ? q + PD : ntile - 1) - (q + 1);
      wait_issues(later);
      store(SN, buf ^ 1);
    }
    __syncthreads();
  };

  {
    const int pre = ntile < PD ? ntile : PD;
#pragma unroll
    for (int i = 0; i < PD; ++i)
      if (i < pre) issue(i, i);
    if (pre > 0) {
      wait_issues(pre - 1);
      store(0, 0);
    }
  }
  __syncthreads();
  int q = 0;
  for (; q + PD <= ntile; q += PD)
    Unroll<0, PD>::run([&](auto i) __attribute__((always_inline)) { step(i, q + decltype(i)::value); });
  Unroll<0, PD - 1>::run([&](auto i) __attribute__((always_inline)) {
    if (q + decltype(i)::value < ntile) step(i, q + decltype(i)::value);
  });

  // acc[j]: lane holds column n0 + 32*(TN*wave + j) + lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + 32 * (TN * wave + j) + lrow;
    if (col >= g.n) continue;
    const float sc = W8 && g.splits == 1 ? g.scale[col] : 1.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = 8 * (r >> 2) + 4 * lk + (r & 3);
      if (row >= g.m) continue;
      if (g.splits == 1) g.Y[row * g.ldy + col] = f32_to_bf16(acc[j][r] * sc);
      else g.part[((int64_t)split * g.m + row) * g.n + col] = acc[j][r];
    }
  }
}

// Y[i][c] = bf16(scale[c] * sum over splits of part[s][i][c]), splits added
// in order; eight split loads are issued before they are summed.
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float *__restrict__ part, int splits, int64_t m,
                                                            int64_t n, const float *__restrict__ scale,
                                                            uint16_t *__restrict__ Y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * n) return;
  const int64_t i = e / n, c = e % n, mn = m * n;
  const float *p = part + i * n + c;
  float s = 0.f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(sp + u) * mn];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; sp < splits; ++sp) s += p[(int64_t)sp * mn];
  if (scale) s *= scale[c];
  Y[i * ldy + c] = f32_to_bf16(s);
}

// Kept int8 rows dequantized for the many-row path:
// Bd[t][c] = bf16(q[idx[t]][c] * scale[c]) (zero rows where idx < 0), 8 columns per thread.
__global__ __launch_bounds__(256) void w8_dequant_rows_kernel(const int8_t *__restrict__ Bq, int64_t ldb,
                                                              const float *__restrict__ scale,
                                                              const int32_t *__restrict__ idx, int64_t k_pad,
                                                              int64_t n, uint16_t *__restrict__ Bd) {
  const int64_t cpr = (n + 7) / 8;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= k_pad * cpr) return;
  const int64_t t = e / cpr, c0 = (e % cpr) * 8;
  const int32_t s = idx[t];
  for (int q = 0; q < 8 && c0 + q < n; ++q) {
    const int64_t c = c0 + q;
    Bd[t * n + c] = s >= 0 ? f32_to_bf16((float)Bq[(int64_t)s * ldb + c] * scale[c]) : (uint16_t)0;
  }
}

struct SkinnyPlan {
  int tiles_n, splits, tiles_per_split;
};

// Workgroups per CU the grid aims at: about one resident round, so each
// workgroup streams a long run of K-tiles instead of paying the pipeline fill
// many times.  LDS (two 16 KiB weight stages, two 4 KiB A_I stages and the
// index list) holds both kernels to 3 resident workgroups per CU; aiming at 3
// or 4 bf16 workgroups per CU measures the same.
constexpr int kWgBf16 = 4, kWgW8 = 3;

SkinnyPlan skinny_plan(bool w8, int64_t n, int64_t k_pad) {
  const int64_t bn = w8 ? kW8BN : 128;
  SkinnyPlan p;
  p.tiles_n = (int)((n + bn - 1) / bn);
  const int64_t nk = k_pad / kBK;
  const int64_t target = 256 * (w8 ? kWgW8 : kWgBf16);
  // Enough workgroups for the target, at least 4 K-tiles each, at most what LDS stages.
  int64_t splits = (target + p.tiles_n - 1) / p.tiles_n;
  const int64_t max_by_depth = nk / 4 > 0 ? nk / 4 : 1;
  if (splits > max_by_depth) splits = max_by_depth;
  const int64_t min_by_lds = (nk + kMaxTilesPerSplit - 1) / kMaxTilesPerSplit;
  if (splits < min_by_lds) splits = min_by_lds;
  if (splits < 1) splits = 1;
  p.tiles_per_split = (int)((nk + splits - 1) / splits);
  p.splits = (int)((nk + p.tiles_per_split - 1) / p.tiles_per_split);
  return p;
}

}  // namespace

hipError_t launch_w8_dequant_rows(const void *Bq, int64_t ldb, const float *scale, const int32_t *idx_clean,
                                  int64_t k_pad, int64_t n, void *Bd, hipStream_t st) {
  KernelTimer timer("w8_dequant", st);
  const int64_t total = k_pad * ((n + 7) / 8);
  hipLaunchKernelGGL(w8_dequant_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     static_cast<const int8_t *>(Bq), ldb, scale, idx_clean, k_pad, n, static_cast<uint16_t *>(Bd));
  return hipGetLastError();
}

bool skinny_ok(int64_t m, const void *B, int64_t ldb, bool w8, int64_t d, int64_t n) {
  const int64_t e = w8 ? 1 : 2;
  return m >= 1 && m <= 32 && reinterpret_cast<uintptr_t>(B) % 16 == 0 && (ldb * e) % 16 == 0 &&
         (uint64_t)((d - 1) * ldb + n) * e < mg::kMaxRecords;
}

size_t skinny_part_bytes(bool w8, int64_t m, int64_t n, int64_t k_pad) {
  const SkinnyPlan p = skinny_plan(w8, n, k_pad);
  return p.splits > 1 ? (size_t)p.splits * m * n * 4 : 0;
}

hipError_t launch_gemm_skinny(const void *A_packed, const int32_t *idx_clean, const void *B, bool w8,
                              const float *scale, int64_t ldb, int64_t d, int64_t m, int64_t n, int64_t k_pad,
                              void *Y, int64_t ldy, float *part, hipStream_t st) {
  const SkinnyPlan p = skinny_plan(w8, n, k_pad);
  SkinnyArgs g{};
  g.A = static_cast<const uint16_t *>(A_packed);
  g.B = B;
  g.ldb = ldb;
  g.scale = scale;
  g.idx = idx_clean;
  g.Y = static_cast<uint16_t *>(Y);
  g.ldy = ldy;
  g.part = part;
  g.m = m;
  g.n = n;
  g.d = d;
  g.k_pad = k_pad;
  g.tiles_n = p.tiles_n;
  g.splits = p.splits;
  g.tiles_per_split = p.tiles_per_split;
  const dim3 grid((unsigned)((int64_t)p.tiles_n * p.splits));
  {
    KernelTimer timer(w8 ? "gemm_skinny_w8" : "gemm_skinny", st);
    if (w8) hipLaunchKernelGGL(gemm_skinny_kernel<true>, grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL(gemm_skinny_kernel<false>, grid, dim3(256), 0, st, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.splits == 1) return hipSuccess;
  KernelTimer timer("skinny_reduce", st);
  const int64_t total = m * n;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part, p.splits,
                     m, n, w8 ? scale : nullptr, static_cast<uint16_t *>(Y), ldy);
  return hipGetLastError();
}

}  // namespace rmm

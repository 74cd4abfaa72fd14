// Fused reduced causal attention: the feature-reduced Q K^T, the causal
// softmax and the token-reduced P V of one layer, without writing S or P to
// memory ("Alcance de Aplicación": reduce the feature dimension of Q K^T and
// the token dimension of P V; "Estrategia de Selección": a token's score is
// the Euclidean norm of its column of P).
//
// The token scores need every row of P before any output can be formed, so
// the work runs in passes over recomputed score tiles:
//   A  (per query row)   m_i = max_j c S_ij,  l_i = sum_j 2^(c S_ij - m_i)
//   B  (per key column)  s_j = sqrt(sum_i P_ij^2) with P_ij = 2^(c S_ij - m_i - log2 l_i)
//   top-k of s           J (kept tokens, ascending)
//   D  (per query row)   O_i = sum_{j in J} P_ij V_j
// with c = log2(e) / sqrt(dh) and S_ij = Q_I[i] . K_I[j] over the kept
// features I, causal: key j is visible from query i when j <= i + (Lk - Lq).
//
// Operands are packed once per call: Q_I [h][Lq][KF] and K_I [h][Lk][KF]
// (KF = kept features padded to 64), and for pass D the kept keys K_J
// [h][kt_pad][KF] and the kept values transposed, V_J^T [h][dh][kt_pad].
// Every matrix product runs on v_mfma_f32_32x32x16_bf16.  A workgroup is 8
// waves; each wave owns 32 rows of the result and the workgroup streams the
// other operand through LDS in 64-row tiles (direct buffer-to-LDS loads, two
// stages), so the tiles are read from L2 once per 256 rows.
//
// Layout of a 32x32 MFMA result: lane l holds column l%32 and rows
// 8*(r/4) + 4*(l/32) + r%4 for its registers r = 0..15.  Pass A and D compute
// S^T (rows = keys, lane = query) so that each lane owns one query; pass B
// computes S (rows = queries, lane = key) so that each lane owns one key.
#include "mfma_gemm.h"
#include "rmm_internal.h"
#include "timing.h"

#define LDS_AS __attribute__((address_space(3)))

namespace rmm {
namespace {

using mg::bf16x8_t;
using mg::f32x16_t;
using mg::rsrc_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;   // rows of the result per workgroup
constexpr int kT = 64;               // streamed tile rows

struct AttnArgs {
  const uint16_t *QI;   // [hq][Lq][KF]
  const uint16_t *KI;   // [hq][Lk][KF]
  const uint16_t *KJ;   // [hq][kt_pad][KF]
  const uint16_t *VJT;  // [hq][dh][kt_pad]
  const int32_t *J;     // [hq][kt_pad] kept tokens, ascending, -1 padded
  float *nml;           // [hq][Lq] -(row max of c S) - log2(row sum): P = 2^(c S + nml)
  float *n2ml;          // [hq][Lq] 2 nml: P^2 = 2^(2 c S + n2ml)
  float *tok;           // [hq][Lk] token scores
  float *opart;         // [blocks_q][hq][128] column sums of O^2 per row block, or null
  uint16_t *O;          // [Lq tokens of o_ts] x [hq of o_hs] x dh
  int64_t o_ts, o_hs;
  int64_t hq, Lq, Lk, kt, kt_pad;
  int causal;
  int64_t off;          // Lk - Lq
  float c2;             // log2(e) / sqrt(dh)
  int64_t blocks_q, blocks_k;   // query and key row blocks of kRows
};

// 16 (or 4) bytes per lane from the buffer straight into LDS: the wave's 64
// lanes fill 1 KiB (256 bytes) at `lds` in lane order.  (Plain functions, so
// that the kernel templates stay instantiable in the host compilation pass.)
__device__ __forceinline__ void lds_load16(rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_load4(rsrc_t r, void *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)lds, 4, voff, soff, 0, 0);
}
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr int vm_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kNegInf = -__builtin_inff();

// A [kT][KF] bf16 tile in LDS: KF/64 halves of [kT][64], each row 128 bytes
// with the 16-byte chunk index XOR-swizzled by the row (mg::swz).
template <int KF>
struct Tile {
  static constexpr int H = KF / 64;
  static constexpr int BYTES = kT * KF * 2;
  static constexpr int BLOCKS = BYTES / 1024;      // 1 KiB direct-load blocks
  static constexpr int PER_WAVE = BLOCKS / kWaves;  // loads per wave
};

// Issue the direct loads of rows [row0, row0 + kT) of a row-major [rows][KF]
// bf16 matrix (resource r) into `dst`.  Load i of a wave fills LDS block
// q = i * kWaves + wave = (half, 8-row group): rows 8 g + lane/8 of that
// half, slot lane%8, which holds logical chunk slot ^ f(row).
template <int KF, int NW = kWaves>
__device__ __forceinline__ void issue_tile(rsrc_t r, int64_t row0, unsigned char *dst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < Tile<KF>::BLOCKS / NW; ++i) {
    const int q = i * NW + wave;
    const int half = q / 8, grp = q % 8;
    const int row = grp * 8 + lane / 8;
    const int slot = lane % 8;
    const int logical = slot ^ ((row ^ (row >> 3)) & 7);
    const uint32_t voff = (uint32_t)((((row0 + row) * KF) + half * 64 + logical * 8) * 2);
    lds_load16(r, dst + q * 1024, voff, 0);
  }
}

// Fragment of LDS tile row `row`, K-slice ks (16 features), for this lane.
template <int KF>
__device__ __forceinline__ bf16x8_t lds_frag(const unsigned char *tile, int row, int ks, int lk) {
  const int half = ks / 4;
  const uint16_t *t = reinterpret_cast<const uint16_t *>(tile + half * (kT * 128));
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(&t[mg::swz(row, (ks % 4) * 2 + lk)]));
}

// Q_I fragments of the wave's 32 rows (lane-fixed row = l%32), straight from memory.
template <int KF>
__device__ __forceinline__ void load_row_frags(const uint16_t *base, int64_t nrows, int64_t row0, int lane,
                                               bf16x8_t *f) {
  const rsrc_t r = mg::make_rsrc(base, (uint64_t)nrows * KF * 2);
  const int64_t row = row0 + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < KF / 16; ++ks)
    f[ks] = __builtin_bit_cast(bf16x8_t,
                               mg::bload16(r, (uint32_t)((row * KF + ks * 16 + (lane >> 5) * 8) * 2)));
}

// Column sums of squares of the bf16 output over this workgroup's queries
// (producer-fused scores for the projection that reads O): lanes add the
// squares of the values they store, the two lane halves and then the waves
// are added in order, and one partial per (row block, head, column) is
// written; colnorm_finish adds the row blocks.
template <int NW>
__device__ __forceinline__ void out_col_partials(float (&cs)[4], int wave, int lane, float *red, float *dst) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) cs[dt] += __shfl_xor(cs[dt], 32, 64);
  if (lane < 32) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) red[wave * 128 + dt * 32 + lane] = cs[dt];
  }
  __syncthreads();
  const int t = wave * 64 + lane;
  if (t < 128) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w * 128 + t];
    dst[t] = s;
  }
}

// ---------------------------------------------------------------- pass A
// Workgroup = 256 queries of one head (8 waves x 32); K_I streams in 64-key
// tiles.  Each lane keeps a running max and sum over the keys it holds;
// lanes l and l+32 (same query, interleaved keys) are merged at the end.
template <int KF>
__global__ __launch_bounds__(kThreads) void attn_stats_kernel(AttnArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * Tile<KF>::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // heaviest query blocks first, across heads
  const int64_t qb = g.blocks_q - 1 - (int64_t)blockIdx.x / g.hq;
  const int64_t h = (int64_t)blockIdx.x % g.hq;
  const int64_t q0l = qb * kRows + 32 * wave;
  bf16x8_t qf[KF / 16];
  load_row_frags<KF>(g.QI + h * g.Lq * KF, g.Lq, q0l, lane, qf);

  const int64_t blk_last = qb * kRows + kRows - 1;   // last query of the block
  const int64_t nkeys = g.causal ? min(g.Lk, blk_last + g.off + 1) : g.Lk;
  const int64_t wave_keys = g.causal ? min(g.Lk, q0l + 31 + g.off + 1) : g.Lk;
  const int nt = (int)cdiv(nkeys, kT);
  const rsrc_t rk = mg::make_rsrc(g.KI + h * g.Lk * KF, (uint64_t)g.Lk * KF * 2);

  // 32-bit row and key numbers below (Lq, Lk < 2^31)
  const int Lk = (int)g.Lk, off = (int)g.off, q0 = (int)q0l, qi = q0 + (lane & 31);
  float m_run = kNegInf, l_run = 0.f;   // raw-score max and sum of 2^(c (s - max))
  if (nt > 0) issue_tile<KF>(rk, 0, smem, wave, lane);
  for (int t = 0; t < nt; ++t) {
    unsigned char *cur = smem + (t & 1) * Tile<KF>::BYTES;
    if (t + 1 < nt) {
      issue_tile<KF>(rk, (int64_t)(t + 1) * kT, smem + ((t + 1) & 1) * Tile<KF>::BYTES, wave, lane);
      __builtin_amdgcn_s_waitcnt(vm_imm(Tile<KF>::PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
    }
    // A bare barrier after the explicit wait: __syncthreads would also wait
    // for the next tile's loads, which must stay in flight.
    __builtin_amdgcn_s_barrier();
    const int tk0 = t * kT;
    if (tk0 < wave_keys) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KF / 16; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag<KF>(cur, sub * 32 + (lane & 31), ks, lane >> 5),
                                                        qf[ks], acc, 0, 0, 0);
        // Keys of this 32-key slice: every query of the wave sees all of them
        // unless the slice crosses the diagonal or the end of the keys.
        const int kb0 = tk0 + sub * 32;
        const bool full = kb0 + 31 < Lk && (!g.causal || kb0 + 31 <= q0 + off);
        if (!full) {
          const int kl = kb0 + 4 * (lane >> 5);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kl + 8 * (r >> 2) + (r & 3);
            const bool ok = key < Lk && (!g.causal || key <= qi + off);
            acc[r] = ok ? acc[r] : kNegInf;
          }
        }
        float tmax = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
        const float m_new = fmaxf(m_run, tmax);   // raw score units (c > 0 keeps the order)
        if (m_new != kNegInf) {
          const float nm = -m_new * g.c2;
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += fexp2(fmaf(acc[r], g.c2, nm));
          l_run = l_run * fexp2((m_run - m_new) * g.c2) + sum;
          m_run = m_new;
        }
      }
    }
    // All waves are done reading `cur` before it is refilled (a bare barrier
    // after the LDS reads drain: the next tile's loads stay in flight).
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
  }
  // merge the two lanes of each query
  const float m_p = __shfl_xor(m_run, 32, 64), l_p = __shfl_xor(l_run, 32, 64);
  const float m = fmaxf(m_run, m_p);
  float l = 0.f;
  if (m != kNegInf)
    l = (m_run == kNegInf ? 0.f : l_run * fexp2((m_run - m) * g.c2)) +
        (m_p == kNegInf ? 0.f : l_p * fexp2((m_p - m) * g.c2));
  if (lane < 32 && qi < g.Lq) {
    // the normaliser folds into the exponent: P = 2^(c s - c max - log2 sum)
    const float v = l > 0.f ? -m * g.c2 - log2f(l) : kNegInf;
    const int64_t o = h * g.Lq + qi;
    g.nml[o] = v;
    g.n2ml[o] = 2.f * v;
  }
}

// ---------------------------------------------------------------- pass B
// Workgroup = 256 keys of one head (8 waves x 32); Q_I streams in 64-query
// tiles with their row statistics.  Each lane sums P^2 over the queries it
// holds for its key; lanes l and l+32 are merged at the end.
template <int KF>
__global__ __launch_bounds__(kThreads) void attn_colsq_kernel(AttnArgs g) {
  constexpr int STAGE = Tile<KF>::BYTES + kT * 4;   // Q tile, then n2ml of its rows
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // causal: the lowest keys see the most queries, so key blocks go in order
  const int64_t kb = (int64_t)blockIdx.x / g.hq;
  const int64_t h = (int64_t)blockIdx.x % g.hq;
  const int64_t k0l = kb * kRows + 32 * wave;
  bf16x8_t kf[KF / 16];
  load_row_frags<KF>(g.KI + h * g.Lk * KF, g.Lk, k0l, lane, kf);
  const int Lq = (int)g.Lq, Lk = (int)g.Lk, off = (int)g.off, k0 = (int)k0l, key = k0 + (lane & 31);
  const float c4 = 2.f * g.c2;   // p^2 = 2^(2 c s + n2ml)

  // first query row any key of the block can be seen from
  const int64_t qfirst = g.causal ? max((int64_t)0, kb * kRows - g.off) : 0;
  const int64_t t_first = qfirst / kT;
  const int64_t nt = cdiv(g.Lq, kT) - t_first;
  const int64_t wave_qfirst = g.causal ? k0l - g.off : 0;   // queries below this see no key of the wave
  const rsrc_t rq = mg::make_rsrc(g.QI + h * g.Lq * KF, (uint64_t)g.Lq * KF * 2);
  const rsrc_t rm = mg::make_rsrc(g.n2ml + h * g.Lq, (uint64_t)g.Lq * 4);

  auto issue = [&](int64_t t, unsigned char *dst) {
    const int64_t row0 = (t_first + t) * kT;
    issue_tile<KF>(rq, row0, dst, wave, lane);
    // row statistics: wave 0 loads the 64 rows' n2ml (4 bytes per lane)
    if (wave == 0) lds_load4(rm, dst + Tile<KF>::BYTES, (uint32_t)((row0 + lane) * 4), 0);
  };

  float c_lane = 0.f;
  if (nt > 0) issue(0, smem);
  for (int64_t t = 0; t < nt; ++t) {
    unsigned char *cur = smem + (t & 1) * STAGE;
    if (t + 1 < nt) {
      issue(t + 1, smem + ((t + 1) & 1) * STAGE);
      if (wave == 0) __builtin_amdgcn_s_waitcnt(vm_imm(Tile<KF>::PER_WAVE + 1));
      else __builtin_amdgcn_s_waitcnt(vm_imm(Tile<KF>::PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
    }
    // A bare barrier after the explicit wait: __syncthreads would also wait
    // for the next tile's loads, which must stay in flight.
    __builtin_amdgcn_s_barrier();
    const int qt0 = (int)((t_first + t) * kT);
    if (qt0 + kT > wave_qfirst) {
      const float *sm = reinterpret_cast<const float *>(cur + Tile<KF>::BYTES);   // n2ml
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KF / 16; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag<KF>(cur, sub * 32 + (lane & 31), ks, lane >> 5),
                                                        kf[ks], acc, 0, 0, 0);
        // Queries of this 32-query slice: all see every key of the wave
        // unless the slice crosses the diagonal or the end of the queries.
        const int qs0 = qt0 + sub * 32;
        const bool full = qs0 + 31 < Lq && k0 + 31 < Lk && (!g.causal || k0 + 31 <= qs0 + off);
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int rr = sub * 32 + 8 * b4 + 4 * (lane >> 5);   // tile row of register 4*b4
          const float4 mv = *reinterpret_cast<const float4 *>(&sm[rr]);
          const float mm[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p2 = fexp2(fmaf(acc[4 * b4 + e], c4, mm[e]));
            if (!full) {
              const int q = qt0 + rr + e;
              const bool ok = q < Lq && key < Lk && (!g.causal || key <= q + off);
              p2 = ok ? p2 : 0.f;
            }
            c_lane += p2;
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // LDS reads of `cur` drained; the next tile's loads stay in flight
    __builtin_amdgcn_s_barrier();
  }
  const float c = c_lane + __shfl_xor(c_lane, 32, 64);
  if (lane < 32 && key < g.Lk) g.tok[h * g.Lk + key] = __builtin_sqrtf(c);
}

// ---------------------------------------------------------------- pass D
// Workgroup = 256 queries of one head; the kept keys K_J and values V_J^T
// stream in 64-token tiles.  The probability tile of a 32-token slice is
// formed in registers (S^T layout: lane = query), rounded to bf16, and
// regrouped across the two lane halves into the A operand of the P V product.
template <int KF>
__global__ __launch_bounds__(kThreads) void attn_out_kernel(AttnArgs g) {
  constexpr int VT_BYTES = 128 * kT * 2;                      // V_J^T tile [128 d][64 kept]
  constexpr int STAGE = Tile<KF>::BYTES + VT_BYTES + kT * 4;  // + kept token ids
  constexpr int VT_PER_WAVE = VT_BYTES / 1024 / kWaves;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, lk = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qb = g.blocks_q - 1 - (int64_t)blockIdx.x / g.hq;
  const int64_t h = (int64_t)blockIdx.x % g.hq;
  const int64_t q0l = qb * kRows + 32 * wave;
  bf16x8_t qf[KF / 16];
  load_row_frags<KF>(g.QI + h * g.Lq * KF, g.Lq, q0l, lane, qf);
  const int off = (int)g.off, kt = (int)g.kt, q0 = (int)q0l, qi = q0 + (lane & 31);
  const float nml = qi < g.Lq ? g.nml[h * g.Lq + qi] : kNegInf;

  // kept tokens the block can see: J is ascending, so count J < limit
  const int32_t *Jh = g.J + h * g.kt_pad;
  int64_t ncount = g.kt;
  if (g.causal) {
    const int64_t limit = qb * kRows + kRows - 1 + g.off;   // last visible token of the block
    int64_t lo = 0, hi = g.kt;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if ((int64_t)Jh[mid] <= limit) lo = mid + 1;
      else hi = mid;
    }
    ncount = lo;
  }
  const int nt = (int)cdiv(ncount, kT);
  const rsrc_t rk = mg::make_rsrc(g.KJ + h * g.kt_pad * KF, (uint64_t)g.kt_pad * KF * 2);
  const rsrc_t rv = mg::make_rsrc(g.VJT + h * 128 * g.kt_pad, (uint64_t)128 * g.kt_pad * 2);
  const rsrc_t rj = mg::make_rsrc(Jh, (uint64_t)g.kt_pad * 4);

  auto issue = [&](int t, unsigned char *dst) {
    const int64_t j0 = (int64_t)t * kT;
    issue_tile<KF>(rk, j0, dst, wave, lane);
    // V_J^T rows d (128), kept positions j0 .. j0+63: same swizzled 128-byte rows
#pragma unroll
    for (int i = 0; i < VT_PER_WAVE; ++i) {
      const int q = i * kWaves + wave;   // 16 blocks of 8 rows
      const int row = q * 8 + lane / 8, slot = lane % 8;
      const int logical = slot ^ ((row ^ (row >> 3)) & 7);
      lds_load16(rv, dst + Tile<KF>::BYTES + q * 1024,
                   (uint32_t)(((int64_t)row * g.kt_pad + j0 + logical * 8) * 2), 0);
    }
    if (wave == 0) lds_load4(rj, dst + Tile<KF>::BYTES + VT_BYTES, (uint32_t)((j0 + lane) * 4), 0);
  };
  constexpr int LPW = Tile<KF>::PER_WAVE + VT_PER_WAVE;

  f32x16_t acc_o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;

  if (nt > 0) issue(0, smem);
  for (int t = 0; t < nt; ++t) {
    unsigned char *cur = smem + (t & 1) * STAGE;
    if (t + 1 < nt) {
      issue(t + 1, smem + ((t + 1) & 1) * STAGE);
      if (wave == 0) __builtin_amdgcn_s_waitcnt(vm_imm(LPW + 1));
      else __builtin_amdgcn_s_waitcnt(vm_imm(LPW));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
    }
    // A bare barrier after the explicit wait: __syncthreads would also wait
    // for the next tile's loads, which must stay in flight.
    __builtin_amdgcn_s_barrier();
    const int32_t *jt = reinterpret_cast<const int32_t *>(cur + Tile<KF>::BYTES + VT_BYTES);
    const uint16_t *vt = reinterpret_cast<const uint16_t *>(cur + Tile<KF>::BYTES);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KF / 16; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag<KF>(cur, sub * 32 + (lane & 31), ks, lk), qf[ks],
                                                      acc, 0, 0, 0);
      // p for the lane's query and the 16 kept rows it holds; every query of
      // the wave sees every token of the slice unless the slice crosses the
      // diagonal or the end of the kept list (tokens ascend: test the last).
      const int js0 = t * kT + sub * 32;
      const bool full = js0 + 31 < kt && (!g.causal || jt[sub * 32 + 31] <= q0 + off);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fexp2(fmaf(acc[r], g.c2, nml));
      if (!full) {
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
          const int rr = sub * 32 + 8 * b4 + 4 * lk;   // tile row of register 4*b4
          const int4 tv = *reinterpret_cast<const int4 *>(&jt[rr]);
          const int32_t tok[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jpos = t * kT + rr + e;
            const bool ok = jpos < kt && tok[e] >= 0 && (!g.causal || tok[e] <= qi + off);
            p[4 * b4 + e] = ok ? p[4 * b4 + e] : 0.f;
          }
        }
      }
      // two 16-token K-slices of the P V product from this 32-token slice
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // lane < 32 needs tokens 16kk+0..7: holds 0..3 (r = 8kk..8kk+3), gets 4..7 from its partner
        // lane >= 32 needs 16kk+8..15: holds 12..15 (r = 8kk+4..8kk+7), gets 8..11 from its partner
        const uint32_t own_lo = pack_bf16x2(p[8 * kk + 0], p[8 * kk + 1]);
        const uint32_t own_hi = pack_bf16x2(p[8 * kk + 2], p[8 * kk + 3]);
        const uint32_t nxt_lo = pack_bf16x2(p[8 * kk + 4], p[8 * kk + 5]);
        const uint32_t nxt_hi = pack_bf16x2(p[8 * kk + 6], p[8 * kk + 7]);
        const uint32_t send_lo = lk ? own_lo : nxt_lo, send_hi = lk ? own_hi : nxt_hi;
        const uint32_t got_lo = (uint32_t)__shfl_xor((int)send_lo, 32, 64);
        const uint32_t got_hi = (uint32_t)__shfl_xor((int)send_hi, 32, 64);
        const uint4 pa = lk ? make_uint4(got_lo, got_hi, nxt_lo, nxt_hi) : make_uint4(own_lo, own_hi, got_lo, got_hi);
        const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, pa);
        const int ksv = sub * 2 + kk;   // 16-token slice of the 64-token tile
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8_t vfrag = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4 *>(&vt[mg::swz(dt * 32 + (lane & 31), ksv * 2 + lk)]));
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pfrag, vfrag, acc_o[dt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // LDS reads of `cur` drained; the next tile's loads stay in flight
    __builtin_amdgcn_s_barrier();
  }
  // acc_o[dt]: lane holds column d = dt*32 + l%32 and queries q0 + 8*(r/4) + 4*(l/32) + r%4
  uint16_t *Oh = g.O + h * g.o_hs;
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t q = q0 + 8 * (r >> 2) + 4 * lk + (r & 3);
      if (q < g.Lq) {
        const uint16_t b = f32_to_bf16(acc_o[dt][r]);
        Oh[q * g.o_ts + dt * 32 + (lane & 31)] = b;
        const float v = bf16_to_f32(b);
        cs[dt] = fmaf(v, v, cs[dt]);
      }
    }
  if (g.opart) {
    __syncthreads();   // the tile stages are free: reuse them for the wave sums
    out_col_partials<kWaves>(cs, wave, lane, reinterpret_cast<float *>(smem),
                             g.opart + (qb * g.hq + h) * 128);
  }
}

// ---------------------------------------------------------------- pass D, 64 queries per wave
// The same output pass with 4 waves of 64 queries (two 32-query groups) per
// workgroup: every K_J and V_J^T fragment read from LDS feeds the MFMAs of
// both groups, which halves the LDS traffic per product, and the two groups'
// independent MFMA and exponential work can overlap within the wave.
constexpr int kWaves2 = 4;
constexpr int kThreads2 = 64 * kWaves2;

template <int KF>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(2))) void attn_out2_kernel(AttnArgs g) {
  constexpr int VT_BYTES = 128 * kT * 2;                      // V_J^T tile [128 d][64 kept]
  constexpr int STAGE = Tile<KF>::BYTES + VT_BYTES + kT * 4;  // + kept token ids
  constexpr int K_PER_WAVE = Tile<KF>::BLOCKS / kWaves2;
  constexpr int VT_PER_WAVE = VT_BYTES / 1024 / kWaves2;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, lk = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t qb = g.blocks_q - 1 - (int64_t)blockIdx.x / g.hq;
  const int64_t h = (int64_t)blockIdx.x % g.hq;
  const int64_t q0l = qb * kRows + 64 * wave;
  bf16x8_t qf[2][KF / 16];
  load_row_frags<KF>(g.QI + h * g.Lq * KF, g.Lq, q0l, lane, qf[0]);
  load_row_frags<KF>(g.QI + h * g.Lq * KF, g.Lq, q0l + 32, lane, qf[1]);
  const int off = (int)g.off, kt = (int)g.kt, q0 = (int)q0l;
  float nml[2];
#pragma unroll
  for (int gq = 0; gq < 2; ++gq) {
    const int qi = q0 + 32 * gq + (lane & 31);
    nml[gq] = qi < g.Lq ? g.nml[h * g.Lq + qi] : kNegInf;
  }

  // kept tokens the block can see: J is ascending, so count J < limit
  const int32_t *Jh = g.J + h * g.kt_pad;
  int64_t ncount = g.kt;
  if (g.causal) {
    const int64_t limit = qb * kRows + kRows - 1 + g.off;   // last visible token of the block
    int64_t lo = 0, hi = g.kt;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if ((int64_t)Jh[mid] <= limit) lo = mid + 1;
      else hi = mid;
    }
    ncount = lo;
  }
  const int nt = (int)cdiv(ncount, kT);
  const rsrc_t rk = mg::make_rsrc(g.KJ + h * g.kt_pad * KF, (uint64_t)g.kt_pad * KF * 2);
  const rsrc_t rv = mg::make_rsrc(g.VJT + h * 128 * g.kt_pad, (uint64_t)128 * g.kt_pad * 2);
  const rsrc_t rj = mg::make_rsrc(Jh, (uint64_t)g.kt_pad * 4);

  auto issue = [&](int t, unsigned char *dst) {
    const int64_t j0 = (int64_t)t * kT;
    issue_tile<KF, kWaves2>(rk, j0, dst, wave, lane);
#pragma unroll
    for (int i = 0; i < VT_PER_WAVE; ++i) {
      const int q = i * kWaves2 + wave;   // 16 blocks of 8 rows
      const int row = q * 8 + lane / 8, slot = lane % 8;
      const int logical = slot ^ ((row ^ (row >> 3)) & 7);
      lds_load16(rv, dst + Tile<KF>::BYTES + q * 1024,
                 (uint32_t)(((int64_t)row * g.kt_pad + j0 + logical * 8) * 2), 0);
    }
    if (wave == 0) lds_load4(rj, dst + Tile<KF>::BYTES + VT_BYTES, (uint32_t)((j0 + lane) * 4), 0);
  };
  constexpr int LPW = K_PER_WAVE + VT_PER_WAVE;

  f32x16_t acc_o[2][4];
#pragma unroll
  for (int gq = 0; gq < 2; ++gq)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[gq][dt][r] = 0.f;

  if (nt > 0) issue(0, smem);
  for (int t = 0; t < nt; ++t) {
    unsigned char *cur = smem + (t & 1) * STAGE;
    if (t + 1 < nt) {
      issue(t + 1, smem + ((t + 1) & 1) * STAGE);
      if (wave == 0) __builtin_amdgcn_s_waitcnt(vm_imm(LPW + 1));
      else __builtin_amdgcn_s_waitcnt(vm_imm(LPW));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_imm(0));
    }
    // A bare barrier after the explicit wait: __syncthreads would also wait
    // for the next tile's loads, which must stay in flight.
    __builtin_amdgcn_s_barrier();
    const int32_t *jt = reinterpret_cast<const int32_t *>(cur + Tile<KF>::BYTES + VT_BYTES);
    const uint16_t *vt = reinterpret_cast<const uint16_t *>(cur + Tile<KF>::BYTES);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int js0 = t * kT + sub * 32;
      const int last_tok = jt[sub * 32 + 31];
      bf16x8_t pf[2][2];
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        f32x16_t acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KF / 16; ++ks) {
          const bf16x8_t kf8 = lds_frag<KF>(cur, sub * 32 + (lane & 31), ks, lk);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf8, qf[gq][ks], acc, 0, 0, 0);
        }
        // Every query of the group sees every token of the slice unless the
        // slice crosses the diagonal or the end of the kept list.
        const int qg0 = q0 + 32 * gq;
        const bool full = js0 + 31 < kt && (!g.causal || last_tok <= qg0 + off);
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fexp2(fmaf(acc[r], g.c2, nml[gq]));
        if (!full) {
          const int qi = qg0 + (lane & 31);
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int rr = sub * 32 + 8 * b4 + 4 * lk;   // tile row of register 4*b4
            const int4 tv = *reinterpret_cast<const int4 *>(&jt[rr]);
            const int32_t tok[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int jpos = t * kT + rr + e;
              const bool ok = jpos < kt && tok[e] >= 0 && (!g.causal || tok[e] <= qi + off);
              p[4 * b4 + e] = ok ? p[4 * b4 + e] : 0.f;
            }
          }
        }
        // regroup into the A operand of two 16-token K-slices (see attn_out_kernel)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint32_t own_lo = pack_bf16x2(p[8 * kk + 0], p[8 * kk + 1]);
          const uint32_t own_hi = pack_bf16x2(p[8 * kk + 2], p[8 * kk + 3]);
          const uint32_t nxt_lo = pack_bf16x2(p[8 * kk + 4], p[8 * kk + 5]);
          const uint32_t nxt_hi = pack_bf16x2(p[8 * kk + 6], p[8 * kk + 7]);
          const uint32_t send_lo = lk ? own_lo : nxt_lo, send_hi = lk ? own_hi : nxt_hi;
          const uint32_t got_lo = (uint32_t)__shfl_xor((int)send_lo, 32, 64);
          const uint32_t got_hi = (uint32_t)__shfl_xor((int)send_hi, 32, 64);
          const uint4 pa = lk ? make_uint4(got_lo, got_hi, nxt_lo, nxt_hi) : make_uint4(own_lo, own_hi, got_lo, got_hi);
          pf[gq][kk] = __builtin_bit_cast(bf16x8_t, pa);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ksv = sub * 2 + kk;   // 16-token slice of the 64-token tile
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8_t vfrag = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const uint4 *>(&vt[mg::swz(dt * 32 + (lane & 31), ksv * 2 + lk)]));
          acc_o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[0][kk], vfrag, acc_o[0][dt], 0, 0, 0);
          acc_o[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[1][kk], vfrag, acc_o[1][dt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // LDS reads of `cur` drained; the next tile's loads stay in flight
    __builtin_amdgcn_s_barrier();
  }
  uint16_t *Oh = g.O + h * g.o_hs;
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gq = 0; gq < 2; ++gq)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t q = q0 + 32 * gq + 8 * (r >> 2) + 4 * lk + (r & 3);
        if (q < g.Lq) {
          const uint16_t b = f32_to_bf16(acc_o[gq][dt][r]);
          Oh[q * g.o_ts + dt * 32 + (lane & 31)] = b;
          const float v = bf16_to_f32(b);
          cs[dt] = fmaf(v, v, cs[dt]);
        }
      }
  if (g.opart) {
    __syncthreads();   // the tile stages are free: reuse them for the wave sums
    out_col_partials<kWaves2>(cs, wave, lane, reinterpret_cast<float *>(smem),
                              g.opart + (qb * g.hq + h) * 128);
  }
}

// Rows of K_I gathered by the kept tokens: KJ[h][j] = KI[h][J[h][j]] (zero rows
// for padding).  One thread per 16-byte chunk.
template <int KF>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ KI, int64_t Lk,
                                                          const int32_t *__restrict__ J, int64_t kt_pad,
                                                          uint16_t *__restrict__ KJ, int64_t total) {
  constexpr int CPR = KF / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int64_t row = c / CPR, ch = c % CPR;   // row over [hq][kt_pad]
  const int64_t h = row / kt_pad;
  const int32_t t = J[row];
  uint4 v = make_uint4(0, 0, 0, 0);
  if (t >= 0 && t < Lk) v = *reinterpret_cast<const uint4 *>(KI + ((h * Lk + t) * KF + ch * 8));
  *reinterpret_cast<uint4 *>(KJ + row * KF + ch * 8) = v;
}

}  // namespace

bool attn_supported(int64_t dh, int64_t kf_pad) { return dh == 128 && (kf_pad == 64 || kf_pad == 128); }

hipError_t launch_attn_passes(int pass, const AttnDesc &d, hipStream_t st) {
  AttnArgs g{};
  g.QI = static_cast<const uint16_t *>(d.QI);
  g.KI = static_cast<const uint16_t *>(d.KI);
  g.KJ = static_cast<const uint16_t *>(d.KJ);
  g.VJT = static_cast<const uint16_t *>(d.VJT);
  g.J = d.J;
  g.nml = d.nml;
  g.n2ml = d.n2ml;
  g.tok = d.tok;
  g.opart = d.opart;
  g.O = static_cast<uint16_t *>(d.O);
  g.o_ts = d.o_ts;
  g.o_hs = d.o_hs;
  g.hq = d.hq;
  g.Lq = d.Lq;
  g.Lk = d.Lk;
  g.kt = d.kt;
  g.kt_pad = d.kt_pad;
  g.causal = d.causal ? 1 : 0;
  g.off = d.Lk - d.Lq;
  g.c2 = (float)(1.4426950408889634 / __builtin_sqrt((double)d.dh));
  g.blocks_q = ceil_div(d.Lq, kRows);
  g.blocks_k = ceil_div(d.Lk, kRows);
  const bool kf128 = d.kf_pad == 128;
  if (pass == 0) {
    KernelTimer timer("attn_stats", st);
    dim3 grid((unsigned)(g.blocks_q * g.hq));
    if (kf128) hipLaunchKernelGGL(attn_stats_kernel<128>, grid, dim3(kThreads), 0, st, g);
    else hipLaunchKernelGGL(attn_stats_kernel<64>, grid, dim3(kThreads), 0, st, g);
  } else if (pass == 1) {
    KernelTimer timer("attn_colsq", st);
    dim3 grid((unsigned)(g.blocks_k * g.hq));
    if (kf128) hipLaunchKernelGGL(attn_colsq_kernel<128>, grid, dim3(kThreads), 0, st, g);
    else hipLaunchKernelGGL(attn_colsq_kernel<64>, grid, dim3(kThreads), 0, st, g);
  } else if (pass == 2) {
    KernelTimer timer("attn_gather", st);
    const int64_t total = d.hq * d.kt_pad * (d.kf_pad / 8);
    dim3 grid((unsigned)ceil_div(total, 256));
    if (kf128)
      hipLaunchKernelGGL(gather_rows_kernel<128>, grid, dim3(256), 0, st, g.KI, d.Lk, d.J, d.kt_pad,
                         static_cast<uint16_t *>(d.KJ), total);
    else
      hipLaunchKernelGGL(gather_rows_kernel<64>, grid, dim3(256), 0, st, g.KI, d.Lk, d.J, d.kt_pad,
                         static_cast<uint16_t *>(d.KJ), total);
  } else {
    KernelTimer timer("attn_out", st);
    dim3 grid((unsigned)(g.blocks_q * g.hq));
    if (kf128) hipLaunchKernelGGL(attn_out_kernel<128>, grid, dim3(kThreads), 0, st, g);
    else hipLaunchKernelGGL(attn_out2_kernel<64>, grid, dim3(kThreads2), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace rmm

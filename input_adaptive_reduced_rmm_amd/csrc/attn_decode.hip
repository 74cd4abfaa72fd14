// Reduced attention for a few new tokens after a long context (decode steps,
// Lq <= 16): the same computation as the fused path in attn.hip - features of
// Q selected by column norm, S = Q[:, I] K[I, :], causal softmax, tokens
// selected by the column norms of P, O = P[:, J] V[J, :] ("Alcance de
// Aplicación", "Estrategia de Selección") - organised for Lq << Lk.
//
// With so few query rows the work is reading the kept feature rows of K and
// the kept token rows of V once, so every pass is split over keys (or kept
// tokens) across many workgroups per head instead of over query blocks:
//   dec_scores  S[i][j] for all keys, straight from the feature-major K
//               (each kept feature row of a 256-key block is 512 contiguous
//               bytes), written to the workspace (Lq x Lk floats per head),
//               with each block's per-query max and sum of 2^(c (S - max));
//   dec_tok_select  one workgroup per head: merges those partial
//               statistics, forms the token scores sqrt(sum_i P_ij^2),
//               P_ij = 2^(c S_ij + nml_i), keeps them in LDS and selects the
//               kept tokens there (contexts up to kSelKeys; longer ones write
//               the scores with dec_tok and select with the top-k kernel);
//   dec_out     per block of 256 kept tokens: P_ij from S, the kept V rows
//               (16-byte loads), partial O sums per (block, head);
//   dec_merge   adds the partial O in block order, rounds to bf16 and (when
//               asked) forms the column scores of O.
// With one new token, the feature selection (|q_f| over the 128 features,
// top k_feat) is one wave per head (dec_feat1).  Everything is float32
// except the bf16 inputs and O; all sums run in a fixed order, so results
// are deterministic.
//
// A batch of sequences (a decode step over several caches) runs through the
// same passes with the (sequence, head) pairs as the rows: each pair reads
// its own sequence's Q, K and V at the sequence strides, its context length
// and kept-token count come from device arrays, and keys past a sequence's
// length score -inf (never selected, weight zero).
#include "rmm_internal.h"
#include "select.h"
#include "timing.h"

namespace rmm {
namespace {

constexpr int kDB = 256;   // keys (or kept tokens) per workgroup pass, one per thread
constexpr int kTokSub = 1;   // 256-token sub-tiles per output workgroup
constexpr int kSelThreads = 1024;   // token selection workgroup
constexpr int kSelKeys = 32768;     // most token scores the selection holds in LDS (128 KiB)
constexpr float kNegInfD = -__builtin_inff();

__device__ __forceinline__ float dexp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct DecArgs {
  const uint16_t *Q;      // element (i, h, f) at Q + i*q_ts + h*q_hs + f
  int64_t q_ts, q_hs;
  const uint16_t *Kt;     // element (g, f, j) at Kt + g*kt_hs + f*ldkt + j
  int64_t kt_hs, ldkt;
  const uint16_t *V;      // element (j, g, d) at V + j*v_ts + g*v_hs + d
  int64_t v_ts, v_hs;
  const int32_t *I;       // [hq][kf_pad] kept features, ascending
  const int32_t *J;       // [hq][kt_pad] kept tokens, ascending
  int32_t *Jw;            // the same rows, written by the token selection
  float *S;               // [hq][Lq][Lk]
  float2 *pstat;          // [hq][nblk][Lq] (block max of S, sum of 2^(c (S - max)))
  float *nml;             // [hq][Lq]
  float *tok;             // [hq][Lk] (the fused selection writes it only when not null)
  float *opart;           // [nsplit][hq][Lq][128]
  uint16_t *O;            // element (i, h, d) at O + i*o_ts + h*o_hs + d
  int64_t o_ts, o_hs;
  float *o_scores;        // [hq][128] or null
  int64_t hq, hkv, Lq, Lk, kf, kf_pad, kt, kt_pad, off;
  int causal, nblk, nsplit;
  float c2;
  // batch of sequences: row r = b * hq + h; Lk is the longest context
  int64_t q_ss, kt_ss, v_ss, o_ss;
  const int32_t *lens;    // [nseq] context lengths (null: Lk for all)
  const int32_t *kts;     // [nseq] kept tokens (null: kt for all)
  int64_t nrows;          // nseq * hq: rows of I, J, S, pstat, nml, tok and opart
  int sblk_keys;          // keys per score block (one pstat entry)
  int kvec;               // K rows 16-byte aligned (pointer and strides multiples of 8 elements)
};

// The sequence of row r, its context length, its causal offset and its
// kept-token count.
struct SeqRow {
  int64_t b, h, Lk, off, kt;
};
__device__ __forceinline__ SeqRow seq_row(const DecArgs &g, int64_t r) {
  SeqRow q;
  q.b = r / g.hq;
  q.h = r - q.b * g.hq;
  q.Lk = g.Lk;
  if (g.lens) {
    const int64_t L = g.lens[q.b];
    q.Lk = L < 1 ? 1 : (L > g.Lk ? g.Lk : L);
  }
  q.off = q.Lk - g.Lq;
  q.kt = g.kt;
  if (g.kts) {   // clamped to [1, min(Lk of the row, kt)] as the top-k clamps it
    const int64_t k = g.kts[q.b], kmax = q.Lk < g.kt ? q.Lk : g.kt;
    q.kt = k < 1 ? 1 : (k > kmax ? kmax : k);
  }
  return q;
}

// Block-wide reduction of LQ values per thread (max or sum) over NW waves;
// returns the result to every thread.  Waves are combined by a pairwise tree
// in wave order.  red: LDS scratch of NW * LQ floats.
template <int LQ, bool MAX, int NW = 4>
__device__ __forceinline__ void block_reduce(float (&v)[LQ], float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float w = __shfl_xor(v[i], o, 64);
      v[i] = MAX ? fmaxf(v[i], w) : v[i] + w;
    }
  }
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < LQ; ++i) red[wave * LQ + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    float t[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) t[w] = red[w * LQ + i];
#pragma unroll
    for (int st = 1; st < NW; st *= 2)
#pragma unroll
      for (int w = 0; w + st < NW; w += 2 * st) t[w] = MAX ? fmaxf(t[w], t[w + st]) : t[w] + t[w + st];
    v[i] = t[0];
  }
}

template <int LQ>
__global__ __launch_bounds__(kDB) void dec_scores_kernel(DecArgs g) {
  __shared__ int32_t sI[128];
  __shared__ __attribute__((aligned(16))) float sq[LQ][128];
  __shared__ float red[4 * LQ];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int64_t h = blockIdx.y;   // row: sequence * hq + head
  const SeqRow sr = seq_row(g, h);
  const int64_t grp = sr.h * g.hkv / g.hq;
  const int Lq = (int)g.Lq, kf = (int)g.kf;
  if (tid < 128) sI[tid] = tid < kf ? g.I[h * g.kf_pad + tid] : 0;
  __syncthreads();
  for (int e = tid; e < LQ * 128; e += kDB) {
    const int i = e / 128, f = e % 128;
    sq[i][f] = (i < Lq && f < kf) ? bf16_to_f32(g.Q[sr.b * g.q_ss + i * g.q_ts + sr.h * g.q_hs + sI[f]]) : 0.f;
  }
  __syncthreads();
  const int64_t j = (int64_t)blk * kDB + tid;
  float s[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) s[i] = 0.f;
  if (j < sr.Lk) {
    const uint16_t *kb = g.Kt + sr.b * g.kt_ss + grp * g.kt_hs + j;
    int f = 0;
    for (; f + 8 <= kf; f += 8) {
      float kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = bf16_to_f32(kb[(int64_t)sI[f + u] * g.ldkt]);
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        // two 16-byte LDS reads (broadcast) per query row and 8 features
        const float4 qa = *reinterpret_cast<const float4 *>(&sq[i][f]);
        const float4 qb = *reinterpret_cast<const float4 *>(&sq[i][f + 4]);
        s[i] = fmaf(qa.x, kv[0], s[i]);
        s[i] = fmaf(qa.y, kv[1], s[i]);
        s[i] = fmaf(qa.z, kv[2], s[i]);
        s[i] = fmaf(qa.w, kv[3], s[i]);
        s[i] = fmaf(qb.x, kv[4], s[i]);
        s[i] = fmaf(qb.y, kv[5], s[i]);
        s[i] = fmaf(qb.z, kv[6], s[i]);
        s[i] = fmaf(qb.w, kv[7], s[i]);
      }
    }
    for (; f < kf; ++f) {
      const float kv = bf16_to_f32(kb[(int64_t)sI[f] * g.ldkt]);
#pragma unroll
      for (int i = 0; i < LQ; ++i) s[i] = fmaf(sq[i][f], kv, s[i]);
    }
  }
  // masked scores are -inf: they add nothing to any later sum
#pragma unroll
  for (int i = 0; i < LQ; ++i) {
    const bool vis = j < sr.Lk && i < Lq && (!g.causal || j <= i + sr.off);
    s[i] = vis ? s[i] : kNegInfD;
    if (i < Lq && j < g.Lk) g.S[(h * g.Lq + i) * g.Lk + j] = s[i];
  }
  float m[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) m[i] = s[i];
  block_reduce<LQ, true>(m, red);
  float l[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) l[i] = m[i] == kNegInfD ? 0.f : dexp2((s[i] - m[i]) * g.c2);
  block_reduce<LQ, false>(l, red);
  if (tid < Lq) {
    float mv = m[0], lv = l[0];
#pragma unroll
    for (int i = 1; i < LQ; ++i)
      if (tid == i) { mv = m[i]; lv = l[i]; }
    g.pstat[(h * g.nblk + blk) * g.Lq + tid] = make_float2(mv, lv);
  }
}

// One query row (a single new token): each thread takes 8 consecutive keys,
// so a kept feature row of K is read as one 16-byte load per thread (a block
// covers 2048 keys).  Blocks wholly past a sequence's context exit at once;
// the statistics merge reads only the blocks a row has.
constexpr int kKPT = 8, kSB1 = kDB * kKPT;
__global__ __launch_bounds__(kDB) void dec_scores1_kernel(DecArgs g) {
  __shared__ int32_t sI[128];
  __shared__ float sq[128];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int64_t h = blockIdx.y;   // row: sequence * hq + head
  const SeqRow sr = seq_row(g, h);
  const int64_t jb = (int64_t)blk * kSB1;
  if (jb >= sr.Lk) return;
  const int64_t grp = sr.h * g.hkv / g.hq;
  const int kf = (int)g.kf;
  if (tid < 128) {
    const int f = tid < kf ? g.I[h * g.kf_pad + tid] : 0;
    sI[tid] = f;
    sq[tid] = tid < kf ? bf16_to_f32(g.Q[sr.b * g.q_ss + sr.h * g.q_hs + f]) : 0.f;
  }
  __syncthreads();
  const int64_t j0 = jb + (int64_t)tid * kKPT;
  float s[kKPT];
#pragma unroll
  for (int e = 0; e < kKPT; ++e) s[e] = 0.f;
  const uint16_t *kb = g.Kt + sr.b * g.kt_ss + grp * g.kt_hs + j0;
  if (g.kvec && j0 + kKPT <= sr.Lk) {
    int f = 0;
    for (; f + 4 <= kf; f += 4) {
      uint4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kv[u] = *reinterpret_cast<const uint4 *>(kb + (int64_t)sI[f + u] * g.ldkt);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float q = sq[f + u];
        const float kx[8] = {bf16_lo(kv[u].x), bf16_hi(kv[u].x), bf16_lo(kv[u].y), bf16_hi(kv[u].y),
                             bf16_lo(kv[u].z), bf16_hi(kv[u].z), bf16_lo(kv[u].w), bf16_hi(kv[u].w)};
#pragma unroll
        for (int e = 0; e < kKPT; ++e) s[e] = fmaf(q, kx[e], s[e]);
      }
    }
    for (; f < kf; ++f) {
      const uint4 kv = *reinterpret_cast<const uint4 *>(kb + (int64_t)sI[f] * g.ldkt);
      const float q = sq[f];
      const float kx[8] = {bf16_lo(kv.x), bf16_hi(kv.x), bf16_lo(kv.y), bf16_hi(kv.y),
                           bf16_lo(kv.z), bf16_hi(kv.z), bf16_lo(kv.w), bf16_hi(kv.w)};
#pragma unroll
      for (int e = 0; e < kKPT; ++e) s[e] = fmaf(q, kx[e], s[e]);
    }
  } else if (j0 < sr.Lk) {
    for (int f = 0; f < kf; ++f) {
      const float q = sq[f];
      const uint16_t *kr = kb + (int64_t)sI[f] * g.ldkt;
#pragma unroll
      for (int e = 0; e < kKPT; ++e)
        if (j0 + e < sr.Lk) s[e] = fmaf(q, bf16_to_f32(kr[e]), s[e]);
    }
  }
  // masked scores are -inf: they add nothing to any later sum
  float m = kNegInfD;
#pragma unroll
  for (int e = 0; e < kKPT; ++e) {
    const int64_t j = j0 + e;
    const bool vis = j < sr.Lk && (!g.causal || j <= sr.off);
    s[e] = vis ? s[e] : kNegInfD;
    m = fmaxf(m, s[e]);
    if (j < g.Lk) g.S[h * g.Lk + j] = s[e];
  }
  float mv[1] = {m};
  block_reduce<1, true>(mv, red);
  float l = 0.f;
  if (mv[0] != kNegInfD) {
#pragma unroll
    for (int e = 0; e < kKPT; ++e) l += dexp2((s[e] - mv[0]) * g.c2);
  }
  float lv[1] = {l};
  block_reduce<1, false>(lv, red);
  if (tid == 0) g.pstat[h * g.nblk + blk] = make_float2(mv[0], lv[0]);
}

// Merge the key blocks' statistics of head h: every thread takes the blocks
// b = tid, tid + 256, ... (loads independent of each other), then block-wide
// max and sum in a fixed order.  Returns nml_i = -c max_i - log2(sum_i).
template <int LQ, int NW = 4>
__device__ __forceinline__ void merge_stats(const DecArgs &g, int64_t h, float (&nml)[LQ], float *red) {
  const int tid = threadIdx.x, Lq = (int)g.Lq;
  // blocks this row has (a shorter sequence has fewer)
  const int nb = g.lens ? (int)((seq_row(g, h).Lk + g.sblk_keys - 1) / g.sblk_keys) : g.nblk;
  float M[LQ], L[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) M[i] = kNegInfD;
  for (int b = tid; b < nb; b += 64 * NW)
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      if (i < Lq) M[i] = fmaxf(M[i], g.pstat[(h * g.nblk + b) * g.Lq + i].x);
  block_reduce<LQ, true, NW>(M, red);
#pragma unroll
  for (int i = 0; i < LQ; ++i) L[i] = 0.f;
  for (int b = tid; b < nb; b += 64 * NW)
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      if (i < Lq) {
        const float2 p = g.pstat[(h * g.nblk + b) * g.Lq + i];
        if (p.x != kNegInfD) L[i] += p.y * dexp2((p.x - M[i]) * g.c2);
      }
  block_reduce<LQ, false, NW>(L, red);
#pragma unroll
  for (int i = 0; i < LQ; ++i) nml[i] = (i < Lq && L[i] > 0.f) ? -M[i] * g.c2 - log2f(L[i]) : kNegInfD;
}

template <int LQ>
__global__ __launch_bounds__(kDB) void dec_tok_kernel(DecArgs g) {
  __shared__ float red[4 * LQ];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int64_t h = blockIdx.y;
  const int Lq = (int)g.Lq;
  if (g.lens && (int64_t)blk * kDB >= seq_row(g, h).Lk) {   // wholly past this sequence's context
    const int64_t j = (int64_t)blk * kDB + tid;
    if (j < g.Lk) g.tok[h * g.Lk + j] = kNegInfD;
    return;
  }
  float snml[LQ];
  merge_stats<LQ>(g, h, snml, red);
  if (blk == 0 && tid < Lq) {
    float v = snml[0];
#pragma unroll
    for (int i = 1; i < LQ; ++i)
      if (tid == i) v = snml[i];
    g.nml[h * g.Lq + tid] = v;
  }
  const int64_t j = (int64_t)blk * kDB + tid;
  if (j >= g.Lk) return;
  if (g.lens && j >= seq_row(g, h).Lk) {   // past this sequence's context: never kept
    g.tok[h * g.Lk + j] = kNegInfD;
    return;
  }
  const float c4 = 2.f * g.c2;
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < LQ; ++i)
    if (i < Lq) {
      const float sv = g.S[(h * g.Lq + i) * g.Lk + j];
      if (sv != kNegInfD) t += dexp2(fmaf(sv, c4, 2.f * snml[i]));
    }
  g.tok[h * g.Lk + j] = __builtin_sqrtf(t);
}

// Token scores and token selection of row h in one workgroup (Lk <= kSelKeys):
// the statistics merge of dec_tok (same partial order, so the same nml and
// scores), every score computed once, parked in LDS as an order-preserving
// key and, when asked, written to tok; then sel::block_select keeps the row's
// kt highest (ties to the lower index) into J.  Keys past the row's context
// score -inf and are never kept (kt <= the row's context), so the select runs
// over the row's own context only.  The keys take Lk x 4 bytes of dynamic
// LDS: two workgroups share a CU while Lk <= 16384.
template <int LQ>
__global__ __launch_bounds__(kSelThreads) void dec_tok_select_kernel(DecArgs g) {
  constexpr int NW = kSelThreads / 64;
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];
  __shared__ sel::BlockShared<kSelThreads> sh;
  __shared__ float red[NW * LQ];
  const int tid = threadIdx.x;
  const int64_t h = blockIdx.x;
  const int Lq = (int)g.Lq;
  const SeqRow sr = seq_row(g, h);
  float snml[LQ];
  merge_stats<LQ, NW>(g, h, snml, red);
  if (tid < Lq) {
    float v = snml[0];
#pragma unroll
    for (int i = 1; i < LQ; ++i)
      if (tid == i) v = snml[i];
    g.nml[h * g.Lq + tid] = v;
  }
  const float c4 = 2.f * g.c2;
  // Every token of the context kept: the selection is the identity (as the
  // top-k kernel's k == d case), and the scores are formed only when asked.
  const bool keep_all = sr.kt >= sr.Lk;
  if (keep_all && !g.tok) {
    for (int64_t t = tid; t < g.kt_pad; t += kSelThreads) g.Jw[h * g.kt_pad + t] = t < sr.kt ? (int32_t)t : -1;
    return;
  }
  uint32_t kor = 0u, kand = 0xFFFFFFFFu;
  // Token score of key j from its Lq values of S (-inf past the context).
  auto score = [&](const float (&sv)[LQ], int64_t j) -> float {
    if (j >= sr.Lk) return kNegInfD;   // past this sequence's context: never kept
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < LQ; ++i)
      if (i < Lq && sv[i] != kNegInfD) a += dexp2(fmaf(sv[i], c4, 2.f * snml[i]));
    return __builtin_sqrtf(a);
  };
  if (g.Lk % 4 == 0) {
    // four keys per thread and load (S rows are 16-byte aligned), U groups
    // of them with their loads in flight together
    constexpr int U = LQ <= 2 ? 2 : 1;
    const int64_t n4 = g.Lk / 4;
    const bool tok16 = g.tok && reinterpret_cast<uintptr_t>(g.tok) % 16 == 0;
    const float4 *S4 = reinterpret_cast<const float4 *>(g.S);
    for (int64_t t0 = tid; t0 < n4; t0 += (int64_t)U * kSelThreads) {
      float4 v[U][LQ];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + (int64_t)u * kSelThreads;
#pragma unroll
        for (int i = 0; i < LQ; ++i)
          v[u][i] = (i < Lq && t < n4) ? S4[(h * g.Lq + i) * n4 + t]
                                       : make_float4(kNegInfD, kNegInfD, kNegInfD, kNegInfD);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + (int64_t)u * kSelThreads;
        if (t >= n4) break;
        float sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sv[LQ];
#pragma unroll
          for (int i = 0; i < LQ; ++i) sv[i] = e == 0 ? v[u][i].x : e == 1 ? v[u][i].y : e == 2 ? v[u][i].z : v[u][i].w;
          sc[e] = score(sv, 4 * t + e);
        }
        if (tok16) *reinterpret_cast<float4 *>(&g.tok[h * g.Lk + 4 * t]) = make_float4(sc[0], sc[1], sc[2], sc[3]);
        else if (g.tok)
#pragma unroll
          for (int e = 0; e < 4; ++e) g.tok[h * g.Lk + 4 * t + e] = sc[e];
        const uint4 key = make_uint4(sel::score_key(sc[0]), sel::score_key(sc[1]), sel::score_key(sc[2]),
                                     sel::score_key(sc[3]));
        *reinterpret_cast<uint4 *>(&keys[4 * t]) = key;
        const uint32_t kk[4] = {key.x, key.y, key.z, key.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * t + e < sr.Lk) {
            kor |= kk[e];
            kand &= kk[e];
          }
      }
    }
  } else {
    // U keys per thread at a time: their S loads are in flight together
    constexpr int U = LQ <= 2 ? 8 : LQ <= 4 ? 4 : 2;
    for (int64_t j0 = tid; j0 < g.Lk; j0 += (int64_t)U * kSelThreads) {
      float sv[U][LQ];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + (int64_t)u * kSelThreads;
#pragma unroll
        for (int i = 0; i < LQ; ++i)
          sv[u][i] = (i < Lq && j < sr.Lk) ? g.S[(h * g.Lq + i) * g.Lk + j] : kNegInfD;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + (int64_t)u * kSelThreads;
        if (j >= g.Lk) break;
        const float t = score(sv[u], j);
        if (g.tok) g.tok[h * g.Lk + j] = t;
        const uint32_t key = sel::score_key(t);
        keys[j] = key;
        if (j < sr.Lk) {
          kor |= key;
          kand &= key;
        }
      }
    }
  }
  if (keep_all) {
    for (int64_t t = tid; t < g.kt_pad; t += kSelThreads) g.Jw[h * g.kt_pad + t] = t < sr.kt ? (int32_t)t : -1;
    return;
  }
  sel::block_select<kSelThreads>([&](int64_t j) -> uint32_t { return keys[j]; }, sr.Lk, kor, kand, sr.kt,
                                 g.kt_pad, g.Jw + h * g.kt_pad, sh);
}

template <int LQ>
__global__ __launch_bounds__(kDB) void dec_out_kernel(DecArgs g) {
  __shared__ int32_t sj[kDB];
  __shared__ float sp[kDB][LQ];
  __shared__ float red[4][LQ * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int64_t h = blockIdx.y;   // row: sequence * hq + head
  const SeqRow sr = seq_row(g, h);
  const int64_t grp = sr.h * g.hkv / g.hq;
  const uint16_t *Vs = g.V + sr.b * g.v_ss;
  const int Lq = (int)g.Lq;
  float nmli[LQ];
#pragma unroll
  for (int i = 0; i < LQ; ++i) nmli[i] = i < Lq ? g.nml[h * g.Lq + i] : kNegInfD;
  // thread: 8 output columns (dq) of 16 token lanes (tg); tokens tg, tg+16, ...
  const int dq = tid & 15, tg = tid >> 4;
  float acc[LQ][8];
#pragma unroll
  for (int i = 0; i < LQ; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int sub = 0; sub < kTokSub; ++sub) {
    const int64_t t0 = ((int64_t)split * kTokSub + sub) * kDB;
    if (t0 >= sr.kt) break;   // splits past this row's kept tokens write zero partials
    const int ntok = (int)(sr.kt - t0 < kDB ? sr.kt - t0 : kDB);
    if (sub > 0) __syncthreads();   // the previous sub-tile's p and rows are consumed
    {
      const int32_t jt = tid < ntok ? g.J[h * g.kt_pad + t0 + tid] : -1;
      sj[tid] = jt;
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        float p = 0.f;
        if (jt >= 0 && i < Lq) {
          const float sv = g.S[(h * g.Lq + i) * g.Lk + jt];
          if (sv != kNegInfD) p = dexp2(fmaf(sv, g.c2, nmli[i]));
        }
        sp[tid][i] = p;
      }
    }
    __syncthreads();
    for (int tt = tg; tt < ntok; tt += 16) {
      const int32_t row = sj[tt];
      if (row < 0) continue;
      const uint4 v = *reinterpret_cast<const uint4 *>(Vs + (int64_t)row * g.v_ts + grp * g.v_hs + dq * 8);
      const float vf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                           bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
      for (int i = 0; i < LQ; ++i) {
        const float p = sp[tt][i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(p, vf[e], acc[i][e]);
      }
    }
  }
  // add the four token lanes of a wave (lane bits 4 and 5), then the waves
#pragma unroll
  for (int i = 0; i < LQ; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[i][e] += __shfl_xor(acc[i][e], 16, 64);
      acc[i][e] += __shfl_xor(acc[i][e], 32, 64);
    }
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < LQ; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][i * 128 + dq * 8 + e] = acc[i][e];
  }
  __syncthreads();
  float *dst = g.opart + ((int64_t)split * g.nrows + h) * g.Lq * 128;
  for (int e = tid; e < Lq * 128; e += kDB) dst[e] = (red[0][e] + red[1][e]) + (red[2][e] + red[3][e]);
}

// Block per (head, 32 columns): O = sum of the split partials in split order
// (eight loads in flight), rounded to bf16; o_scores[h][d] = norm over the Lq
// rows of that bf16 O, rows added in order.
__global__ __launch_bounds__(256) void dec_merge_kernel(DecArgs g) {
  __shared__ float sq[16][32];
  const int64_t h = blockIdx.x;
  const int d0 = blockIdx.y * 32;
  const int Lq = (int)g.Lq;
  for (int e = threadIdx.x; e < Lq * 32; e += 256) {
    const int i = e / 32, d = d0 + e % 32;
    const float *p = g.opart + (h * g.Lq + i) * 128 + d;
    const int64_t stride = g.nrows * g.Lq * 128;
    float s = 0.f;
    int sp = 0;
    for (; sp + 8 <= g.nsplit; sp += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(sp + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; sp < g.nsplit; ++sp) s += p[(int64_t)sp * stride];
    const uint16_t b = f32_to_bf16(s);
    const int64_t sb = h / g.hq, sh = h - sb * g.hq;
    g.O[sb * g.o_ss + i * g.o_ts + sh * g.o_hs + d] = b;
    const float v = bf16_to_f32(b);
    sq[i][e % 32] = v * v;
  }
  if (!g.o_scores) return;
  __syncthreads();
  if (threadIdx.x < 32) {
    float cs = 0.f;
    for (int i = 0; i < Lq; ++i) cs += sq[i][threadIdx.x];
    g.o_scores[h * 128 + d0 + threadIdx.x] = __builtin_sqrtf(cs);
  }
}

// Feature selection of one new token per (sequence, head) row, one wave per
// row: scores |q_f| = sqrt(q_f^2) (the column norm over a single row, as the
// column-score kernel forms it), then the k_feat highest of the 128 features
// (ties to the lower index) into I, ascending.
__global__ __launch_bounds__(256) void dec_feat1_kernel(const uint16_t *__restrict__ Q, int64_t q_ss, int64_t q_hs,
                                                        int64_t hq, int64_t nrows, int kf, int kf_pad,
                                                        int32_t *__restrict__ I) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= nrows) return;   // whole waves
  const int64_t b = r / hq, h = r - b * hq;
  const uint16_t *q = Q + b * q_ss + h * q_hs;
  const float x0 = bf16_to_f32(q[lane]), x1 = bf16_to_f32(q[64 + lane]);
  sel::wave_select128(sel::score_key(__builtin_sqrtf(x0 * x0)), sel::score_key(__builtin_sqrtf(x1 * x1)), kf,
                      kf_pad, I + r * kf_pad);
}

}  // namespace

hipError_t launch_dec_feat1(const void *Q, int64_t q_ss, int64_t q_hs, int64_t nseq, int64_t hq, int64_t kf,
                            int64_t kf_pad, int32_t *I, hipStream_t st) {
  KernelTimer timer("dec_feat", st);
  const int64_t rows = nseq * hq;
  hipLaunchKernelGGL(dec_feat1_kernel, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(Q), q_ss, q_hs, hq, rows, (int)kf, (int)kf_pad, I);
  return hipGetLastError();
}

bool attn_decode_select_fused(int64_t Lk) { return Lk <= kSelKeys; }

bool attn_decode_ok(int64_t Lq, int64_t dh) { return Lq >= 1 && Lq <= 16 && dh == 128; }

AttnDecodeSizes attn_decode_sizes(int64_t Lq, int64_t Lk, int64_t Hq, int64_t kt) {
  AttnDecodeSizes z;
  z.nblk = (int)ceil_div(Lk, Lq == 1 ? kSB1 : kDB);   // score blocks (one statistics entry each)
  z.ntokblk = (int)ceil_div(Lk, kDB);
  z.nsplit = (int)ceil_div(kt, kDB * kTokSub);
  z.s_bytes = (size_t)Hq * Lq * Lk * 4;
  z.pstat_bytes = (size_t)Hq * z.nblk * Lq * 8;
  z.nml_bytes = (size_t)Hq * Lq * 4;
  z.opart_bytes = (size_t)z.nsplit * Hq * Lq * 128 * 4;
  return z;
}

#define RMM_DEC_LAUNCH(KERNEL, LQV, GRID, ARGS, ST)                                                  \
  do {                                                                                              \
    switch (LQV) {                                                                                  \
      case 1: hipLaunchKernelGGL(KERNEL<1>, GRID, dim3(kDB), 0, ST, ARGS); break;                   \
      case 2: hipLaunchKernelGGL(KERNEL<2>, GRID, dim3(kDB), 0, ST, ARGS); break;                   \
      case 4: hipLaunchKernelGGL(KERNEL<4>, GRID, dim3(kDB), 0, ST, ARGS); break;                   \
      case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(kDB), 0, ST, ARGS); break;                   \
      default: hipLaunchKernelGGL(KERNEL<16>, GRID, dim3(kDB), 0, ST, ARGS); break;                 \
    }                                                                                               \
  } while (0)

hipError_t launch_attn_decode(int pass, const AttnDecodeDesc &d, hipStream_t st) {
  DecArgs g{};
  g.Q = static_cast<const uint16_t *>(d.Q);
  g.q_ts = d.q_ts;
  g.q_hs = d.q_hs;
  g.Kt = static_cast<const uint16_t *>(d.Kt);
  g.kt_hs = d.kt_hs;
  g.ldkt = d.ldkt;
  g.V = static_cast<const uint16_t *>(d.V);
  g.v_ts = d.v_ts;
  g.v_hs = d.v_hs;
  g.I = d.I;
  g.J = d.J;
  g.Jw = d.J;
  g.S = d.S;
  g.pstat = reinterpret_cast<float2 *>(d.pstat);
  g.nml = d.nml;
  g.tok = d.tok;
  g.opart = d.opart;
  g.O = static_cast<uint16_t *>(d.O);
  g.o_ts = d.o_ts;
  g.o_hs = d.o_hs;
  g.o_scores = d.o_scores;
  g.hq = d.hq;
  g.hkv = d.hkv;
  g.Lq = d.Lq;
  g.Lk = d.Lk;
  g.kf = d.kf;
  g.kf_pad = d.kf_pad;
  g.kt = d.kt;
  g.kt_pad = d.kt_pad;
  g.off = d.Lk - d.Lq;
  g.causal = d.causal ? 1 : 0;
  const int64_t nseq = d.nseq < 1 ? 1 : d.nseq;
  g.q_ss = d.q_ss;
  g.kt_ss = d.kt_ss;
  g.v_ss = d.v_ss;
  g.o_ss = d.o_ss;
  g.lens = d.lens;
  g.kts = d.kts;
  g.nrows = nseq * d.hq;
  if (g.nrows > 65535) return hipErrorInvalidValue;
  const AttnDecodeSizes z = attn_decode_sizes(d.Lq, d.Lk, g.nrows, d.kt);
  g.nblk = z.nblk;
  g.nsplit = z.nsplit;
  g.sblk_keys = d.Lq == 1 ? kSB1 : kDB;
  g.kvec = reinterpret_cast<uintptr_t>(d.Kt) % 16 == 0 && d.ldkt % 8 == 0 && d.kt_hs % 8 == 0 && d.kt_ss % 8 == 0;
  g.c2 = (float)(1.4426950408889634 / __builtin_sqrt(128.0));
  const int lq = d.Lq <= 1 ? 1 : d.Lq <= 2 ? 2 : d.Lq <= 4 ? 4 : d.Lq <= 8 ? 8 : 16;
  if (pass == 0) {
    KernelTimer timer("dec_scores", st);
    if (d.Lq == 1)
      hipLaunchKernelGGL(dec_scores1_kernel, dim3((unsigned)z.nblk, (unsigned)g.nrows), dim3(kDB), 0, st, g);
    else
      RMM_DEC_LAUNCH(dec_scores_kernel, lq, dim3((unsigned)z.nblk, (unsigned)g.nrows), g, st);
  } else if (pass == 1) {
    KernelTimer timer("dec_tok", st);
    RMM_DEC_LAUNCH(dec_tok_kernel, lq, dim3((unsigned)z.ntokblk, (unsigned)g.nrows), g, st);
  } else if (pass == 4) {
    // token scores and selection in one launch (attn_decode_select_fused)
    if (d.Lk > kSelKeys) return hipErrorInvalidValue;
    KernelTimer timer("dec_tok_select", st);
    const unsigned kb = (unsigned)((d.Lk * 4 + 15) / 16 * 16);   // the row keys in LDS
    switch (lq) {
      case 1: hipLaunchKernelGGL(dec_tok_select_kernel<1>, dim3((unsigned)g.nrows), dim3(kSelThreads), kb, st, g); break;
      case 2: hipLaunchKernelGGL(dec_tok_select_kernel<2>, dim3((unsigned)g.nrows), dim3(kSelThreads), kb, st, g); break;
      case 4: hipLaunchKernelGGL(dec_tok_select_kernel<4>, dim3((unsigned)g.nrows), dim3(kSelThreads), kb, st, g); break;
      case 8: hipLaunchKernelGGL(dec_tok_select_kernel<8>, dim3((unsigned)g.nrows), dim3(kSelThreads), kb, st, g); break;
      default: hipLaunchKernelGGL(dec_tok_select_kernel<16>, dim3((unsigned)g.nrows), dim3(kSelThreads), kb, st, g); break;
    }
  } else if (pass == 2) {
    KernelTimer timer("dec_out", st);
    RMM_DEC_LAUNCH(dec_out_kernel, lq, dim3((unsigned)z.nsplit, (unsigned)g.nrows), g, st);
  } else {
    KernelTimer timer("dec_merge", st);
    hipLaunchKernelGGL(dec_merge_kernel, dim3((unsigned)g.nrows, 4), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace rmm

"""Unit parity of each HIP kernel against the CPU oracle, through the C ABI.

Shapes span several tiles with ragged tails, the degenerate cases (k = 1,
k = d, d = 1, m = 1), strided and misaligned layouts, ties and non-positive
scores.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, TOL_F32, check_scores, check_selection, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF, F32 = torch.bfloat16, torch.float32


def _acts(m, d, seed, dtype=BF):
    a = synth.lognormal_col_activations(synth.stream(seed, 77, 1), m, d, 1.0, bf16=dtype == BF)
    return a


# ------------------------------------------------------------------ colnorm
COLNORM_SHAPES = [(1, 1), (3, 7), (64, 512), (257, 1000), (100, 128), (33, 4100), (1000, 8), (4096, 128),
                  (2048, 2048), (513, 28672)]


@pytest.mark.parametrize("dtype", [BF, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("m,d", COLNORM_SHAPES)
def test_colnorm(m, d, dtype):
    A = _acts(m, d, m * 7 + d, dtype)
    s = R.rmm_colnorm(dev_tensor(A, dtype)).cpu().numpy()
    want = oracle.column_scores(A)
    assert s.shape == (d,)
    print(f"  score rms rel err {check_scores(s, want):.2e}")


def test_colnorm_batched_strided_and_scalar_path():
    # Q-like layout [L][H][dh]: heads are strided views.
    L, H, dh = 300, 5, 128
    Q = _acts(L, H * dh, 3).reshape(L, H, dh)
    Qd = dev_tensor(Q, BF)
    s = R.rmm_colnorm(Qd.permute(1, 0, 2)).cpu().numpy()          # [H, L, dh] view
    for h in range(H):
        check_scores(s[h], oracle.column_scores(Q[:, h, :]))
    # misaligned base (scalar path): drop the first column of a wider matrix
    W = _acts(77, 301, 4)
    Wd = dev_tensor(W, BF)
    s2 = R.rmm_colnorm(Wd[:, 1:]).cpu().numpy()
    check_scores(s2, oracle.column_scores(W[:, 1:]))


def test_colnorm_is_deterministic():
    A = dev_tensor(_acts(4096, 4096, 5), BF)
    a = R.rmm_colnorm(A)
    b = R.rmm_colnorm(A)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ top-k
TOPK_CASES = [(1, [1]), (2, [1, 2]), (5, [1, 2, 4, 5]), (127, [1, 31, 32, 33, 63, 126, 127]),
              (128, [1, 39, 64, 90, 103, 127, 128]), (1000, [1, 500, 999]), (4096, [1, 2048, 3277, 4095]),
              (28672, [1, 8602, 14336, 22938, 28671]), (40000, [1, 20000, 39999])]


@pytest.mark.parametrize("d,ks", TOPK_CASES)
def test_topk_random(d, ks):
    rng = np.random.default_rng(d)
    s = np.abs(rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float32)
    sd = dev_tensor(s, F32)
    for k in ks:
        idx = R.rmm_topk(sd, k).cpu().numpy()
        assert idx.shape == (R.rmm_k_pad(k),)
        check_selection(idx, s, s.astype(np.float64), k)


@pytest.mark.parametrize("kind", ["all_equal", "few_values", "zeros_and_neg", "neg_zero", "spread"])
def test_topk_ties_and_signs(kind):
    rng = np.random.default_rng(11)
    d = 3000
    if kind == "all_equal":
        s = np.full(d, 0.7, np.float32)
    elif kind == "few_values":
        s = rng.integers(0, 4, d).astype(np.float32) * 0.5
    elif kind == "zeros_and_neg":
        s = np.where(rng.random(d) < 0.3, 0.0, rng.standard_normal(d)).astype(np.float32)
    elif kind == "neg_zero":
        s = np.where(rng.random(d) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        s[::97] = 1.0
    else:
        s = (rng.standard_normal(d) * 1e30).astype(np.float32)
        s[::7] = 1e-38
    sd = dev_tensor(s, F32)
    for k in (1, 2, 17, 64, 1499, 2999, 3000):
        idx = R.rmm_topk(sd, k).cpu().numpy()
        check_selection(idx, s, s.astype(np.float64), k)


def test_topk_batched():
    rng = np.random.default_rng(12)
    s = np.abs(rng.standard_normal((32, 4096))).astype(np.float32)
    s[3] = 1.0                                    # one fully tied row
    idx = R.rmm_topk(dev_tensor(s, F32), 2048).cpu().numpy()
    for b in range(32):
        check_selection(idx[b], s[b], s[b].astype(np.float64), 2048)


# ------------------------------------------------------------------ gemm
GEMM_SHAPES = [(1, 64, 8, 1), (16, 512, 200, 256), (129, 300, 77, 150), (256, 2048, 512, 1024),
               (100, 130, 129, 65), (300, 1000, 384, 999), (64, 4096, 1, 4096), (1, 1, 1, 1),
               # large-tile path (>= 200 tiles of 256 x 256), ragged edges
               (2048, 1000, 6500, 517), (4000, 700, 4100, 350), (4096, 2048, 4096, 1024)]


@pytest.mark.parametrize("m,d,n,k", GEMM_SHAPES)
def test_gemm_bf16_on_given_indices(m, d, n, k):
    rng = np.random.default_rng(m + d + n + k)
    A = _acts(m, d, m + d)
    B = synth.weight(synth.stream(1, 77, n + d), d, n)
    I = np.sort(rng.choice(d, size=k, replace=False)).astype(np.int32)
    Y = R.rmm_gemm(dev_tensor(A, BF), dev_tensor(B, BF), dev_tensor(I, torch.int32), k).float().cpu().numpy()
    want = oracle.reduced_product(A, B, I)
    assert rel_fro(Y, want) < TOL_BF16


def test_gemm_bf16_unsorted_and_invalid_indices_and_strides():
    rng = np.random.default_rng(3)
    m, d, n, k = 200, 700, 300, 400
    A = _acts(m, d + 9, 21)                       # wider storage: lda > d
    B = synth.weight(synth.stream(1, 77, 5), d, n + 13)
    I = rng.choice(d, size=k, replace=False).astype(np.int32)   # unsorted
    I_bad = I.copy()
    I_bad[::10] = -1
    I_bad[5::10] = d + 3                          # out of range -> contributes zero
    Ad = dev_tensor(A, BF)[:, :d]
    Bd = dev_tensor(B, BF)[:, :n]
    Yfull = torch.zeros((m, n + 5), dtype=BF, device=DEV)
    R.rmm_gemm(Ad, Bd, dev_tensor(I_bad, torch.int32), k, out=Yfull[:, :n])
    keep = I_bad[(I_bad >= 0) & (I_bad < d)]
    want = oracle.reduced_product(A[:, :d], B[:, :n], keep)
    assert rel_fro(Yfull[:, :n].float().cpu().numpy(), want) < TOL_BF16
    assert torch.all(Yfull[:, n:] == 0)           # nothing written past n


# Persistent 256 x 256 GEMM (m >= 1024, >= 192 tiles): ragged last row tile, a
# last column tile narrower than 256 next to full ones, and Y a view into a
# larger buffer.  Full column tiles leave through the LDS-staged epilogue (rows
# past m dropped by the store resource), the partial one through the register
# and per-element paths; nothing outside the view may change.
@pytest.mark.parametrize("m,d,n,k,pad", [(3000, 1000, 4096, 500, 0), (2100, 800, 6152, 400, 8),
                                         (1500, 640, 8192, 320, 24), (1030, 512, 49408, 256, 16)])
def test_gemm_persistent_epilogue_paths(m, d, n, k, pad):
    rng = np.random.default_rng(m + n + pad)
    A = _acts(m, d, m + 3)
    B = synth.weight(synth.stream(1, 91, n + d), d, n)
    I = np.sort(rng.choice(d, size=k, replace=False)).astype(np.int32)
    sentinel = 7.0
    Ybig = torch.full((m + 3, n + pad), sentinel, dtype=BF, device=DEV)
    R.rmm_gemm(dev_tensor(A, BF), dev_tensor(B, BF), dev_tensor(I, torch.int32), k, out=Ybig[:m, :n])
    got = Ybig.float().cpu().numpy()
    assert np.all(got[m:] == sentinel), "rows past m were written"
    assert np.all(got[:, n:] == sentinel), "columns past n were written"
    # every row of the ragged last row tile, plus rows spread over the others
    rows = np.unique(np.concatenate([np.arange((m - 1) // 256 * 256, m), rng.choice(m, size=200, replace=False)]))
    want = oracle.reduced_product(A[rows], B, I)
    assert rel_fro(got[rows, :n], want) < TOL_BF16
    # the last (narrow) column tile on its own, where the paths differ
    c0 = (n - 1) // 256 * 256
    assert rel_fro(got[rows, c0:n], want[:, c0:]) < TOL_BF16


@pytest.mark.parametrize("m,d,n,k", [(64, 512, 512, 256), (1, 8, 3, 2), (65, 130, 70, 100), (200, 1024, 333, 1024)])
def test_gemm_f32(m, d, n, k):
    rng = np.random.default_rng(m * n)
    A = _acts(m, d, 8, F32)
    B = synth.weight(synth.stream(2, 77, d), d, n, bf16=False)
    I = np.sort(rng.choice(d, size=k, replace=False)).astype(np.int32)
    Y = R.rmm_gemm(dev_tensor(A, F32), dev_tensor(B, F32), dev_tensor(I, torch.int32), k).cpu().numpy()
    assert rel_fro(Y, oracle.reduced_product(A, B, I)) < TOL_F32


def test_gemm_rho_one_matches_dense():
    m, d, n = 256, 1024, 384
    A = _acts(m, d, 31)
    B = synth.weight(synth.stream(3, 77, 1), d, n)
    Y, idx, s, k = R.rmm_linear(dev_tensor(A, BF), dev_tensor(B, BF), 1.0)
    assert k == d
    assert np.array_equal(idx.cpu().numpy()[:d], np.arange(d))
    assert rel_fro(Y.float().cpu().numpy(), A.astype(np.float64) @ B.astype(np.float64)) < TOL_BF16


def test_gemm_is_deterministic():
    A = dev_tensor(_acts(512, 2048, 41), BF)
    B = dev_tensor(synth.weight(synth.stream(4, 77, 1), 2048, 1024), BF)
    y1, i1, _, _ = R.rmm_linear(A, B, 0.5)
    y2, i2, _, _ = R.rmm_linear(A, B, 0.5)
    assert torch.equal(i1, i2) and torch.equal(y1, y2)


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("L,Hq,Hkv,k", [(64, 4, 2, 64), (200, 4, 4, 39), (130, 8, 2, 1), (96, 2, 1, 128)])
def test_qk_unit(L, Hq, Hkv, k):
    Q, Kt, V = synth.attention_qkv(5, 77, L, Hq, Hkv, 128)
    S, idx = R.rmm_qk(dev_tensor(Q, BF), dev_tensor(Kt, BF), k)
    S = S.cpu().numpy()
    idx = idx.cpu().numpy()
    gpu_scores = R.rmm_colnorm(dev_tensor(Q, BF).permute(1, 0, 2)).cpu().numpy()
    for h in range(Hq):
        check_selection(idx[h], gpu_scores[h], oracle.column_scores(Q[:, h, :]), k)
        want = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], idx[h][:k])
        assert rel_fro(S[h], want) < TOL_BF16


@pytest.mark.parametrize("L,Hq,Hkv,k,dh", [(64, 4, 2, 32, 128), (300, 4, 4, 150, 128), (129, 2, 1, 1, 128),
                                          (100, 2, 2, 100, 128), (700, 2, 1, 333, 64), (200, 2, 2, 64, 192),
                                          (1000, 3, 1, 999, 128)])
def test_pv_unit(L, Hq, Hkv, k, dh):
    Q, Kt, V = synth.attention_qkv(6, 77, L, Hq, Hkv, dh)
    P = synth.causal_probs(Q, Kt, 128 ** -0.5)                    # torch bf16 on CPU
    Pn = P.float().numpy()
    O, idx = R.rmm_pv(P.to(DEV), dev_tensor(V, BF), k)
    O = O.float().cpu().numpy()
    idx = idx.cpu().numpy()
    gpu_scores = R.rmm_colnorm(P.to(DEV)).cpu().numpy()
    for h in range(Hq):
        check_selection(idx[h], gpu_scores[h], oracle.column_scores(Pn[h]), k)
        want = oracle.reduced_product(Pn[h], V[:, oracle.kv_head(h, Hq, Hkv), :], idx[h][:k])
        assert rel_fro(O[:, h, :], want) < TOL_BF16


# ------------------------------------------------------------------ causal attention
@pytest.mark.parametrize("Lq,Lk,Hq,Hkv,k", [(300, 300, 4, 2, 64), (200, 330, 2, 1, 39), (1000, 1000, 2, 2, 128),
                                            (129, 129, 2, 1, 1)])
def test_qk_causal_skips_only_upper_tiles(Lq, Lk, Hq, Hkv, k):
    Q, _, _ = synth.attention_qkv(7, 77, Lq, Hq, Hkv, 128)
    _, Kt, _ = synth.attention_qkv(8, 77, Lk, Hq, Hkv, 128)
    S0 = torch.full((Hq, Lq, Lk), float("nan"), device=DEV)
    S, idx = R.rmm_qk(dev_tensor(Q, BF), dev_tensor(Kt, BF), k, S=S0, causal=True)
    S = S.cpu().numpy()
    idx = idx.cpu().numpy()
    allowed = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq)
    for h in range(Hq):
        want = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], idx[h][:k])
        got = S[h]
        assert not np.isnan(got[allowed]).any()
        assert rel_fro(got[allowed], want[allowed]) < TOL_BF16


@pytest.mark.parametrize("k", [40, 100])   # one and two K tiles (the two store paths)
@pytest.mark.parametrize("Lq,Lk,causal", [(300, 300, True), (300, 300, False), (200, 332, True), (77, 36, False),
                                           (77, 36, True), (129, 129, False), (64, 128, True)])
def test_qk_strided_output_writes_only_its_block(Lq, Lk, causal, k):
    """S is a view into a larger NaN-filled buffer: every element outside the view
    (padding columns before and after each row, rows past Lq, other heads) stays
    NaN, and the view holds the reduced product where the mask allows."""
    Hq, Hkv = 3, 1
    Q, _, _ = synth.attention_qkv(11, 77, Lq, Hq, Hkv, 128)
    _, Kt, _ = synth.attention_qkv(12, 77, Lk, Hq, Hkv, 128)
    full = torch.full((Hq + 1, Lq + 5, Lk + 12), float("nan"), device=DEV)
    view = full[:Hq, :Lq, 4:4 + Lk]
    S, idx = R.rmm_qk(dev_tensor(Q, BF), dev_tensor(Kt, BF), k, S=view, causal=causal)
    F = full.cpu().numpy()
    outside = np.ones(F.shape, dtype=bool)
    outside[:Hq, :Lq, 4:4 + Lk] = False
    assert np.isnan(F[outside]).all(), "a store landed outside S"
    idx = idx.cpu().numpy()
    allowed = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq) if causal else np.ones((Lq, Lk), bool)
    for h in range(Hq):
        want = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], idx[h][:k])
        got = F[h, :Lq, 4:4 + Lk]
        assert not np.isnan(got[allowed]).any()
        assert rel_fro(got[allowed], want[allowed]) < TOL_BF16


@pytest.mark.parametrize("Lq,Lk,Hq,Hkv,k", [(300, 300, 4, 2, 150), (200, 330, 2, 1, 165), (1000, 1000, 2, 2, 333),
                                            (700, 700, 2, 1, 1), (640, 640, 2, 2, 640)])
def test_pv_causal_never_uses_upper_triangle(Lq, Lk, Hq, Hkv, k):
    Q, _, _ = synth.attention_qkv(9, 77, Lq, Hq, Hkv, 128)
    _, Kt, V = synth.attention_qkv(10, 77, Lk, Hq, Hkv, 128)
    P = synth.causal_probs(Q, Kt, 128 ** -0.5)                    # exact zeros above the diagonal
    Pn = P.float().numpy()
    above = np.arange(Lk)[None, :] > np.arange(Lq)[:, None] + (Lk - Lq)
    Pg = P.clone()
    Pg[:, torch.from_numpy(above)] = float("nan")                 # poison what must not be used
    O, idx = R.rmm_pv(Pg.to(DEV), dev_tensor(V, BF), k, causal=True)
    O = O.float().cpu().numpy()
    idx = idx.cpu().numpy()
    sc = R.rmm_colnorm(P.to(DEV)).cpu().numpy()                   # scores of the clean P
    assert not np.isnan(O).any()
    for h in range(Hq):
        check_selection(idx[h], sc[h], oracle.column_scores(Pn[h]), k)
        want = oracle.reduced_product(Pn[h], V[:, oracle.kv_head(h, Hq, Hkv), :], idx[h][:k])
        assert rel_fro(O[:, h, :], want) < TOL_BF16

"""Seeded random sweep over every entry point: shapes, ratios, strides and masks
drawn from a fixed generator, so each case is reproducible from its id.

Each case runs the library through the C ABI and checks it against the
float64 oracle by the same rules as the unit tests: index sets by the gap rule
(bit-exact on the GPU's own float32 scores; bit-exact against the oracle when
the k-th/(k+1)-th gap exceeds 1e-5), products to the relative Frobenius bound
(1e-2 for bf16 operands, 1e-5 for float32), producers to one bf16 rounding.
The draws cover all kernel paths: few-row (m <= 32), row-gather (32 < m <
1024) and packed (m >= 1024) products, rows narrower and wider than one
tile, unaligned leading dimensions, and the one-token decode passes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, TOL_F32, check_selection, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16


def _rng(tag, i):
    return np.random.default_rng([20261, tag, i])


def _rho(rng):
    # decimal ratios as a user would write them
    return float(rng.choice([0.1, 0.25, 0.3, 0.5, 0.55, 0.7, 0.8, 0.9, 1.0]))


def _linear_case(i):
    rng = _rng(1, i)
    band = i % 3
    m = int([rng.integers(1, 33), rng.integers(33, 1024), rng.integers(1024, 2600)][band])
    d = int(rng.integers(1, 3000))
    n = int(rng.integers(1, 1500))
    if rng.random() < 0.5:          # aligned shapes (vector paths)
        d, n = max(8, d // 8 * 8), max(8, n // 8 * 8)
    return m, d, n, _rho(rng), int(rng.integers(0, 2)) * int(rng.integers(1, 9))


@pytest.mark.parametrize("i", range(60))
def test_sweep_linear_bf16(i):
    m, d, n, rho, pad = _linear_case(i)
    print(f"  m={m} d={d} n={n} rho={rho} lda=d+{pad}", flush=True)
    rng = _rng(2, i)
    A = synth.bf16_round(synth.outlier_activations(rng, m, d + pad, 0.01, 20.0))
    B = synth.weight(_rng(3, i), d, n)
    Ad = dev_tensor(A, BF)[:, :d]
    Y, idx, s, k = R.rmm_linear(Ad, dev_tensor(B, BF), rho)
    assert k == oracle.retained_count(rho, d)
    s_gpu = s.cpu().numpy()
    s_ora = oracle.column_scores(A[:, :d])
    np.testing.assert_allclose(s_gpu, s_ora, rtol=1e-5, atol=1e-30)
    check_selection(idx.cpu().numpy(), s_gpu, s_ora, k)
    I = idx.cpu().numpy()[:k]
    rows = np.arange(m) if m <= 600 else np.sort(rng.choice(m, size=600, replace=False))
    want = oracle.reduced_product(A[rows, :d], B, I)
    assert rel_fro(Y.float().cpu().numpy()[rows], want) < TOL_BF16


@pytest.mark.parametrize("i", range(16))
def test_sweep_linear_f32(i):
    rng = _rng(4, i)
    m, d, n = int(rng.integers(1, 300)), int(rng.integers(1, 1100)), int(rng.integers(1, 700))
    rho = _rho(rng)
    print(f"  m={m} d={d} n={n} rho={rho}", flush=True)
    A = synth.lognormal_col_activations(rng, m, d, 1.0, bf16=False).astype(np.float32)
    B = synth.weight(_rng(5, i), d, n, bf16=False).astype(np.float32)
    Y, idx, s, k = R.rmm_linear(dev_tensor(A, torch.float32), dev_tensor(B, torch.float32), rho)
    s_gpu = s.cpu().numpy()
    s_ora = oracle.column_scores(A)
    check_selection(idx.cpu().numpy(), s_gpu, s_ora, k)
    want = oracle.reduced_product(A, B, idx.cpu().numpy()[:k])
    assert rel_fro(Y.cpu().numpy(), want) < TOL_F32


@pytest.mark.parametrize("i", range(30))
def test_sweep_topk_batched(i):
    rng = _rng(6, i)
    batch, d = int(rng.integers(1, 40)), int(rng.integers(1, 40000))
    k = int(rng.integers(1, d + 1))
    kind = i % 3
    if kind == 0:
        s = rng.random((batch, d)).astype(np.float32)
    elif kind == 1:       # few distinct values: many ties at rank k
        s = rng.integers(0, 5, (batch, d)).astype(np.float32)
    else:                 # column norms with outliers
        s = (128 + 0.7 * rng.standard_normal((batch, d))).astype(np.float32)
        s[:, rng.choice(d, size=max(1, d // 200), replace=False)] *= 30
    print(f"  batch={batch} d={d} k={k} kind={kind}", flush=True)
    idx = R.rmm_topk(dev_tensor(s, torch.float32), k).cpu().numpy()
    for b in range(batch):
        # the scores are exact float32 values here, so the selection must match exactly
        got = idx[b]
        assert np.all(got[k:] == -1)
        assert np.array_equal(got[:k], oracle.select_top(s[b].astype(np.float64), k))


@pytest.mark.parametrize("i", range(30))
def test_sweep_qk_pv(i):
    rng = _rng(7, i)
    Lq = int(rng.integers(1, 700))
    Lk = Lq + int(rng.integers(0, 300)) if rng.random() < 0.5 else Lq
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2]))
    causal = bool(rng.integers(0, 2))
    kf = int(rng.integers(1, 129))
    kt = int(rng.integers(1, Lk + 1))
    print(f"  Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} kf={kf} kt={kt} causal={causal}", flush=True)
    Q, _, _ = synth.attention_qkv(30 + i, 77, Lq, Hq, Hkv, 128)
    _, Kt, V = synth.attention_qkv(60 + i, 77, Lk, Hq, Hkv, 128)
    S, I = R.rmm_qk(dev_tensor(Q, BF), dev_tensor(Kt, BF), kf, causal=causal)
    S, I = S.cpu().numpy(), I.cpu().numpy()
    fs = R.rmm_colnorm(dev_tensor(Q, BF).permute(1, 0, 2)).cpu().numpy()
    allowed = (np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq)) if causal else np.ones((Lq, Lk), bool)
    for h in range(Hq):
        check_selection(I[h], fs[h], oracle.column_scores(Q[:, h, :]), kf)
        want = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], I[h][:kf])
        if allowed.any():
            assert rel_fro(S[h][allowed], want[allowed]) < TOL_BF16
    # P: softmax of the dense logits, rounded to bf16 (input preparation; the library takes P)
    if causal:
        P = synth.causal_probs(Q, Kt, 128 ** -0.5)
    else:
        Sd = torch.stack([torch.from_numpy(Q[:, h, :]).float() @ torch.from_numpy(Kt[oracle.kv_head(h, Hq, Hkv)]).float()
                          for h in range(Hq)])
        P = torch.softmax(Sd * 128 ** -0.5, dim=-1).to(BF)
    Pn = P.float().numpy().astype(np.float64)
    O, J = R.rmm_pv(P.to(DEV), dev_tensor(V, BF), kt, causal=causal)
    O, J = O.float().cpu().numpy(), J.cpu().numpy()
    ps = R.rmm_colnorm(P.to(DEV)).cpu().numpy()
    for h in range(Hq):
        Ph = np.where(allowed, Pn[h], 0.0) if causal else Pn[h]
        check_selection(J[h], ps[h], oracle.column_scores(Ph), kt)
        want = oracle.reduced_product(Ph, V[:, oracle.kv_head(h, Hq, Hkv), :], J[h][:kt])
        assert rel_fro(O[:, h, :], want) < TOL_BF16


@pytest.mark.parametrize("i", range(24))
def test_sweep_fused_attention(i):
    from test_gpu_attention import W4K, _operands, check_fused

    rng = _rng(8, i)
    decode = i % 2 == 1
    Lq = int(rng.integers(1, 17)) if decode else int(rng.integers(17, 600))
    Lk = Lq + int(rng.integers(0, 1500 if decode else 300))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    kf = int(rng.integers(1, 129))
    kt = int(rng.integers(1, Lk + 1))
    causal = bool(rng.integers(0, 2)) or decode
    print(f"  Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} kf={kf} kt={kt} causal={causal}", flush=True)
    Q, Kt, V = _operands(W4K, Lq, Lk, Hq, Hkv)
    print(f"  near ties: {check_fused(Q, Kt, V, kf, kt, causal, rows=128, seed=i)}")


@pytest.mark.parametrize("i", range(16))
def test_sweep_gemm_w8(i):
    rng = _rng(9, i)
    m = int([rng.integers(1, 33), rng.integers(33, 400)][i % 2])
    d = int(rng.integers(8, 3000)) // 16 * 16 + 16
    n = int(rng.integers(16, 1500)) // 16 * 16
    rho = _rho(rng)
    print(f"  m={m} d={d} n={n} rho={rho}", flush=True)
    A = synth.bf16_round(synth.outlier_activations(rng, m, d, 0.01, 20.0))
    q, sc = synth.int8_per_column(synth.weight(_rng(10, i), d, n))
    Ad = dev_tensor(A, BF)
    s = R.rmm_colnorm(Ad)
    k = R.rmm_k_from_rho(rho, d)
    idx = R.rmm_topk(s, k)
    Y = R.rmm_gemm_w8(Ad, dev_tensor(q, torch.int8), dev_tensor(sc, torch.float32), idx, k)
    want = oracle.reduced_product_w8(A, q, sc, idx.cpu().numpy()[:k])
    assert rel_fro(Y.float().cpu().numpy(), want) < TOL_BF16


@pytest.mark.parametrize("i", range(16))
def test_sweep_producers(i):
    rng = _rng(11, i)
    m = int(rng.integers(1, 3000))
    d = 512 * int(rng.integers(1, 17))
    n = 8 * int(rng.integers(1, 1200))
    print(f"  m={m} d={d} (rmsnorm) n={n} (swiglu)", flush=True)
    X = synth.bf16_round(synth.outlier_activations(rng, m, d, 0.005, 30.0) * rng.uniform(0.05, 20.0, (m, 1)))
    w = synth.bf16_round(rng.uniform(0.2, 1.5, d))
    Y, s = R.rmm_rmsnorm_scored(dev_tensor(X, BF), dev_tensor(w, BF), 1e-5)
    Yn = Y.float().cpu().numpy().astype(np.float64)
    ref = oracle.rmsnorm(X, w, 1e-5)
    assert np.all(np.abs(Yn - ref) <= (2.0 ** -8 + 2e-5) * np.abs(ref) + 1e-30)
    np.testing.assert_allclose(s.cpu().numpy(), oracle.column_scores(Yn), rtol=1e-5, atol=1e-30)
    G = synth.bf16_round(rng.standard_normal((m, n)) * 2)
    U = synth.bf16_round(rng.standard_normal((m, n)))
    H, s2 = R.rmm_swiglu_scored(dev_tensor(G, BF), dev_tensor(U, BF))
    Hn = H.float().cpu().numpy().astype(np.float64)
    ref2 = oracle.swiglu(G, U)
    assert np.all(np.abs(Hn - ref2) <= 2.0 ** -8 * np.abs(ref2) + 1e-30)
    np.testing.assert_allclose(s2.cpu().numpy(), oracle.column_scores(Hn), rtol=1e-5, atol=1e-30)

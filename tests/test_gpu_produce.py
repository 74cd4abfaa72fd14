"""Producer-fused scoring: rmm_swiglu_scored writes H = silu(G) * U and the
column scores of H in one pass; rmm_rmsnorm_scored writes the RMS-normalised
rows Y = X w / sqrt(mean(X^2) + eps) and the column scores of Y in one pass.

H is compared element by element with the float64 oracle (one bf16 rounding:
relative error at most 2^-8, plus an absolute floor for values that underflow
in float32; Y adds the float32 error of the row's mean square, below 2e-5); the scores are compared with the oracle's column norms of the
bf16 H the kernel wrote (relative 1e-5) and with rmm_colnorm on that H; the
top-k selection on them follows the gap rule.
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


def _pre(m, n, seed, tensor):
    # gate / up pre-activations: N(0,1) with a few outlier columns, as the layer's activations
    return synth.outlier_activations(synth.stream(seed, 79, tensor), m, n, 0.005, 30.0)


def check_swiglu(m, n, seed, rho=0.8):
    G, U = _pre(m, n, seed, 1), _pre(m, n, seed, 2)
    Gd, Ud = dev_tensor(G, BF), dev_tensor(U, BF)
    H, s = R.rmm_swiglu_scored(Gd, Ud)
    Hn = H.float().cpu().numpy().astype(np.float64)
    ref = oracle.swiglu(G, U)
    assert np.all(np.abs(Hn - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), "H differs beyond one bf16 rounding"
    sn = s.cpu().numpy()
    s_ora = oracle.column_scores(Hn)
    np.testing.assert_allclose(sn, s_ora, rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(sn, R.rmm_colnorm(H).cpu().numpy(), rtol=1e-5, atol=1e-30)
    k = R.rmm_k_from_rho(rho, n)
    idx = R.rmm_topk(s, k).cpu().numpy()
    return check_selection(idx, sn, s_ora, k)


@pytest.mark.parametrize("m,n", [(1, 8), (7, 520), (300, 1000), (2048, 8192), (5000, 2056)])
def test_swiglu_scored(m, n):
    print(f"  near ties: {check_swiglu(m, n, m + n)}")


def test_swiglu_scored_llama8b_down_input_full():
    """The 16k-token layer's down-projection input: 16384 x 14336."""
    print(f"  near ties: {check_swiglu(16384, 14336, 7)}")
    torch.cuda.empty_cache()


def test_swiglu_scored_strided_and_deterministic():
    m, n = 513, 1024
    UG = dev_tensor(np.concatenate([_pre(m, n, 3, 2), _pre(m, n, 3, 1)], axis=1), BF)   # [up | gate]
    Hfull = torch.zeros((m, n + 16), dtype=BF, device=DEV)
    H, s1 = R.rmm_swiglu_scored(UG[:, n:], UG[:, :n], H=Hfull[:, :n])
    _, s2 = R.rmm_swiglu_scored(UG[:, n:], UG[:, :n], H=Hfull[:, :n])
    assert torch.equal(s1, s2)
    assert torch.all(Hfull[:, n:] == 0)
    ref = oracle.swiglu(UG[:, n:].float().cpu().numpy(), UG[:, :n].float().cpu().numpy())
    Hn = Hfull[:, :n].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Hn - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_swiglu_scored_needs_aligned_rows():
    G = dev_tensor(_pre(4, 12, 5, 1), BF)
    with pytest.raises(R.RMMError) as e:
        R.rmm_swiglu_scored(G, G.clone())
    assert e.value.status == R.RMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def _rms_inputs(m, d, seed):
    # residual-stream rows: N(0,1) with outlier channels and a per-row scale; gain around 1
    X = synth.outlier_activations(synth.stream(seed, 83, 1), m, d, 0.005, 30.0)
    X = X * synth.stream(seed, 83, 2).uniform(0.05, 20.0, size=(m, 1))
    w = synth.stream(seed, 83, 3).uniform(0.2, 1.5, size=d)
    return synth.bf16_round(X), synth.bf16_round(w)


def check_rmsnorm(m, d, seed, eps=1e-5, rho=0.5):
    X, w = _rms_inputs(m, d, seed)
    Y, s = R.rmm_rmsnorm_scored(dev_tensor(X, BF), dev_tensor(w, BF), eps)
    Yn = Y.float().cpu().numpy().astype(np.float64)
    ref = oracle.rmsnorm(X, w, eps)
    err = np.abs(Yn - ref) / np.maximum(np.abs(ref), 1e-30)
    assert err.max() <= 2.0 ** -8 + 2e-5, f"Y differs beyond one bf16 rounding: {err.max()}"
    sn = s.cpu().numpy()
    s_ora = oracle.column_scores(Yn)
    np.testing.assert_allclose(sn, s_ora, rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(sn, R.rmm_colnorm(Y).cpu().numpy(), rtol=1e-5, atol=1e-30)
    k = R.rmm_k_from_rho(rho, d)
    idx = R.rmm_topk(s, k).cpu().numpy()
    return check_selection(idx, sn, s_ora, k)


@pytest.mark.parametrize("m,d", [(1, 512), (3, 1536), (257, 2048), (2051, 3072), (4099, 4096), (600, 8192)])
def test_rmsnorm_scored(m, d):
    print(f"  near ties: {check_rmsnorm(m, d, m + d)}")


def test_rmsnorm_scored_llama8b_hidden_full():
    """The 16k-token layer's attention input: 16384 x 4096."""
    print(f"  near ties: {check_rmsnorm(16384, 4096, 9)}")
    torch.cuda.empty_cache()


def test_rmsnorm_scored_eps_and_constant_rows():
    # constant rows normalise to sign(c) w / sqrt(1 + eps / c^2); eps = 0 gives exactly sign(c) w
    d = 1024
    w = synth.bf16_round(synth.stream(4, 83, 3).uniform(0.2, 1.5, size=d))
    X = np.repeat(np.array([[-3.0], [0.5], [2.0 ** -20]]), d, axis=1)
    for eps in (0.0, 1e-5, 4.0):
        Y, s = R.rmm_rmsnorm_scored(dev_tensor(X, BF), dev_tensor(w, BF), eps)
        Yn = Y.float().cpu().numpy().astype(np.float64)
        ref = oracle.rmsnorm(X, w, eps)
        assert np.all(np.abs(Yn - ref) <= (2.0 ** -8 + 2e-5) * np.abs(ref))
        if eps == 0.0:
            np.testing.assert_array_equal(Yn, np.sign(X) * w)
        np.testing.assert_allclose(s.cpu().numpy(), oracle.column_scores(Yn), rtol=1e-5)


def test_rmsnorm_scored_strided_and_deterministic():
    m, d = 1030, 2048
    X, w = _rms_inputs(m, d, 5)
    Xwide = torch.zeros((m, d + 64), dtype=BF, device=DEV)
    Xwide[:, 32:32 + d] = dev_tensor(X, BF)
    Yfull = torch.zeros((m, d + 24), dtype=BF, device=DEV)
    wd = dev_tensor(w, BF)
    Y, s1 = R.rmm_rmsnorm_scored(Xwide[:, 32:32 + d], wd, 1e-6, Y=Yfull[:, 8:8 + d])
    _, s2 = R.rmm_rmsnorm_scored(Xwide[:, 32:32 + d], wd, 1e-6, Y=Yfull[:, 8:8 + d])
    assert torch.equal(s1, s2)
    assert torch.all(Yfull[:, :8] == 0) and torch.all(Yfull[:, 8 + d:] == 0)
    ref = oracle.rmsnorm(X, w, 1e-6)
    Yn = Yfull[:, 8:8 + d].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yn - ref) <= (2.0 ** -8 + 2e-5) * np.abs(ref) + 1e-30)


def test_rmsnorm_scored_rejects():
    X = torch.zeros((4, 1000), dtype=BF, device=DEV)
    with pytest.raises(R.RMMError) as e:
        R.rmm_rmsnorm_scored(X, torch.ones(1000, dtype=BF, device=DEV))
    assert e.value.status == R.RMM_ERR_UNSUPPORTED
    X = torch.zeros((4, 512 * 17), dtype=BF, device=DEV)
    with pytest.raises(R.RMMError) as e:
        R.rmm_rmsnorm_scored(X, torch.ones(512 * 17, dtype=BF, device=DEV))
    assert e.value.status == R.RMM_ERR_UNSUPPORTED
    X = torch.zeros((4, 512), dtype=BF, device=DEV)
    with pytest.raises(R.RMMError) as e:
        R.rmm_rmsnorm_scored(X, torch.ones(512, dtype=BF, device=DEV), eps=-1.0)
    assert e.value.status == R.RMM_ERR_INVALID_ARG
    torch.cuda.synchronize()


# ------------------------------------------------------------------ scores of a GEMM's output
@pytest.mark.parametrize("m,d,n,rho,dt", [
    (2048, 2048, 6144, 0.5, torch.bfloat16),      # persistent NT kernel: scores from the epilogue
    (1300, 1024, 12800, 0.7, torch.bfloat16),     # NT kernel with a ragged last row slab and column tile
    (500, 1536, 1000, 0.8, torch.bfloat16),       # row-gather core, scores in a second pass
    (16, 2048, 3000, 0.5, torch.bfloat16),        # few-row kernel
    (64, 512, 512, 0.5, torch.float32),           # fp32 product
])
def test_gemm_scored(m, d, n, rho, dt):
    """rmm_gemm_scored: Y bitwise equal to rmm_gemm's, and its column scores equal
    the float64 column norms of the Y values written (1e-5 relative)."""
    rng = synth.stream(0, 96, m + n)
    A = synth.outlier_activations(rng, m, d, 0.01, 20.0)
    B = synth.weight(synth.stream(0, 96, d + 7), d, n)
    Ad, Bd = dev_tensor(A, dt), dev_tensor(B, dt)
    k = R.rmm_k_from_rho(rho, d)
    idx = R.rmm_topk(R.rmm_colnorm(Ad), k)
    Y0 = R.rmm_gemm(Ad, Bd, idx, k)
    Y, sc = R.rmm_gemm_scored(Ad, Bd, idx, k)
    torch.cuda.synchronize()
    bits = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(Y.view(bits), Y0.view(bits))
    Yh = Y.float().cpu().numpy()
    np.testing.assert_allclose(sc.cpu().numpy(), oracle.column_scores(Yh), rtol=1e-5, atol=1e-30)
    I = idx.cpu().numpy()[:k]
    tol = TOL_BF16 if dt == torch.bfloat16 else TOL_F32
    assert rel_fro(Yh, oracle.reduced_product(A, B, I)) < tol

"""Producer-fused scoring: rmm_swiglu_scored writes H = silu(G) * U and the
column scores of H in one pass.

H is compared element by element with the float64 oracle (one bf16 rounding:
relative error at most 2^-8, plus an absolute floor for values that underflow
in float32); the scores are compared with the oracle's column norms of the
bf16 H the kernel wrote (relative 1e-5) and with rmm_colnorm on that H; the
top-k selection on them follows the gap rule.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import check_selection, dev_tensor

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

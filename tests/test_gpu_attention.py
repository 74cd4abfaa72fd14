"""Parity of the fused reduced attention (rmm_attention) with the float64 oracle.

The fused call selects features of Q by column norm, recomputes S = Q[:, I]
K[I, :] and the softmax tile by tile, scores tokens by the column norms of
the float32 probabilities, keeps the top k_tok tokens and returns
P[:, J] V[J, :] without ever writing S or P.  Checks, per head:

* I and J follow the gap rule (bit-exact against the oracle's selection on
  the GPU's own float32 scores; bit-exact against the float64 selection when
  the k-th/(k+1)-th gap exceeds 1e-5; near ties counted);
* the token scores match the oracle's column norms of P (computed with the
  GPU's I, so a tie-swap in I does not move them) to a relative 2e-5, with
  an absolute floor of 1e-6 of the largest score (float32 exponentials
  underflow where float64 ones do not);
* O matches the oracle's P[:, J] V[J, :] (with the GPU's J) to the bf16
  relative Frobenius bound 1e-2; P enters the product rounded to bf16;
* the column scores of O returned with it (for the projection that reads O)
  match the oracle's column norms of the bf16 O to a relative 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, check_selection, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
W4K = synth.WORKLOADS["attn-32h-4k"]
W8B = synth.WORKLOADS["llama3.1-8b-layer-16k"]


def _operands(w, Lq, Lk, Hq, Hkv):
    """Q for the last Lq of Lk tokens (queries follow their context), K and V for all Lk."""
    Q, Kt, V = synth.attention_operands(w, L=Lk, Hq=Hq, Hkv=Hkv)
    return np.ascontiguousarray(Q[Lk - Lq:]), Kt, V


def _run(Q, Kt, V, kf, kt, causal, ws_fill=None):
    Lq, Hq, dh = Q.shape
    Lk = Kt.shape[2]
    Qd, Ktd, Vd = (dev_tensor(x, torch.bfloat16) for x in (Q, Kt, V))
    ts = torch.full((Hq, Lk), float("nan"), dtype=torch.float32, device=DEV)
    os_ = torch.full((Hq, dh), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(R.rmm_attention_workspace_bytes(Lq, Lk, Hq, dh, kf, kt), dtype=torch.uint8, device=DEV)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    O, I, J = R.rmm_attention(Qd, Ktd, Vd, kf, kt, tok_scores=ts, ws=ws, causal=causal, o_scores=os_)
    fs = R.rmm_colnorm(Qd.permute(1, 0, 2))          # the feature scores the call selected on
    torch.cuda.synchronize()
    # column scores of O for the projection that reads it, against the bf16 O written
    On = O.float().cpu().numpy().astype(np.float64).reshape(Lq, Hq * dh)
    np.testing.assert_allclose(os_.cpu().numpy().reshape(-1), oracle.column_scores(On), rtol=1e-5, atol=1e-30)
    return O, I, J, ts, fs


def _head_oracle(Q, Kt, h, I, causal, scale):
    """Probabilities of head h given its feature set I (float64)."""
    Lq, Hq, _ = Q.shape
    S = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Kt.shape[0])], I)[None]
    return (oracle.causal_softmax(S, scale) if causal else oracle.full_softmax(S, scale))[0]


def check_fused(Q, Kt, V, kf, kt, causal, heads=None, rows=None, seed=0):
    Lq, Hq, dh = Q.shape
    Hkv, _, Lk = Kt.shape
    O, I, J, ts, fs = _run(Q, Kt, V, kf, kt, causal)
    O = O.float().cpu().numpy()
    I, J, ts, fs = (x.cpu().numpy() for x in (I, J, ts, fs))
    assert I.shape == (Hq, R.rmm_k_pad(kf)) and J.shape == (Hq, R.rmm_k_pad(kt))
    assert np.all(np.isfinite(ts)) and np.all(np.isfinite(O))
    scale = 1.0 / math.sqrt(dh)
    rng = np.random.default_rng(seed)
    near = 0
    for h in (range(Hq) if heads is None else heads):
        near += check_selection(I[h], fs[h], oracle.column_scores(Q[:, h, :]), kf)
        P = _head_oracle(Q, Kt, h, I[h][:kf], causal, scale)
        tok = oracle.column_scores(P)
        np.testing.assert_allclose(ts[h], tok, rtol=2e-5, atol=1e-6 * tok.max())
        near += check_selection(J[h], ts[h], tok, kt)
        r = np.arange(Lq) if rows is None or rows >= Lq else np.sort(rng.choice(Lq, size=rows, replace=False))
        want = oracle.reduced_product(P[r], V[:, oracle.kv_head(h, Hq, Hkv), :], J[h][:kt])
        err = rel_fro(O[r, h, :], want)
        assert err < TOL_BF16, f"head {h}: O rel fro {err:.3e}"
        del P
    return near


# (Lq, Lk, Hq, Hkv, k_feat, k_tok, causal): ragged tails, grouped heads, padded
# feature counts (kf=100 pads to 128), queries after a longer context, one-token
# decode, every feature and token kept, a single kept feature and token.
SMALL = [
    (300, 300, 4, 2, 64, 150, True),
    (512, 512, 4, 4, 64, 256, True),
    (256, 256, 2, 1, 100, 100, False),
    (200, 333, 4, 1, 1, 1, True),
    (1, 777, 4, 2, 128, 777, True),
    (130, 130, 2, 2, 128, 130, True),
    (64, 64, 2, 1, 7, 64, False),
    (1000, 1000, 2, 2, 33, 999, False),
    (257, 1025, 2, 1, 50, 300, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "Lq{}_Lk{}_h{}x{}_kf{}_kt{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_fused_attention_small(case):
    Lq, Lk, Hq, Hkv, kf, kt, causal = case
    Q, Kt, V = _operands(W4K, Lq, Lk, Hq, Hkv)
    near = check_fused(Q, Kt, V, kf, kt, causal)
    print(f"  near ties: {near}")


# A few new tokens after a longer context (decode steps: Lq <= 16 runs passes split
# over keys): one token, a few, sixteen; grouped heads; with and without the mask.
DECODE = [
    (1, 300, 4, 2, 64, 150, True),
    (3, 1025, 4, 1, 40, 500, True),
    (16, 4096, 8, 2, 64, 2048, True),
    (16, 16, 2, 2, 128, 16, True),
    (7, 2000, 4, 4, 100, 1999, False),
    (2, 513, 2, 1, 1, 1, True),
    # the longest context the one-workgroup token selection holds (32768 keys,
    # 128 KiB of LDS)
    (1, 32768, 2, 1, 64, 16384, True),
    # contexts longer than the one-workgroup token selection holds in LDS
    # (32768 scores): token scores and top-k as two launches
    (1, 40000, 2, 1, 64, 20000, True),
    (4, 33000, 2, 2, 32, 1000, True),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "Lq{}_Lk{}_h{}x{}_kf{}_kt{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_fused_attention_decode(case):
    Lq, Lk, Hq, Hkv, kf, kt, causal = case
    Q, Kt, V = _operands(W4K, Lq, Lk, Hq, Hkv)
    print(f"  near ties: {check_fused(Q, Kt, V, kf, kt, causal)}")


@pytest.mark.parametrize("Lq,Lk", [(1, 3000), (5, 3000), (1, 40000)])
def test_fused_attention_decode_without_token_scores(Lq, Lk):
    """Asking for the token scores changes no output: O, I and J are bitwise the same."""
    Hq, Hkv, kf, kt = 4, 2, 64, Lk // 2
    Q, Kt, V = (dev_tensor(x, torch.bfloat16) for x in _operands(W4K, Lq, Lk, Hq, Hkv))
    ts = torch.empty((Hq, Lk), dtype=torch.float32, device=DEV)
    a = R.rmm_attention(Q, Kt, V, kf, kt, causal=True, tok_scores=ts)
    b = R.rmm_attention(Q, Kt, V, kf, kt, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    J = b[2].cpu().numpy()
    for h in range(Hq):
        assert np.array_equal(J[h][:kt], oracle.select_top(ts[h].cpu().numpy().astype(np.float64), kt))


@pytest.mark.parametrize("Lq,Lk", [(1, 1000), (1, 20000), (3, 5000)])
def test_fused_attention_decode_ties_keep_lowest_indices(Lq, Lk):
    """All-equal scores in both selections of a decode step: |q| equal over the
    features (q = +-1) and every key zero, so every token's probability and score
    tie. Both selections must then keep the lowest indices, and O the mean of the
    kept V rows."""
    Hq, Hkv, kf, kt = 4, 2, 37, Lk // 3
    rng = np.random.default_rng(17)
    Q = np.where(rng.random((Lq, Hq, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    Kt = np.zeros((Hkv, 128, Lk), np.float32)
    V = rng.standard_normal((Lk, Hkv, 128)).astype(np.float32)
    Qd, Ktd, Vd = dev_tensor(Q, torch.bfloat16), dev_tensor(Kt, torch.bfloat16), dev_tensor(V, torch.bfloat16)
    ts = torch.empty((Hq, Lk), dtype=torch.float32, device=DEV)
    O, I, J = R.rmm_attention(Qd, Ktd, Vd, kf, kt, causal=False, tok_scores=ts)
    torch.cuda.synchronize()
    I, J, O, ts = I.cpu().numpy(), J.cpu().numpy(), O.float().cpu().numpy(), ts.cpu().numpy()
    Vk = Vd.float().cpu().numpy().astype(np.float64)     # V as the kernels read it (bf16)
    P = np.full((Lq, Lk), 1.0 / Lk)                       # every key scores zero: uniform probabilities
    for h in range(Hq):
        assert np.array_equal(I[h][:kf], np.arange(kf)) and np.all(I[h][kf:] == -1)
        assert np.all(ts[h] == ts[h][0])
        assert np.array_equal(J[h][:kt], np.arange(kt)) and np.all(J[h][kt:] == -1)
        want = oracle.reduced_product(P, Vk[:, oracle.kv_head(h, Hq, Hkv), :], J[h][:kt])
        assert rel_fro(O[:, h, :], want) < TOL_BF16


def test_fused_attention_decode_unaligned_values_use_the_general_path():
    """V rows that are not 16-byte aligned go through the general passes: same results."""
    Lq, Lk, Hq, Hkv, kf, kt = 4, 700, 4, 2, 64, 350
    Q, Kt, V = _operands(W4K, Lq, Lk, Hq, Hkv)
    Vw = np.zeros((Lk, Hkv, 129), dtype=np.float32)
    Vw[:, :, :128] = V
    Qd, Ktd = dev_tensor(Q, torch.bfloat16), dev_tensor(Kt, torch.bfloat16)
    Vd = dev_tensor(Vw, torch.bfloat16)[:, :, :128]            # head stride 129: unaligned rows
    O, I, J = R.rmm_attention(Qd, Ktd, Vd, kf, kt, causal=True)
    O2, I2, J2 = R.rmm_attention(Qd, Ktd, dev_tensor(V, torch.bfloat16), kf, kt, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(I, I2) and torch.equal(J, J2)
    assert rel_fro(O.float().cpu().numpy(), O2.float().cpu().numpy()) < 1e-2


@pytest.mark.parametrize("Lq", [1, 16])
def test_fused_attention_decode_llama8b_16k_context(Lq):
    """Decode steps after the 16k-token context of the LLaMA-3.1-8B layer, rho = 0.5."""
    at = W8B.attention
    Q, Kt, V = synth.attention_operands(W8B)
    Q = np.ascontiguousarray(Q[at.L - Lq:])
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    print(f"  near ties: {check_fused(Q, Kt, V, kf, kt, True, heads=[0, 13, 31])}")
    torch.cuda.empty_cache()


def test_fused_attention_full_retention_is_attention():
    """k_feat = dh and k_tok = Lk: the result is ordinary causal attention."""
    L, Hq, Hkv = 384, 4, 2
    Q, Kt, V = _operands(W4K, L, L, Hq, Hkv)
    O, I, J, _, _ = _run(Q, Kt, V, 128, L, True)
    assert np.array_equal(I.cpu().numpy()[:, :128], np.tile(np.arange(128), (Hq, 1)))
    Jn = J.cpu().numpy()
    assert np.array_equal(Jn[:, :L], np.tile(np.arange(L), (Hq, 1)))
    ref = oracle.reduced_attention(Q, Kt, V, 128, L, causal=True)
    assert rel_fro(O.float().cpu().numpy(), ref["O"]) < TOL_BF16


def test_fused_attention_ignores_workspace_contents():
    """Nothing in the workspace needs clearing: garbage in it changes no output bit."""
    Q, Kt, V = _operands(W4K, 300, 300, 4, 2)
    a = _run(Q, Kt, V, 64, 150, True, ws_fill=0)
    b = _run(Q, Kt, V, 64, 150, True, ws_fill=0xFF)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)


def test_fused_attention_rejects_bad_requests():
    Q, Kt, V = (dev_tensor(x, torch.bfloat16) for x in _operands(W4K, 64, 64, 2, 1))
    with pytest.raises(R.RMMError) as e:          # more tokens kept than exist
        R.rmm_attention(Q, Kt, V, 64, 65)
    assert e.value.status == R.RMM_ERR_INVALID_ARG
    with pytest.raises(R.RMMError) as e:          # causal queries beyond the keys
        R.rmm_attention(torch.cat([Q, Q]), Kt, V, 64, 32, causal=True)
    assert e.value.status == R.RMM_ERR_INVALID_ARG
    Q64, K64, V64 = Q[:, :, :64].contiguous(), Kt[:, :64, :].contiguous(), V[:, :, :64].contiguous()
    with pytest.raises(R.RMMError) as e:          # head size the fused kernels do not serve
        R.rmm_attention(Q64, K64, V64, 32, 32)
    assert e.value.status == R.RMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_fused_attention_llama8b_16k_sampled():
    """The 16k-token LLaMA-3.1-8B attention at rho = 0.5, in the launch the bench times.

    Every head's feature set follows the gap rule; token scores, J and sampled
    output rows are checked against the oracle on heads 0 and 31.
    """
    at = W8B.attention
    Q, Kt, V = synth.attention_operands(W8B)
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    O, I, J, ts, fs = _run(Q, Kt, V, kf, kt, True)
    O = O.float().cpu().numpy()
    I, J, ts, fs = (x.cpu().numpy() for x in (I, J, ts, fs))
    near = 0
    for h in range(at.Hq):
        near += check_selection(I[h], fs[h], oracle.column_scores(Q[:, h, :]), kf)
    rng = np.random.default_rng(5)
    scale = 1.0 / math.sqrt(at.dh)
    for h in (0, at.Hq - 1):
        P = _head_oracle(Q, Kt, h, I[h][:kf], True, scale)
        tok = oracle.column_scores(P)
        np.testing.assert_allclose(ts[h], tok, rtol=2e-5, atol=1e-6 * tok.max())
        near += check_selection(J[h], ts[h], tok, kt)
        r = np.sort(rng.choice(at.L, size=64, replace=False))
        want = oracle.reduced_product(P[r], V[:, oracle.kv_head(h, at.Hq, at.Hkv), :], J[h][:kt])
        assert rel_fro(O[r, h, :], want) < TOL_BF16
        del P
    print(f"  fused llama3.1-8b attention: near ties {near}")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

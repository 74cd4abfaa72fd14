"""Chain parity on the five synthetic workloads, at their full sizes and in the
launch configuration bench.py times (the library picks tiles from the shapes).

Scores are compared with the float64 oracle over every row; index sets follow
the gap rule (bit-exact whenever the k-th/(k+1)-th float64 gap exceeds 1e-5,
and always bit-exact against the oracle's selection on the GPU's own float32
scores); outputs are compared on every row when the oracle can afford it and
on seeded samples of rows (and heads) otherwise.  Near ties are counted and
printed.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, TOL_F32, check_scores, check_selection, dev_tensor, rank_gap, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class _Cache:
    """Small FIFO cache: operands and oracle scores recur across parametrized cases."""

    def __init__(self, size):
        self.size, self.d = size, {}

    def get(self, key, make):
        if key not in self.d:
            while len(self.d) >= self.size:
                self.d.pop(next(iter(self.d)))
            self.d[key] = make()
        return self.d[key]


_ACTS, _WEIGHTS, _SCORES = _Cache(2), _Cache(1), _Cache(6)


def check_projection(w, lin, sample_rows=None):
    """Run scores -> top-k -> reduced GEMM on the GPU and check against the oracle."""
    akey = (w.wid, synth.activation_key(w, lin))
    A = _ACTS.get(akey, lambda: synth.linear_activation(w, lin))
    B = _WEIGHTS.get((w.wid, lin.tensor_b, lin.d, lin.n), lambda: synth.linear_weight(w, lin))
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    Ad, Bd = dev_tensor(A, dt), dev_tensor(B, dt)
    Y, idx, s, k = R.rmm_linear(Ad, Bd, lin.rho)
    assert k == oracle.retained_count(lin.rho, lin.d)
    s_gpu = s.cpu().numpy()
    s_ora = _SCORES.get(akey, lambda: oracle.column_scores(A))
    rms = check_scores(s_gpu, s_ora)
    near = check_selection(idx.cpu().numpy(), s_gpu, s_ora, k)
    I = idx.cpu().numpy()[:k]
    if sample_rows is None:
        got = Y.float().cpu().numpy()
        want = oracle.reduced_product(A, B, I)
    else:
        rows = np.sort(np.random.default_rng(lin.m + lin.n).choice(lin.m, size=sample_rows, replace=False))
        got = Y.float().cpu().numpy()[rows]
        want = oracle.reduced_product(A[rows], B, I)
    err = rel_fro(got, want)
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    print(f"  {w.key}/{lin.name}: k={k} rel_fro={err:.2e} near_tie={near} gap={rank_gap(s_ora, k):.2e} score_rms={rms:.2e}")
    assert err < tol
    del Ad, Bd, Y
    return near


# ------------------------------------------------------------------ xw fp32
def test_xw_fp32_64x512():
    w = synth.WORKLOADS["xw-fp32-64x512"]
    check_projection(w, w.linears[0])
    _free()


# ------------------------------------------------------------------ LLaMA-3.2-1B projections
W1B = synth.WORKLOADS["llama3.2-1b-proj-2k"]


@pytest.mark.parametrize("name", sorted([l.name for l in W1B.linears]))
def test_llama1b_projection(name):
    lin = [l for l in W1B.linears if l.name == name][0]
    check_projection(W1B, lin)
    _free()


# ------------------------------------------------------------------ attention helpers
def check_qk(Q, Kt, k, heads, rows_per_head, seed=0):
    Lq, Hq, dh = Q.shape
    Hkv = Kt.shape[0]
    Qd, Ktd = dev_tensor(Q, torch.bfloat16), dev_tensor(Kt, torch.bfloat16)
    S, idx = R.rmm_qk(Qd, Ktd, k)
    sc = R.rmm_colnorm(Qd.permute(1, 0, 2)).cpu().numpy()
    idx = idx.cpu().numpy()
    rng = np.random.default_rng(seed)
    near = 0
    for h in heads:
        s_ora = oracle.column_scores(Q[:, h, :])
        check_scores(sc[h], s_ora)
        near += check_selection(idx[h], sc[h], s_ora, k)
        rows = np.sort(rng.choice(Lq, size=min(rows_per_head, Lq), replace=False))
        got = S[h][torch.from_numpy(rows).to(DEV)].cpu().numpy()
        want = oracle.reduced_product(Q[rows, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], idx[h][:k])
        assert rel_fro(got, want) < TOL_BF16
    del S, Qd, Ktd
    return near


def check_pv(P, V, k, heads, rows_per_head, seed=0):
    """P: torch bf16 on the device [Hq][Lq][Lk]; V numpy [Lk][Hkv][dh]."""
    Hq, Lq, Lk = P.shape
    Hkv = V.shape[1]
    Vd = dev_tensor(V, torch.bfloat16)
    O, idx = R.rmm_pv(P, Vd, k)
    sc = R.rmm_colnorm(P).cpu().numpy()
    idx = idx.cpu().numpy()
    rng = np.random.default_rng(seed)
    near = 0
    for h in heads:
        Ph = P[h].float().cpu().numpy()
        s_ora = oracle.column_scores(Ph)
        check_scores(sc[h], s_ora, atol=1e-30)
        near += check_selection(idx[h], sc[h], s_ora, k)
        rows = np.sort(rng.choice(Lq, size=min(rows_per_head, Lq), replace=False))
        got = O[torch.from_numpy(rows).to(DEV), h, :].float().cpu().numpy()
        want = oracle.reduced_product(Ph[rows], V[:, oracle.kv_head(h, Hq, Hkv), :], idx[h][:k])
        assert rel_fro(got, want) < TOL_BF16
        del Ph
    del O, Vd
    return near


# ------------------------------------------------------------------ attention, 32 heads x 4096
def test_attention_32h_4k_full():
    w = synth.WORKLOADS["attn-32h-4k"]
    at = w.attention
    Q, Kt, V = synth.attention_operands(w)
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    n1 = check_qk(Q, Kt, kf, heads=range(at.Hq), rows_per_head=256)
    P = synth.causal_probs(Q, Kt, 1.0 / math.sqrt(at.dh), device=DEV)
    n2 = check_pv(P, V, kt, heads=[0, 7, 19, 31], rows_per_head=256)
    print(f"  attn-32h-4k: near ties qk={n1} pv={n2}")
    del P
    _free()


def test_attention_chain_against_oracle():
    """QK^T -> causal softmax -> PV end to end (reduced size) against the float64 chain."""
    w = synth.WORKLOADS["attn-32h-4k"]
    L, Hq = 512, 4
    Q, Kt, V = synth.attention_operands(w, L=L, Hq=Hq, Hkv=Hq)
    ref = oracle.attention_chain(Q, Kt, V, 0.5)
    kf = R.rmm_k_from_rho(0.5, 128)
    kt = R.rmm_k_from_rho(0.5, L)
    S, I = R.rmm_qk(dev_tensor(Q, torch.bfloat16), dev_tensor(Kt, torch.bfloat16), kf)
    mask = torch.ones(L, L, dtype=torch.bool, device=DEV).triu(1)
    P = torch.softmax((S / math.sqrt(128)).masked_fill(mask, float("-inf")), dim=-1).to(torch.bfloat16)
    O, J = R.rmm_pv(P, dev_tensor(V, torch.bfloat16), kt)
    err = rel_fro(O.float().cpu().numpy(), ref["O"])
    J = J.cpu().numpy()[:, :kt]
    overlap = np.mean([len(set(J[h]) & set(ref["J"][h])) / kt for h in range(Hq)])
    # Feature selection sees the same Q bytes as the oracle: the gap rule applies.
    qs = R.rmm_colnorm(dev_tensor(Q, torch.bfloat16).permute(1, 0, 2)).cpu().numpy()
    Ig = I.cpu().numpy()
    for h in range(Hq):
        check_selection(Ig[h], qs[h], oracle.column_scores(Q[:, h, :]), kf)
    # Token sets are chosen from P, which the GPU chain rounds to bf16 and the
    # float64 chain does not: report the overlap, require near agreement.
    print(f"  chain: rel_fro={err:.2e} token-set overlap={overlap:.4f}")
    assert err < TOL_BF16
    assert overlap > 0.95
    _free()


# ------------------------------------------------------------------ LLaMA-3.1-8B layer, 16k tokens
W8B = synth.WORKLOADS["llama3.1-8b-layer-16k"]


@pytest.mark.parametrize("name", [l.name for l in W8B.linears])
def test_llama8b_projection_full(name):
    lin = [l for l in W8B.linears if l.name == name][0]
    check_projection(W8B, lin, sample_rows=96)
    _free()


def test_llama8b_attention_full():
    at = W8B.attention
    Q, Kt, V = synth.attention_operands(W8B)
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    n1 = check_qk(Q, Kt, kf, heads=range(at.Hq), rows_per_head=48)
    _free()
    P = synth.causal_probs(Q, Kt, 1.0 / math.sqrt(at.dh), device=DEV)
    n2 = check_pv(P, V, kt, heads=[0, 31], rows_per_head=48)
    print(f"  llama3.1-8b attention: near ties qk={n1} pv={n2}")
    del P
    _free()


# ------------------------------------------------------------------ LLaMA-3.1-70B layer
W70 = synth.WORKLOADS["llama3.1-70b-layer"]


@pytest.mark.parametrize("name", sorted([l.name for l in W70.linears if "@m16@" in l.name]))
def test_llama70b_decode_projection(name):
    lin = [l for l in W70.linears if l.name == name][0]
    check_projection(W70, lin)
    _free()


@pytest.mark.parametrize("name", sorted([l.name for l in W70.linears if "@m8192@" in l.name]))
def test_llama70b_prefill_projection(name):
    lin = [l for l in W70.linears if l.name == name][0]
    check_projection(W70, lin, sample_rows=64)
    _free()


def test_llama70b_attention_full():
    at = W70.attention
    Q, Kt, V = synth.attention_operands(W70)
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    check_qk(Q, Kt, kf, heads=[0, 9, 40, 63], rows_per_head=48)
    _free()
    P = synth.causal_probs(Q, Kt, 1.0 / math.sqrt(at.dh), device=DEV)
    check_pv(P, V, kt, heads=[0, 63], rows_per_head=48)
    del P
    _free()

"""Causal Q K^T and P V at the workloads' full sizes, in the launch configuration
bench.py times (causal=True, 32 or 64 query heads over 8 kv heads).

rmm_qk (causal): every head's feature selection is checked against the float64
oracle under the gap rule (and bit-exactly against the oracle's selection on
the GPU's own scores).  S is filled with NaN before the call; one row from
every 128-query block of every head (plus the first and last rows) is
compared with the oracle's reduced product over all the column tiles the
causal tile list holds for that row, and the columns past them must still be
NaN: that pins the closed-form tile list at hundreds of tiles per head.

rmm_pv (causal): the entries of P above the causal diagonal are overwritten
with NaN before the call; the library must treat them as zeros (reading R8).
The oracle reads the same bytes with those entries set to zero.  Every head's
token selection is checked (the oracle's column norms over each head's full
P), and one output row from every 128-query block of every head against the
oracle's reduced product with the GPU's kept tokens.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, check_scores, check_selection, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TILE = 128


def _rows_to_check(L, seed):
    """One seeded row in every 128-row block, plus the first and the last row."""
    rng = np.random.default_rng(seed)
    rows = {0, L - 1}
    for b0 in range(0, L, TILE):
        rows.add(int(rng.integers(b0, min(b0 + TILE, L))))
    return np.array(sorted(rows))


class _State:
    """GPU results of one workload, kept while its head groups are checked."""
    key = None
    data = None


def _free():
    _State.key, _State.data = None, None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(key):
    if _State.key == key:
        return _State.data
    _free()
    w = synth.WORKLOADS[key]
    at = w.attention
    Q, Kt, V = synth.attention_operands(w)
    Lq, Hq, dh = Q.shape
    Hkv, _, Lk = Kt.shape
    kf = oracle.retained_count(at.rho, at.dh)
    kt = oracle.retained_count(at.rho, at.L)
    Qd, Ktd, Vd = dev_tensor(Q, torch.bfloat16), dev_tensor(Kt, torch.bfloat16), dev_tensor(V, torch.bfloat16)
    print(f"  {key}: causal rmm_qk, Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} kf={kf}", flush=True)
    S = torch.full((Hq, Lq, Lk), float("nan"), dtype=torch.float32, device=DEV)
    fs = torch.empty((Hq, dh), dtype=torch.float32, device=DEV)
    S, I = R.rmm_qk(Qd, Ktd, kf, S=S, causal=True, feat_scores=fs)
    rows = _rows_to_check(Lq, 17)
    rows_d = torch.from_numpy(rows).to(DEV)
    S_rows = S[:, rows_d, :].cpu().numpy()            # [Hq][rows][Lk]
    del S
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"  {key}: causal rmm_pv, kt={kt}", flush=True)
    P = synth.causal_probs(Qd, Ktd, 1.0 / math.sqrt(at.dh), device=DEV)
    upper = torch.ones((Lq, Lk), dtype=torch.bool, device=DEV).triu_(1 + (Lk - Lq))
    for h in range(Hq):
        P[h].masked_fill_(upper, float("nan"))
    del upper
    ts = torch.empty((Hq, Lk), dtype=torch.float32, device=DEV)
    O, J = R.rmm_pv(P, Vd, kt, causal=True, tok_scores=ts)
    torch.cuda.synchronize()
    data = dict(Q=Q, Kt=Kt, V=V, P=P, kf=kf, kt=kt, rows=rows, S_rows=S_rows,
                I=I.cpu().numpy(), fs=fs.cpu().numpy(), J=J.cpu().numpy(), ts=ts.cpu().numpy(),
                O_rows=O[rows_d].float().cpu().numpy())
    del O
    _State.key, _State.data = key, data
    return data


def _check_qk_heads(key, heads):
    g = _run(key)
    Q, Kt, kf, rows = g["Q"], g["Kt"], g["kf"], g["rows"]
    Lq, Hq, _ = Q.shape
    Hkv, _, Lk = Kt.shape
    off = Lk - Lq
    c0 = 1 + (TILE - 1 + off) // TILE            # column tiles held by tile row 0
    tiles_n = -(-Lk // TILE)
    near = 0
    for h in heads:
        s_ora = oracle.column_scores(Q[:, h, :])
        check_scores(g["fs"][h], s_ora)
        near += check_selection(g["I"][h], g["fs"][h], s_ora, kf)
        I = g["I"][h][:kf]
        want = oracle.reduced_product(Q[rows, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], I)
        for j, t in enumerate(rows):
            ncol = min(max(t // TILE + c0, 0), tiles_n) * TILE
            ncol = min(ncol, Lk)
            assert ncol >= min(t + off + 1, Lk), "the tile list misses a column the row needs"
            got = g["S_rows"][h, j]
            assert np.all(np.isfinite(got[:ncol])), (h, t, "unwritten entry inside the tile list")
            assert rel_fro(got[:ncol], want[j, :ncol]) < TOL_BF16, (h, t)
            assert np.all(np.isnan(got[ncol:])), (h, t, "a tile past the causal tile list was written")
    return near


def _check_pv_heads(key, heads):
    g = _run(key)
    V, P, kt, rows = g["V"], g["P"], g["kt"], g["rows"]
    Hq, Lq, Lk = P.shape
    Hkv = V.shape[1]
    near = 0
    for h in heads:
        # the causal matrix the library reads: the bytes of P with the entries
        # above the diagonal taken as zero
        Ph = torch.tril(P[h].float().cpu(), diagonal=Lk - Lq).numpy()
        assert np.all(np.isfinite(Ph))
        s_ora = oracle.column_scores(Ph)
        check_scores(g["ts"][h], s_ora, atol=1e-30)
        near += check_selection(g["J"][h], g["ts"][h], s_ora, kt)
        J = g["J"][h][:kt]
        want = oracle.reduced_product(Ph[rows], V[:, oracle.kv_head(h, Hq, Hkv), :], J)
        got = g["O_rows"][:, h, :]
        assert np.all(np.isfinite(got)), (h, "a NaN above the diagonal reached the output")
        assert rel_fro(got, want) < TOL_BF16, h
        del Ph
    return near


def _groups(Hq, n):
    step = Hq // n
    return [list(range(i, i + step)) for i in range(0, Hq, step)]


CASES = [("attn-32h-4k", 32, 1), ("llama3.1-8b-layer-16k", 32, 4), ("llama3.1-70b-layer", 64, 4)]
PARAMS = [(key, tuple(hs)) for key, Hq, n in CASES for hs in _groups(Hq, n)]


@pytest.mark.parametrize("key,heads", PARAMS, ids=[f"{k}-h{h[0]}-{h[-1]}" for k, h in PARAMS])
def test_causal_qk_pv_full(key, heads):
    n1 = _check_qk_heads(key, heads)
    n2 = _check_pv_heads(key, heads)
    print(f"  {key} heads {heads[0]}..{heads[-1]}: near ties qk={n1} pv={n2}")
    if heads[-1] == synth.WORKLOADS[key].attention.Hq - 1:
        _free()

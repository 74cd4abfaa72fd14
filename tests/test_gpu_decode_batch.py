"""Parity of the batched decode step (rmm_attention_decode_batch) with the
float64 oracle, one sequence at a time.

Each sequence b has its own cache of lens[b] tokens inside a padded
[B, ..., Lmax] buffer whose unused positions hold NaN: nothing past a
sequence's length may be read for its scores or selected.  Per (sequence,
head): the kept features are the top k_feat of |q| (exact, so bit-exact
against the oracle), the token scores match the oracle's probabilities,
the kept tokens follow the gap rule, and O matches the oracle's
P[:, J] V[J, :] to the bf16 bound.  With one sequence the call equals
rmm_attention with Lq = 1 bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, check_selection, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF = torch.bfloat16
W = synth.WORKLOADS["attn-32h-4k"]


def _batch(lens, Hq, Hkv, seed):
    """Per-sequence Q (the last position of its context), K and V, padded to Lmax with NaN."""
    B, Lmax, dh = len(lens), max(lens), 128
    Qb = np.zeros((B, Hq, dh), np.float32)
    Ktb = np.full((B, Hkv, dh, Lmax), np.nan, np.float32)
    Vb = np.full((B, Lmax, Hkv, dh), np.nan, np.float32)
    per = []
    for b, L in enumerate(lens):
        Q, Kt, V = synth.attention_operands(W, seed=seed + b, L=L, Hq=Hq, Hkv=Hkv)
        Qb[b] = Q[L - 1]
        Ktb[b, :, :, :L] = Kt
        Vb[b, :L] = V
        per.append((np.ascontiguousarray(Q[L - 1:]), Kt, V))
    return Qb, Ktb, Vb, per


def _run(Qb, Ktb, Vb, lens, kts, kf, kt_max):
    B, Hq, _ = Qb.shape
    Lmax = Ktb.shape[3]
    ts = torch.full((B * Hq, Lmax), 7.0, dtype=torch.float32, device=DEV)
    O, I, J = R.rmm_attention_decode_batch(
        dev_tensor(Qb, BF), dev_tensor(Ktb, BF), dev_tensor(Vb, BF),
        torch.tensor(lens, dtype=torch.int32, device=DEV), torch.tensor(kts, dtype=torch.int32, device=DEV),
        kf, kt_max, tok_scores=ts)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), I.cpu().numpy(), J.cpu().numpy(), ts.cpu().numpy()


def check_batch(lens, Hq, Hkv, kf, rho, seed=0):
    kts = [oracle.retained_count(rho, L) for L in lens]
    Qb, Ktb, Vb, per = _batch(lens, Hq, Hkv, seed)
    O, I, J, ts = _run(Qb, Ktb, Vb, lens, kts, kf, max(kts))
    assert np.all(np.isfinite(O)), "a NaN past some sequence's length was read"
    near = 0
    for b, (L, kt) in enumerate(zip(lens, kts)):
        Q, Kt, V = per[b]
        ref = oracle.reduced_attention(Q, Kt, V, kf, kt, causal=True)
        for h in range(Hq):
            r = b * Hq + h
            fs = np.abs(Qb[b, h].astype(np.float64))          # the call's feature scores: |q|, exact
            near += check_selection(I[r], fs, oracle.column_scores(Q[:, h, :]), kf)
            tok = ts[r, :L]
            assert np.all(np.isneginf(ts[r, L:])), "positions past the context must score -inf"
            # the oracle's token scores with the GPU's feature set (a tie swap in I must not move them)
            S = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], I[r][:kf])[None]
            P = oracle.causal_softmax(S, 128 ** -0.5)[0]
            tok_ora = oracle.column_scores(P)
            np.testing.assert_allclose(tok, tok_ora, rtol=2e-5, atol=1e-6 * tok_ora.max())
            near += check_selection(J[r], tok, tok_ora, kt)
            want = oracle.reduced_product(P, V[:, oracle.kv_head(h, Hq, Hkv), :], J[r][:kt])
            assert rel_fro(O[b, h][None], want) < TOL_BF16, f"sequence {b} head {h}"
        # the whole chain in float64 on its own selections agrees too (no near tie here moves O far)
        assert rel_fro(O[b], ref["O"][0]) < 2 * TOL_BF16
    return near


CASES = [
    # lens, Hq, Hkv, k_feat, rho
    ([300], 4, 2, 64, 0.5),
    ([1, 7, 64, 300, 1025], 4, 2, 64, 0.5),
    ([2000, 17, 1500, 999], 8, 2, 100, 0.3),
    ([4096] * 3 + [257, 33, 1], 8, 8, 1, 0.8),
    ([129, 128, 127, 700], 2, 1, 128, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{len(c[0])}_Lmax{max(c[0])}_h{c[1]}x{c[2]}_kf{c[3]}_rho{c[4]}")
def test_decode_batch(case):
    lens, Hq, Hkv, kf, rho = case
    print(f"  near ties: {check_batch(lens, Hq, Hkv, kf, rho)}")


def test_decode_batch_one_sequence_equals_rmm_attention():
    L, Hq, Hkv, kf, kt = 1000, 4, 2, 64, 500
    Q, Kt, V = synth.attention_operands(W, seed=5, L=L, Hq=Hq, Hkv=Hkv)
    Qd = dev_tensor(np.ascontiguousarray(Q[L - 1:]), BF)
    Ktd, Vd = dev_tensor(Kt, BF), dev_tensor(V, BF)
    O1, I1, J1 = R.rmm_attention(Qd, Ktd, Vd, kf, kt, causal=True)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    kts = torch.tensor([kt], dtype=torch.int32, device=DEV)
    O2, I2, J2 = R.rmm_attention_decode_batch(Qd.reshape(1, Hq, 128), Ktd[None], Vd[None], lens, kts, kf, kt)
    assert torch.equal(I1, I2) and torch.equal(J1, J2)
    assert torch.equal(O1.reshape(1, Hq, 128), O2)


def test_decode_batch_counts_are_clamped():
    """k_tok above a sequence's length or above kt_max, or below 1, is clamped to
    [1, min(lens[b], kt_max)]; the index row then lists the clamped count first."""
    lens = [50, 300, 80]
    Hq, Hkv, kf, kt_max = 2, 1, 32, 100
    Qb, Ktb, Vb, per = _batch(lens, Hq, Hkv, 9)
    O, I, J, ts = _run(Qb, Ktb, Vb, lens, [400, 250, 0], kf, kt_max)
    assert np.all(np.isfinite(O))
    for b, (L, kt) in enumerate(zip(lens, [50, 100, 1])):
        Q, Kt, V = per[b]
        for h in range(Hq):
            r = b * Hq + h
            S = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], I[r][:kf])[None]
            P = oracle.causal_softmax(S, 128 ** -0.5)[0]
            assert np.array_equal(J[r][:kt], oracle.select_top(ts[r, :L].astype(np.float64), kt))
            # the rest of the row is padding: no position at or past lens[b] is listed
            assert np.all(J[r][kt:] == -1), (b, h, J[r][kt:][J[r][kt:] != -1][:8])
            want = oracle.reduced_product(P, V[:, oracle.kv_head(h, Hq, Hkv), :], J[r][:kt])
            assert rel_fro(O[b, h][None], want) < TOL_BF16


def test_decode_batch_in_a_graph():
    lens = [700, 33, 1500]
    Hq, Hkv, kf = 4, 2, 64
    kts = [oracle.retained_count(0.5, L) for L in lens]
    Qb, Ktb, Vb, _ = _batch(lens, Hq, Hkv, 11)
    Qd, Ktd, Vd = dev_tensor(Qb, BF), dev_tensor(Ktb, BF), dev_tensor(Vb, BF)
    ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kd = torch.tensor(kts, dtype=torch.int32, device=DEV)
    O = torch.empty((3, Hq, 128), dtype=BF, device=DEV)
    I = torch.empty((3 * Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=DEV)
    J = torch.empty((3 * Hq, R.rmm_k_pad(max(kts))), dtype=torch.int32, device=DEV)
    ws = torch.empty(R.rmm_attention_decode_batch_workspace_bytes(3, Hq, 128, max(lens), max(kts)),
                     dtype=torch.uint8, device=DEV)

    def step():
        R.rmm_attention_decode_batch(Qd, Ktd, Vd, ld, kd, kf, max(kts), O=O, idx_feat=I, idx_tok=J, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = (O.clone(), I.clone(), J.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        O.fill_(float("nan"))
        I.fill_(-7)
        J.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, ref[0]) and torch.equal(I, ref[1]) and torch.equal(J, ref[2]), f"replay {rep}"


def test_decode_batch_bench_shape_sampled():
    """The bench's batched step: 16 sequences with contexts drawn uniformly from
    [4096, 16384] in a 16384-token cache, 32 query / 8 kv heads, rho = 0.5;
    every sequence checked on a sample of its heads."""
    rng = np.random.default_rng([0, 91, 16])
    lens = [int(x) for x in np.sort(rng.integers(4096, 16384 + 1, size=16))]
    Hq, Hkv, kf = 32, 8, 64
    kts = [oracle.retained_count(0.5, L) for L in lens]
    B, Lmax, dh = len(lens), 16384, 128
    Qb = np.zeros((B, Hq, dh), np.float32)
    Ktb = np.zeros((B, Hkv, dh, Lmax), np.float32)
    Vb = np.zeros((B, Lmax, Hkv, dh), np.float32)
    per = []
    for b, L in enumerate(lens):
        Q, Kt, V = synth.attention_operands(W, seed=100 + b, L=L, Hq=Hq, Hkv=Hkv)
        Qb[b] = Q[L - 1]
        Ktb[b, :, :, :L] = Kt
        Vb[b, :L] = V
        per.append((Q[L - 1:], Kt, V))
    O, I, J, ts = _run(Qb, Ktb, Vb, lens, kts, kf, max(kts))
    pick = np.random.default_rng(7)
    for b, (L, kt) in enumerate(zip(lens, kts)):
        Q, Kt, V = per[b]
        for h in pick.choice(Hq, size=3, replace=False):
            r = b * Hq + h
            check_selection(I[r], np.abs(Qb[b, h].astype(np.float64)), oracle.column_scores(Q[:, h, :]), kf)
            S = oracle.reduced_product(Q[:, h, :], Kt[oracle.kv_head(h, Hq, Hkv)], I[r][:kf])[None]
            P = oracle.causal_softmax(S, 128 ** -0.5)[0]
            tok = oracle.column_scores(P)
            np.testing.assert_allclose(ts[r, :L], tok, rtol=2e-5, atol=1e-6 * tok.max())
            check_selection(J[r], ts[r, :L], tok, kt)
            want = oracle.reduced_product(P, V[:, oracle.kv_head(h, Hq, Hkv), :], J[r][:kt])
            assert rel_fro(O[b, h][None], want) < TOL_BF16, f"sequence {b} head {h}"

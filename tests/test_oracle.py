"""Pins for the CPU oracle: closed forms, exact arithmetic, brute force, identities.

None of these re-types the oracle's own formula: each checks a fact that the
pages' definitions or plain mathematics fix, chosen so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- k
def test_retained_count_workload_table():
    rows = json.load(open(os.path.join(GOLD, "retained_counts.json")))
    for r in rows["rows"] + rows["decimal_traps"]:
        assert O.retained_count(r["rho"], r["d"]) == r["k"], r


def test_retained_count_matches_integer_arithmetic():
    # rho = p / 10^q exactly (a decimal the caller typed): k = ceil(p*d / 10^q)
    # computed with integers only.
    rng = np.random.default_rng(1)
    for _ in range(4000):
        q = int(rng.integers(1, 5))
        den = 10 ** q
        p = int(rng.integers(1, den + 1))
        d = int(rng.integers(1, 40000))
        rho = float(f"{p}e-{q}")
        assert O.retained_count(rho, d) == (p * d + den - 1) // den


@pytest.mark.parametrize("rho", [0.0, -0.1, 1.0000001, float("nan"), 2.0])
def test_retained_count_rejects_bad_rho(rho):
    with pytest.raises(ValueError):
        O.retained_count(rho, 10)


def test_retained_count_edges():
    assert O.retained_count(1.0, 1) == 1
    assert O.retained_count(1e-9, 5) == 1          # any positive rho keeps at least one index
    assert O.retained_count(1.0, 28672) == 28672
    with pytest.raises(ValueError):
        O.retained_count(0.5, 0)


# ---------------------------------------------------------------------- scores
def test_scores_closed_forms():
    m = 7
    A = np.zeros((m, 5))
    A[:, 0] = -2.5                      # constant column c: |c| * sqrt(m)
    A[:2, 1] = [3.0, 4.0]               # 3-4-5
    A[:3, 2] = [1.0, -2.0, 2.0]         # 1-2-2-3
    A[0, 4] = -9.0                      # single entry: its magnitude
    s = O.column_scores(A)
    assert s.shape == (5,)
    assert s[0] == pytest.approx(2.5 * math.sqrt(m), rel=1e-15)
    assert s[1] == 5.0
    assert s[2] == 3.0
    assert s[3] == 0.0
    assert s[4] == 9.0


def test_scores_run_over_rows_not_columns():
    # A non-square matrix whose row norms and column norms differ: column j of
    # A = [[1, 2, 2], [0, 0, 0]] has norm (1, 2, 2), its rows have (3, 0).
    A = np.array([[1.0, 2.0, 2.0], [0.0, 0.0, 0.0]])
    np.testing.assert_array_equal(O.column_scores(A), [1.0, 2.0, 2.0])


def test_scores_invariances():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((33, 9))
    s = O.column_scores(A)
    np.testing.assert_allclose(O.column_scores(A[rng.permutation(33)]), s, rtol=1e-14)
    alpha = rng.uniform(-3, 3, 9)
    np.testing.assert_allclose(O.column_scores(A * alpha), s * np.abs(alpha), rtol=1e-14)
    # Sum of squared column norms = squared Frobenius norm.
    assert math.fsum(s ** 2) == pytest.approx(float((A ** 2).sum()), rel=1e-13)


# ------------------------------------------------------------------- selection
def _brute_best(s, k):
    """All k-subsets: minimise the dropped squared mass, then the lexicographic order."""
    d = len(s)
    best = None
    for I in itertools.combinations(range(d), k):
        drop = [j for j in range(d) if j not in I]
        mass = math.fsum(float(s[j]) ** 2 for j in drop)
        key = (mass, I)
        if best is None or key < best:
            best = key
    return best


def _brute_minmax(s, k):
    d = len(s)
    return min(max([float(s[j]) for j in range(d) if j not in I], default=-1.0)
               for I in itertools.combinations(range(d), k))


@pytest.mark.parametrize("kind", ["random", "ties", "zeros", "integers"])
def test_select_top_is_bruteforce_optimum(kind):
    rng = np.random.default_rng({"random": 3, "ties": 4, "zeros": 5, "integers": 6}[kind])
    for trial in range(40):
        d = int(rng.integers(1, 11))
        if kind == "random":
            s = rng.random(d)
        elif kind == "ties":
            s = rng.integers(0, 3, d).astype(float) * 0.75
        elif kind == "zeros":
            s = np.where(rng.random(d) < 0.5, 0.0, rng.random(d))
        else:
            s = rng.integers(0, 6, d).astype(float)
        for k in range(1, d + 1):
            I = O.select_top(s, k)
            mass, lexbest = _brute_best(s, k)
            assert tuple(I.tolist()) == lexbest, (s, k)
            dropped = [j for j in range(d) if j not in set(I.tolist())]
            assert math.fsum(float(s[j]) ** 2 for j in dropped) == mass
            # minimax reading: the largest dropped score is as small as possible
            assert max([float(s[j]) for j in dropped], default=-1.0) == _brute_minmax(s, k)
            # every kept score >= every dropped score
            if dropped:
                assert min(s[I]) >= max(s[dropped])


def test_select_top_special_cases():
    s = np.full(9, 0.3)
    np.testing.assert_array_equal(O.select_top(s, 4), [0, 1, 2, 3])    # all tied -> lowest indices
    r = np.random.default_rng(7).random(50)
    np.testing.assert_array_equal(O.select_top(r, 50), np.arange(50))   # k = d keeps everything
    t = np.array([0.1, 0.9, 0.2, 0.9, 0.5])
    np.testing.assert_array_equal(O.select_top(t, 1), [1])              # argmax, lowest index on a tie
    np.testing.assert_array_equal(O.select_top(t, 3), [1, 3, 4])        # ascending order
    with pytest.raises(ValueError):
        O.select_top(t, 0)
    with pytest.raises(ValueError):
        O.select_top(t, 6)


def test_random_subset_never_beats_topk():
    # Control: a random k-subset never drops less squared mass than top-k.
    rng = np.random.default_rng(8)
    for _ in range(200):
        d = int(rng.integers(2, 200))
        s = np.abs(rng.standard_normal(d)) * np.exp(rng.standard_normal(d))
        k = int(rng.integers(1, d))
        I = O.select_top(s, k)
        R = rng.choice(d, size=k, replace=False)
        m_top = math.fsum(s ** 2) - math.fsum(s[I] ** 2)
        m_rand = math.fsum(s ** 2) - math.fsum(s[R] ** 2)
        assert m_top <= m_rand + 1e-12 * math.fsum(s ** 2)


# ----------------------------------------------------------------- the product
def test_worked_example_by_hand():
    # A = [[3,0,1],[4,0,1]]: column norms (5, 0, sqrt 2).  rho = 0.5, d = 3 ->
    # k = ceil(1.5) = 2 -> I = {0, 2}.  With B = [[1,2],[3,4],[5,6]]:
    # Y = [[3*1+1*5, 3*2+1*6], [4*1+1*5, 4*2+1*6]] = [[8,12],[9,14]].
    A = np.array([[3.0, 0.0, 1.0], [4.0, 0.0, 1.0]])
    B = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    Y, I, s, k = O.rmm(A, B, 0.5)
    assert k == 2
    np.testing.assert_array_equal(I, [0, 2])
    np.testing.assert_allclose(s, [5.0, 0.0, math.sqrt(2.0)], rtol=1e-15)
    np.testing.assert_array_equal(Y, [[8.0, 12.0], [9.0, 14.0]])


def test_rho_one_is_the_dense_product():
    # Integer-valued operands make every float64 product and sum exact, so
    # rho = 1 must reproduce the dense product bit for bit.
    rng = np.random.default_rng(9)
    A = rng.integers(-50, 50, (17, 23)).astype(np.float64)
    B = rng.integers(-50, 50, (23, 11)).astype(np.float64)
    Y, I, _, k = O.rmm(A, B, 1.0)
    assert k == 23
    np.testing.assert_array_equal(I, np.arange(23))
    exact = np.array([[sum(int(A[i, t]) * int(B[t, j]) for t in range(23)) for j in range(11)]
                      for i in range(17)], dtype=np.float64)
    np.testing.assert_array_equal(Y, exact)
    Ar = rng.standard_normal((17, 23))
    Yr, _, _, _ = O.rmm(Ar, B, 1.0)
    np.testing.assert_allclose(Yr, Ar @ B, rtol=1e-13, atol=1e-13)


def test_complement_identity():
    rng = np.random.default_rng(10)
    A = rng.standard_normal((31, 40)) * np.exp(rng.standard_normal(40))
    B = rng.standard_normal((40, 13))
    Y, I, _, _ = O.rmm(A, B, 0.3)
    Ic = np.setdiff1d(np.arange(40), I)
    Yc = O.reduced_product(A, B, Ic)
    np.testing.assert_allclose(Y + Yc, A @ B, rtol=0, atol=1e-12 * np.abs(A @ B).max())


def test_error_equals_dropped_mass_for_orthonormal_rows():
    # B with orthonormal rows (d <= n): ||AB - A_I B_I||_F^2 = sum_{j not in I} s_j^2.
    rng = np.random.default_rng(11)
    m, d, n = 25, 12, 30
    A = rng.standard_normal((m, d)) * np.exp(rng.standard_normal(d))
    Qm, _ = np.linalg.qr(rng.standard_normal((n, d)))
    B = Qm.T                                   # [d, n], B B^T = I_d
    for rho in (0.25, 0.5, 0.75, 1.0):
        Y, I, s, k = O.rmm(A, B, rho)
        err = np.linalg.norm(A @ B - Y) ** 2
        drop = np.setdiff1d(np.arange(d), I)
        assert err == pytest.approx(math.fsum(s[drop] ** 2), rel=1e-10, abs=1e-20)


def test_exact_when_dropped_columns_are_zero():
    rng = np.random.default_rng(12)
    A = rng.standard_normal((9, 10))
    A[:, [1, 4, 7, 8]] = 0.0
    B = rng.standard_normal((10, 6))
    Y, I, _, k = O.rmm(A, B, 0.6)
    assert k == 6
    assert not set(I.tolist()) & {1, 4, 7, 8}
    np.testing.assert_allclose(Y, A @ B, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------- attention
def test_kv_head_grouping():
    assert [O.kv_head(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [O.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert [O.kv_head(h, 64, 8) for h in (0, 7, 8, 63)] == [0, 0, 1, 7]


def test_qk_orthonormal_keys_and_head_map():
    # Kt[g] has orthonormal rows scaled by (g+1): for query head h,
    # ||Q_h Kt_g - S_h||^2 = (g+1)^2 * dropped mass of Q_h's columns.
    rng = np.random.default_rng(13)
    Lq, Lk, Hq, Hkv, dh = 19, 24, 4, 2, 8
    Q = rng.standard_normal((Lq, Hq, dh)) * np.exp(rng.standard_normal((1, Hq, dh)))
    Kt = np.empty((Hkv, dh, Lk))
    for g in range(Hkv):
        Qm, _ = np.linalg.qr(rng.standard_normal((Lk, dh)))
        Kt[g] = (g + 1) * Qm.T
    k = 3
    S, I, sc = O.reduced_qk(Q, Kt, k)
    assert S.shape == (Hq, Lq, Lk) and I.shape == (Hq, k)
    for h in range(Hq):
        g = h * Hkv // Hq
        dense = Q[:, h, :] @ Kt[g]
        drop = np.setdiff1d(np.arange(dh), I[h])
        assert np.linalg.norm(dense - S[h]) ** 2 == pytest.approx((g + 1) ** 2 * math.fsum(sc[h][drop] ** 2),
                                                                  rel=1e-10)


def test_qk_head_map_zero_and_ones():
    Lq, Lk, Hq, Hkv, dh = 3, 5, 4, 2, 4
    Q = np.ones((Lq, Hq, dh))
    Kt = np.stack([np.zeros((dh, Lk)), np.ones((dh, Lk))])
    S, _, _ = O.reduced_qk(Q, Kt, 2)
    assert np.all(S[0] == 0) and np.all(S[1] == 0)   # heads 0,1 read kv head 0
    assert np.all(S[2] == 2) and np.all(S[3] == 2)   # heads 2,3 read kv head 1 (k = 2 ones)


def test_causal_softmax_closed_forms():
    Hq, L = 2, 6
    P = O.causal_softmax(np.zeros((Hq, L, L)), 0.3)
    for i in range(L):
        np.testing.assert_allclose(P[:, i, : i + 1], 1.0 / (i + 1), rtol=1e-15)
        assert np.all(P[:, i, i + 1:] == 0.0)
    rng = np.random.default_rng(14)
    S = rng.standard_normal((Hq, L, L)) * 4
    P = O.causal_softmax(S, 0.7)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, rtol=1e-14)
    assert np.all(np.triu(P[0], 1) == 0.0) and np.all(np.triu(P[1], 1) == 0.0)
    # softmax is invariant to a per-row shift; the scale multiplies the logits
    np.testing.assert_allclose(O.causal_softmax(S + rng.standard_normal((Hq, L, 1)), 0.7), P, rtol=1e-12)
    # two allowed logits a, b in row 1: p0 = 1 / (1 + exp(scale*(b - a)))
    a, b, sc = S[0, 1, 0], S[0, 1, 1], 0.7
    assert P[0, 1, 0] == pytest.approx(1.0 / (1.0 + math.exp(sc * (b - a))), rel=1e-13)


def test_pv_uniform_causal_closed_form():
    # Q = 0 -> S = 0 -> P[i, j] = 1/(i+1) for j <= i.  Column norms
    # sqrt(sum_{i>=j} (i+1)^-2) strictly decrease in j, so J = [0, k) and
    # O[i] = (1/(i+1)) * sum_{j <= min(i, k-1)} V[j].
    rng = np.random.default_rng(15)
    L, Hq, Hkv, dh = 12, 2, 1, 5
    Q = np.zeros((L, Hq, dh))
    Kt = rng.standard_normal((Hkv, dh, L))
    V = rng.standard_normal((L, Hkv, dh))
    for rho in (0.25, 0.5, 1.0):
        out = O.attention_chain(Q, Kt, V, rho)
        k = math.ceil(rho * L - 1e-12)
        for h in range(Hq):
            np.testing.assert_array_equal(out["J"][h], np.arange(k))
        for i in range(L):
            want = V[: min(i, k - 1) + 1, 0, :].sum(axis=0) / (i + 1)
            np.testing.assert_allclose(out["O"][i, 0], want, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(out["O"][i, 1], want, rtol=1e-13, atol=1e-15)


def test_pv_scores_are_column_norms_over_query_rows():
    # P_h = [[1, 0], [0.6, 0.8]]: column norms (sqrt(1.36), 0.8) -> k=1 keeps token 0.
    P = np.array([[[1.0, 0.0], [0.6, 0.8]]])
    V = np.array([[[1.0, 2.0]], [[10.0, 20.0]]])      # [Lk=2][Hkv=1][dh=2]
    Oo, J, sc = O.reduced_pv(P, V, 1)
    np.testing.assert_allclose(sc[0], [math.sqrt(1.36), 0.8], rtol=1e-15)
    np.testing.assert_array_equal(J[0], [0])
    np.testing.assert_allclose(Oo[:, 0, :], [[1.0, 2.0], [0.6, 1.2]], rtol=1e-15)


def test_rho_one_attention_is_textbook_causal_attention():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(16)
    L, Hq, Hkv, dh = 10, 4, 2, 8
    Q = rng.standard_normal((L, Hq, dh))
    Kt = rng.standard_normal((Hkv, dh, L))
    V = rng.standard_normal((L, Hkv, dh))
    out = O.attention_chain(Q, Kt, V, 1.0)
    q = torch.from_numpy(Q).permute(1, 0, 2)                       # [Hq, L, dh]
    kk = torch.from_numpy(Kt).permute(0, 2, 1).repeat_interleave(Hq // Hkv, 0)
    vv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True)
    np.testing.assert_allclose(out["O"], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_full_softmax_closed_forms():
    Hq, Lq, Lk = 2, 3, 5
    P = O.full_softmax(np.zeros((Hq, Lq, Lk)), 0.9)
    np.testing.assert_allclose(P, 1.0 / Lk, rtol=1e-15)          # uniform over every key
    rng = np.random.default_rng(17)
    S = rng.standard_normal((Hq, Lq, Lk)) * 3
    P = O.full_softmax(S, 0.4)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, rtol=1e-14)
    assert np.all(P > 0)                                           # nothing is masked
    # two keys: p0 = 1 / (1 + exp(scale*(b - a)))
    P2 = O.full_softmax(np.array([[[2.0, -1.0]]]), 0.4)
    assert P2[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(0.4 * (-3.0))), rel=1e-14)
    # the last query of a causal square block sees every key: the rows agree
    Sq = rng.standard_normal((Hq, Lk, Lk))
    np.testing.assert_allclose(O.full_softmax(Sq, 0.4)[:, -1], O.causal_softmax(Sq, 0.4)[:, -1], rtol=1e-14)


def test_reduced_attention_separate_counts_closed_form():
    # Q = 0 -> S = 0 whatever k_feat keeps; causal P[i, j] = 1/(i+1), so the
    # token scores fall with j and J = [0, k_tok); O[i] = sum_{j<=min(i,k_tok-1)} V[j] / (i+1).
    rng = np.random.default_rng(18)
    L, Hq, Hkv, dh = 9, 2, 1, 6
    Q = np.zeros((L, Hq, dh))
    Kt = rng.standard_normal((Hkv, dh, L))
    V = rng.standard_normal((L, Hkv, dh))
    out = O.reduced_attention(Q, Kt, V, 2, 4, causal=True)
    assert out["I"].shape == (Hq, 2) and out["J"].shape == (Hq, 4)
    np.testing.assert_array_equal(out["I"], [[0, 1], [0, 1]])      # all-zero scores: lowest indices
    for i in range(L):
        want = V[: min(i, 3) + 1, 0, :].sum(axis=0) / (i + 1)
        np.testing.assert_allclose(out["O"][i, 0], want, rtol=1e-13, atol=1e-15)
    # token score of key j: sqrt(sum_{i >= j} (i+1)^-2)
    tj = [math.sqrt(sum((i + 1) ** -2 for i in range(j, L))) for j in range(L)]
    np.testing.assert_allclose(out["tok"][1], tj, rtol=1e-14)
    # without the mask every query averages all keys: J keeps the first k_tok
    # (equal scores, lower index first) and O[i] = sum_{j<k_tok} V[j] / L
    out = O.reduced_attention(Q, Kt, V, 2, 4, causal=False)
    np.testing.assert_array_equal(out["J"][0], np.arange(4))
    np.testing.assert_allclose(out["O"][:, 1], np.broadcast_to(V[:4, 0].sum(axis=0) / L, (L, dh)), rtol=1e-13)


def test_full_attention_is_textbook_attention():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(19)
    Lq, Lk, Hq, Hkv, dh = 7, 11, 4, 2, 8
    Q = rng.standard_normal((Lq, Hq, dh))
    Kt = rng.standard_normal((Hkv, dh, Lk))
    V = rng.standard_normal((Lk, Hkv, dh))
    q = torch.from_numpy(Q).permute(1, 0, 2)
    kk = torch.from_numpy(Kt).permute(0, 2, 1).repeat_interleave(Hq // Hkv, 0)
    vv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    out = O.reduced_attention(Q, Kt, V, dh, Lk, causal=False)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=False)
    np.testing.assert_allclose(out["O"], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    # a single causal query placed after its context sees every key
    out1 = O.reduced_attention(Q[-1:], Kt, V, dh, Lk, causal=True)
    np.testing.assert_allclose(out1["O"][0], ref.permute(1, 0, 2).numpy()[-1], rtol=1e-10, atol=1e-12)


def test_w8_product_worked_example():
    # A = [1 2 3]; q rows (1, -2), (3, 4), (-5, 6); scales (0.5, 0.25); keep {0, 2}:
    # column 0: 1*(1*0.5) + 3*(-5*0.5) = -7;  column 1: 1*(-2*0.25) + 3*(6*0.25) = 4.
    A = np.array([[1.0, 2.0, 3.0]])
    q = np.array([[1, -2], [3, 4], [-5, 6]], dtype=np.int8)
    s = np.array([0.5, 0.25], dtype=np.float32)
    np.testing.assert_array_equal(O.reduced_product_w8(A, q, s, [0, 2]), [[-7.0, 4.0]])


def test_w8_product_scales_columns_and_drops_rows():
    rng = np.random.default_rng(20)
    m, d, n = 5, 9, 6
    A = rng.standard_normal((m, d))
    q = rng.integers(-127, 128, size=(d, n)).astype(np.int8)
    s = rng.uniform(0.01, 0.1, size=n).astype(np.float32)
    I = np.array([1, 4, 5, 8])
    Y = O.reduced_product_w8(A, q, s, I)
    # doubling one column's scale doubles that output column only (powers of two: exact)
    s2 = s.copy()
    s2[3] *= 2
    Y2 = O.reduced_product_w8(A, q, s2, I)
    np.testing.assert_array_equal(Y2[:, 3], 2 * Y[:, 3])
    np.testing.assert_array_equal(np.delete(Y2, 3, axis=1), np.delete(Y, 3, axis=1))
    # dropped rows of q do not matter: overwrite them and nothing changes
    qx = q.copy()
    qx[np.setdiff1d(np.arange(d), I)] = 99
    np.testing.assert_array_equal(O.reduced_product_w8(A, qx, s, I), Y)
    # element by element against the sum it stands for
    for i in range(m):
        for c in range(n):
            want = sum(A[i, t] * (float(q[t, c]) * float(s[c])) for t in I)
            assert Y[i, c] == pytest.approx(want, rel=1e-13, abs=1e-15)
    # keeping every row and unit scales is the integer product
    Yf = O.reduced_product_w8(A, q, np.ones(n, dtype=np.float32), np.arange(d))
    np.testing.assert_allclose(Yf, A @ q.astype(np.int64), rtol=1e-13)


def test_swiglu_closed_forms():
    x = np.array([0.0, math.log(3.0), -math.log(3.0), 50.0, -800.0, 1e-3])
    s = O.swiglu(x, np.ones_like(x))
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)      # sigmoid(ln 3) = 3/4
    assert s[2] == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)     # sigmoid(-ln 3) = 1/4
    assert s[3] == pytest.approx(50.0, rel=1e-15)
    assert s[4] == 0.0                                                  # e^800 overflows: x / inf
    assert s[5] == pytest.approx(1e-3 * 0.5 + 1e-6 / 4, rel=1e-9)      # x sigmoid(x) ~ x/2 + x^2/4
    rng = np.random.default_rng(21)
    g = rng.standard_normal(50) * 4
    # silu(x) - silu(-x) = x, and the up factor multiplies elementwise
    np.testing.assert_allclose(O.swiglu(g, np.ones(50)) - O.swiglu(-g, np.ones(50)), g, rtol=1e-13, atol=1e-14)
    u = rng.standard_normal(50)
    np.testing.assert_allclose(O.swiglu(g, u), O.swiglu(g, np.ones(50)) * u, rtol=1e-15)


def test_rmsnorm_worked_examples():
    # [3, 4]: mean square 12.5, so y = x / sqrt(12.5) = [0.84852..., 1.13137...]
    y = O.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    np.testing.assert_allclose(y, [[3 / np.sqrt(12.5), 4 / np.sqrt(12.5)]], rtol=1e-15)
    np.testing.assert_allclose(y, [[0.848528137423857, 1.131370849898476]], rtol=1e-14)
    # ones with eps = 3: sqrt(1 + 3) = 2, gain w applied per column
    y = O.rmsnorm(np.ones((2, 4)), np.array([1.0, 2.0, -1.0, 0.5]), 3.0)
    np.testing.assert_allclose(y, [[0.5, 1.0, -0.5, 0.25]] * 2, rtol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((7, 96)) * rng.uniform(0.1, 10.0, size=(7, 1))
    w = rng.uniform(0.5, 2.0, size=96)
    # unit gain, eps = 0: every row has mean square exactly 1
    y1 = O.rmsnorm(X, np.ones(96), 0.0)
    np.testing.assert_allclose(np.mean(y1 * y1, axis=1), 1.0, rtol=1e-13)
    # scale invariance per row with eps = 0; sign follows x
    sc = rng.uniform(0.01, 100.0, size=(7, 1))
    np.testing.assert_allclose(O.rmsnorm(X * sc, w, 0.0), O.rmsnorm(X, w, 0.0), rtol=1e-12)
    np.testing.assert_array_equal(np.sign(O.rmsnorm(X, w, 1e-5)), np.sign(X))
    # the gain multiplies columns; the normaliser is one number per row
    np.testing.assert_allclose(O.rmsnorm(X, w, 1e-5), O.rmsnorm(X, np.ones(96), 1e-5) * w, rtol=1e-15)
    r = X[:, :1] / O.rmsnorm(X, np.ones(96), 1e-5)[:, :1]
    np.testing.assert_allclose(r[:, 0], np.sqrt(np.mean(X * X, axis=1) + 1e-5), rtol=1e-13)
    # a constant row c normalises to sign(c) * w when eps = 0
    np.testing.assert_allclose(O.rmsnorm(np.full((1, 5), -2.5), np.arange(1.0, 6.0), 0.0), [[-1, -2, -3, -4, -5]],
                               rtol=1e-15)

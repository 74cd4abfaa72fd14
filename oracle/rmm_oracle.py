"""CPU oracle for Reduced Matrix Multiplication (RMM).  TEST INFRASTRUCTURE ONLY.

What it is
    A plain float64 NumPy statement of the computation described on the pages
    "Reduced Matrix Multiplication: Input-Adaptive Matrix-Product Reduction for
    LLM Inference" (gist.science explainer, Spanish and Chinese editions,
    section "Metodología" / "方法论"; arXiv:2608.13426 abstract):

      * every product has the unified form Y = A B, A the activation and B the
        weight or intermediate representation ("Metodología", first paragraph);
      * an input-dependent subset I of the shared contraction dimension d is
        kept and A[:, I] B[I, :] replaces A B ("Mecanismo Central");
      * index j is scored by the activation column norm s_j = ||A[:, j]||_2 and
        the k = ceil(rho * d) best scores are kept, rho being the user's
        retention ratio ("Estrategia de Selección");
      * the sites are the feature dimension of Q K^T, optionally the token
        dimension of P V, and the hidden dimension of projections X W
        ("Alcance de Aplicación").

    The method's result has a plain definition (a deterministic selection and
    an exact reduced product), so each function below is that definition
    written out, with library primitives (an elementwise square, a sum, a
    sort, a matmul) as steps and no blocking, fusion or reordering.

Readings where the pages are silent
    R1  k = ceil(rho*d) with rho taken as the decimal number the caller wrote
        (the shortest decimal string that round-trips the float), computed in
        exact rational arithmetic; rho must lie in (0, 1].
    R2  Ties at rank k are broken toward the lower index, which makes I unique.
    R3  I is returned in ascending index order.
    R4  No rescaling of the reduced product (the pages print the bare product).
    R5  Scores run over all rows of this call's A; attention selects per query
        head.
    R6  Grouped-query attention: query head h reads kv head g(h) = h*Hkv // Hq.
    R7  The softmax scale stays 1/sqrt(dh) whatever k is.
    R8  Causally masked probabilities are exact zeros and enter the P column
        norms as such.

Who may use it
    Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
    ``bench.py``.  The HIP library never imports, calls or links anything here,
    and nothing here imports the library.

Pins
    Every function is pinned by the CPU tests against closed forms, exact
    rational arithmetic, brute force over all k-subsets, and identities that a
    dropped term, a wrong sign/index or a transposed operand would break.  The
    only unpinned quantity is "GPU time versus the pages' published numbers":
    the pages print no numeric worked example (parity unpinned for that).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "retained_count",
    "column_scores",
    "select_top",
    "reduced_product",
    "reduced_product_w8",
    "swiglu",
    "rmsnorm",
    "rmm",
    "kv_head",
    "reduced_qk",
    "causal_softmax",
    "full_softmax",
    "reduced_pv",
    "reduced_attention",
    "attention_chain",
]


def retained_count(rho: float, d: int) -> int:
    """k = ceil(rho * d), the number of kept contraction indices.

    Follows "Estrategia de Selección" (k = ceil(rho d), rho the user-set
    retention ratio).  rho is read as a decimal (reading R1): ``repr`` gives
    the shortest decimal string that maps back to the same double, and the
    ceiling is taken on the exact rational rho*d, so rho = 0.55, d = 100 gives
    55 (a binary-float product would give 56).
    """
    if not (isinstance(d, (int, np.integer)) and d >= 1):
        raise ValueError("d must be a positive integer")
    rho = float(rho)
    if not (0.0 < rho <= 1.0) or math.isnan(rho):
        raise ValueError("rho must lie in (0, 1]")
    return int(math.ceil(Fraction(repr(rho)) * int(d)))


def column_scores(A) -> np.ndarray:
    """s_j = ||A[:, j]||_2 over every row of A, in float64.

    "Estrategia de Selección": the importance of contraction index j is the
    Euclidean norm of activation column j.  Square every entry, add down each
    column, take the square root.
    """
    A64 = np.asarray(A, dtype=np.float64)
    if A64.ndim != 2:
        raise ValueError("A must be 2-D [m, d]")
    return np.sqrt((A64 * A64).sum(axis=0))


def select_top(scores, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, ascending order.

    "Estrategia de Selección" keeps the top-k scores; readings R2/R3 fix the
    tie-break and the order.  A full sort: primary key descending score,
    secondary key ascending index; keep the first k, then sort them by index.
    """
    s = np.asarray(scores, dtype=np.float64)
    d = s.shape[0]
    if not (1 <= k <= d):
        raise ValueError("need 1 <= k <= d")
    order = np.lexsort((np.arange(d), -s))
    return np.sort(order[:k]).astype(np.int64)


def reduced_product(A, B, I) -> np.ndarray:
    """A[:, I] @ B[I, :] in float64 ("Mecanismo Central"), with no rescaling (R4)."""
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    I = np.asarray(I, dtype=np.int64)
    return A64[:, I] @ B64[I, :]


def reduced_product_w8(A, Bq, scale, I) -> np.ndarray:
    """A[:, I] @ (Bq[I, :] * scale) in float64, scale applied per output column.

    The reduced product over a weight held as INT8 values with one scale per
    output column; the abstract states that the method works with INT8
    weights, and the selection (on A) does not change.  The weight entering
    the product is exactly q * scale.
    """
    B = np.asarray(Bq, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[None, :]
    return reduced_product(A, B, I)


def swiglu(G, U) -> np.ndarray:
    """silu(G) * U elementwise in float64, silu(x) = x / (1 + e^-x).

    The gated MLP activation of a LLaMA-style layer: the input of the down
    projection, whose column scores ("Estrategia de Selección") the producer
    can accumulate as it writes it.
    """
    G64 = np.asarray(G, dtype=np.float64)
    U64 = np.asarray(U, dtype=np.float64)
    with np.errstate(over="ignore"):
        return G64 / (1.0 + np.exp(-G64)) * U64


def rmsnorm(X, w, eps: float) -> np.ndarray:
    """RMS normalisation of each row in float64: x * w / sqrt(mean(x^2) + eps).

    The normalisation that produces the A of the q, k, v, gate and up
    projections of a LLaMA-style layer; its column scores ("Estrategia de
    Selección") can be accumulated by the producer as it writes A.
    """
    X64 = np.asarray(X, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    ms = np.mean(X64 * X64, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        return X64 / np.sqrt(ms + float(eps)) * w64[None, :]


def rmm(A, B, rho: float):
    """One reduced product Y ~ A B: returns (Y, I, s, k).

    Steps in the pages' order: score the columns of A, keep the top
    k = ceil(rho d), multiply the kept slices.  Used for the projection site
    X W ("Alcance de Aplicación", MLP and linear projections).
    """
    A64 = np.asarray(A, dtype=np.float64)
    d = A64.shape[1]
    k = retained_count(rho, d)
    s = column_scores(A64)
    I = select_top(s, k)
    return reduced_product(A64, B, I), I, s, k


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head h under grouped-query attention (reading R6)."""
    return (h * Hkv) // Hq


def reduced_qk(Q, Kt, k: int):
    """Feature-reduced attention scores, per query head.

    Q  [Lq][Hq][dh] (token-major), Kt [Hkv][dh][Lk] (keys stored feature-major).
    For each query head h: s = column scores of Q_h = Q[:, h, :] over its Lq
    rows, I_h = top-k of s, S_h = Q_h[:, I_h] @ Kt[g(h)][I_h, :].
    "Alcance de Aplicación": reduce the feature dimension of Q K^T; here A = Q_h
    and B = K_h^T, so the contraction index is the head feature.

    Returns S [Hq][Lq][Lk] (float64), I [Hq][k] and the scores [Hq][dh].
    """
    Q64 = np.asarray(Q, dtype=np.float64)
    K64 = np.asarray(Kt, dtype=np.float64)
    Lq, Hq, dh = Q64.shape
    Hkv, dh2, Lk = K64.shape
    if dh2 != dh:
        raise ValueError("head dims differ")
    S = np.empty((Hq, Lq, Lk), dtype=np.float64)
    I = np.empty((Hq, k), dtype=np.int64)
    sc = np.empty((Hq, dh), dtype=np.float64)
    for h in range(Hq):
        Qh = Q64[:, h, :]
        sc[h] = column_scores(Qh)
        I[h] = select_top(sc[h], k)
        S[h] = reduced_product(Qh, K64[kv_head(h, Hq, Hkv)], I[h])
    return S, I, sc


def causal_softmax(S, scale: float) -> np.ndarray:
    """P[h, i, j] = softmax_j(scale * S[h, i, j]) over j <= i + (Lk - Lq); zero above.

    The attention probabilities between the two reduced products (reading R7
    for the scale, R8 for the exact zeros).  Row max subtracted, float64.
    """
    S64 = np.asarray(S, dtype=np.float64)
    Hq, Lq, Lk = S64.shape
    allowed = np.arange(Lk)[None, :] <= (np.arange(Lq)[:, None] + (Lk - Lq))
    P = np.zeros_like(S64)
    for h in range(Hq):
        z = np.where(allowed, S64[h] * scale, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(z), 0.0)
        P[h] = e / e.sum(axis=1, keepdims=True)
    return P


def full_softmax(S, scale: float) -> np.ndarray:
    """P[h, i, j] = softmax_j(scale * S[h, i, j]) over every key (no mask).

    The probabilities of attention without a causal mask (an encoder, or a
    query block that follows its whole context).  Row max subtracted, float64.
    """
    S64 = np.asarray(S, dtype=np.float64)
    z = S64 * scale
    z = z - z.max(axis=2, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=2, keepdims=True)


def reduced_pv(P, V, k: int):
    """Token-reduced attention output, per query head.

    P [Hq][Lq][Lk], V [Lk][Hkv][dh].  For each head h: s = column scores of
    P_h over its Lq query rows, J_h = top-k tokens, O[:, h, :] =
    P_h[:, J_h] @ V[J_h, g(h), :].  "Alcance de Aplicación": optionally reduce
    the token dimension of P V; A = P_h, B = V_g(h).

    Returns O [Lq][Hq][dh] (float64), J [Hq][k] and the scores [Hq][Lk].
    """
    P64 = np.asarray(P, dtype=np.float64)
    V64 = np.asarray(V, dtype=np.float64)
    Hq, Lq, Lk = P64.shape
    Lk2, Hkv, dh = V64.shape
    if Lk2 != Lk:
        raise ValueError("token counts differ")
    O = np.empty((Lq, Hq, dh), dtype=np.float64)
    J = np.empty((Hq, k), dtype=np.int64)
    sc = np.empty((Hq, Lk), dtype=np.float64)
    for h in range(Hq):
        sc[h] = column_scores(P64[h])
        J[h] = select_top(sc[h], k)
        O[:, h, :] = reduced_product(P64[h], V64[:, kv_head(h, Hq, Hkv), :], J[h])
    return O, J, sc


def reduced_attention(Q, Kt, V, k_feat: int, k_tok: int, causal: bool = True,
                      scale: float | None = None):
    """Reduced Q K^T -> softmax -> reduced P V for one layer, float64.

    "Alcance de Aplicación": the feature dimension of Q K^T keeps k_feat
    indices per query head (scored on Q_h), the token dimension of P V keeps
    k_tok tokens per query head (scored on P_h); "Estrategia de Selección"
    scores both by column norms.  The softmax sits between the two products;
    causal masks key u from query t when u > t + (Lk - Lq) (reading R8).

    Returns dict with S, P, O, I, J and the token scores ("tok") [Hq][Lk].
    """
    Q64 = np.asarray(Q, dtype=np.float64)
    dh = Q64.shape[2]
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    S, I, _ = reduced_qk(Q64, Kt, k_feat)
    P = causal_softmax(S, scale) if causal else full_softmax(S, scale)
    O, J, tok = reduced_pv(P, V, k_tok)
    return {"S": S, "P": P, "O": O, "I": I, "J": J, "tok": tok}


def attention_chain(Q, Kt, V, rho: float, scale: float | None = None):
    """Reduced QK^T -> causal softmax -> reduced PV for one layer, float64.

    k for the feature reduction is ceil(rho*dh), for the token reduction
    ceil(rho*Lk).  Returns dict with S, P, O, I, J (and the token scores).
    """
    dh = np.asarray(Q).shape[2]
    Lk = np.asarray(Kt).shape[2]
    return reduced_attention(Q, Kt, V, retained_count(rho, dh), retained_count(rho, Lk),
                             causal=True, scale=scale)

"""Primitive seeded draws.

Every random stream is a NumPy PCG64 generator keyed by
``SeedSequence([seed, workload_id, tensor_id])`` so that any single tensor of
any workload can be regenerated on its own, on any machine, bit for bit.

bf16 operands are produced as float32 arrays whose values are exactly
representable in bfloat16 (rounded to nearest, ties to even).  Converting such
an array to ``torch.bfloat16`` or to float64 is exact, so the GPU and the
oracle consume the same numbers.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "stream",
    "bf16_round",
    "normal",
    "outlier_activations",
    "lognormal_col_activations",
    "weight",
    "int8_per_column",
    "attention_qkv",
    "causal_probs",
]


def stream(seed: int, workload_id: int, tensor_id: int) -> np.random.Generator:
    """Independent PCG64 stream for one tensor of one workload."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload_id, tensor_id])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); finite inputs only.

    Returns float32 holding bf16-exact values.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def outlier_activations(rng: np.random.Generator, m: int, d: int, frac: float, factor: float,
                        bf16: bool = True, col_rng: np.random.Generator | None = None) -> np.ndarray:
    """N(0,1) activations with round(frac*d) outlier channels multiplied by ``factor``.

    The outlier channels are drawn uniformly without replacement from
    ``col_rng`` (by default the body's stream, after the body).  With a
    separate ``col_rng`` the first m' rows of an m-row draw equal the m'-row
    draw.
    """
    a = normal(rng, (m, d))
    n_out = int(round(frac * d))
    if n_out > 0:
        cols = (col_rng if col_rng is not None else rng).choice(d, size=n_out, replace=False)
        a[:, cols] *= np.float32(factor)
    return bf16_round(a) if bf16 else a


def lognormal_col_activations(rng: np.random.Generator, m: int, d: int, sigma: float,
                              bf16: bool = True, col_rng: np.random.Generator | None = None) -> np.ndarray:
    """A[i, j] = z[i, j] * c[j] with z ~ N(0,1) and c[j] = exp(N(0, sigma^2)).

    The column scales come from ``col_rng`` when given (then row prefixes are
    stable across m), else from ``rng`` after the body.
    """
    z = normal(rng, (m, d))
    c = np.exp(sigma * (col_rng if col_rng is not None else rng).standard_normal(d)).astype(np.float32)
    a = z * c[None, :]
    return bf16_round(a) if bf16 else a


def weight(rng: np.random.Generator, d_in: int, d_out: int, bf16: bool = True) -> np.ndarray:
    """Weight stored as B[d_in][d_out] (rows are the contraction index), N(0, 1/d_in).

    The second parameter of N(.,.) is read as the variance: std = 1/sqrt(d_in).
    """
    w = normal(rng, (d_in, d_out), std=1.0 / np.sqrt(d_in))
    return bf16_round(w) if bf16 else w


def int8_per_column(B: np.ndarray):
    """Symmetric per-output-column INT8 form of a weight B [d][n]: scale[c] =
    max_j |B[j, c]| / 127 (1 for an all-zero column), q = round(B / scale)
    clipped to [-127, 127].  Returns (q int8 [d][n], scale float32 [n]).  This
    is how the INT8 weight inputs are prepared; it is not part of the method."""
    B = np.asarray(B, dtype=np.float32)
    amax = np.abs(B).max(axis=0)
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(B / scale[None, :]), -127, 127).astype(np.int8)
    return q, scale


def attention_qkv(seed: int, workload_id: int, L: int, Hq: int, Hkv: int, dh: int,
                  sigma: float = 0.7):
    """Q, K, V for one attention layer.

    Q[t, h, j] = z * cq[h, j] and K[t, g, j] = z * ck[g, j] with z ~ N(0,1) and
    per-head, per-dimension scales c ~ log-normal(0, sigma^2) drawn independently
    for Q and K; V ~ N(0,1).

    Returns (Q [L][Hq][dh], Kt [Hkv][dh][L], V [L][Hkv][dh]) as bf16-exact
    float32.  K is handed out transposed (key-feature-major) because that is
    the operand layout the reduced QK^T product consumes.
    """
    rq = stream(seed, workload_id, 10)
    rk = stream(seed, workload_id, 11)
    rv = stream(seed, workload_id, 12)
    cq = np.exp(sigma * stream(seed, workload_id, 13).standard_normal((Hq, dh))).astype(np.float32)
    ck = np.exp(sigma * stream(seed, workload_id, 14).standard_normal((Hkv, dh))).astype(np.float32)
    Q = bf16_round(normal(rq, (L, Hq, dh)) * cq[None])
    K = bf16_round(normal(rk, (L, Hkv, dh)) * ck[None])
    V = bf16_round(normal(rv, (L, Hkv, dh)))
    Kt = np.ascontiguousarray(K.transpose(1, 2, 0))
    return Q, Kt, V


def causal_probs(Q, Kt, scale: float, device=None, out=None):
    """Attention probabilities P[h] = causal-softmax(Q_h K_g(h)^T * scale), rounded to bf16.

    This builds the P operand of the P.V product the way a causal decoder layer
    produces it (rows sum to one, exact zeros above the diagonal).  It uses the
    dense logits; it is input preparation, not part of the reduction method.
    Kv head g(h) = h * Hkv // Hq (grouped-query attention).

    ``Q``/``Kt`` may be NumPy arrays or torch tensors; the work runs in torch on
    ``device`` (CPU by default) one head at a time and returns a torch bf16
    tensor [Hq][Lq][Lk] (written into ``out`` when given).
    """
    import torch

    dev = torch.device(device) if device is not None else torch.device("cpu")
    Qt = torch.as_tensor(Q).to(dev)
    Kt_t = torch.as_tensor(Kt).to(dev)
    Lq, Hq, dh = Qt.shape
    Hkv, _, Lk = Kt_t.shape
    if out is None:
        out = torch.empty((Hq, Lq, Lk), dtype=torch.bfloat16, device=dev)
    mask = torch.ones((Lq, Lk), dtype=torch.bool, device=dev).triu_(1 + (Lk - Lq))
    for h in range(Hq):
        g = h * Hkv // Hq
        q = Qt[:, h, :].to(torch.float32).contiguous()
        k = Kt_t[g].to(torch.float32).contiguous()
        s = torch.matmul(q, k) * scale
        s.masked_fill_(mask, float("-inf"))
        out[h].copy_(torch.softmax(s, dim=-1).to(torch.bfloat16))
    return out

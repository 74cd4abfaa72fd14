"""The five synthetic workloads, as shape/ratio registries plus operand builders.

Shapes follow the model families the pages evaluate (LLaMA 3.2-1B, LLaMA 3.1-8B,
LLaMA 3.1-70B) and the two application sites they name: linear/MLP
projections XW and the attention products QK^T and PV.  Every builder takes
optional size overrides so tests can draw the *same distributions* at sizes a
CPU oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import (attention_qkv, bf16_round, int8_per_column, lognormal_col_activations, normal,
                  outlier_activations, stream, weight)

__all__ = ["Linear", "Attention", "Workload", "WORKLOADS", "linear_operands", "linear_activation",
           "linear_weight", "linear_weight_int8", "activation_key", "attention_operands"]


@dataclass(frozen=True)
class Linear:
    """One reduced projection Y[m, n] = A[m, d] B[d, n] at retention ratio rho."""
    name: str
    m: int
    d: int
    n: int
    rho: float
    tensor_a: int       # tensor id of the activation stream
    tensor_b: int       # tensor id of the weight stream


@dataclass(frozen=True)
class Attention:
    """One attention layer: S = Q_I K_I^T per head (feature dim), O = P_J V_J (token dim)."""
    L: int
    Hq: int
    Hkv: int
    dh: int
    rho: float


@dataclass(frozen=True)
class Workload:
    wid: int
    key: str
    dtype: str                      # "f32" or "bf16"
    act: str                        # activation recipe: "lognormal1", "outlier"
    act_frac: float = 0.0
    act_factor: float = 1.0
    act_sigma: float = 1.0
    linears: tuple = field(default_factory=tuple)
    attention: Attention | None = None
    silu_down: bool = False         # down-projection input = silu(X Wg) * (X Wu)


def _layer(m, hidden, kv, mlp, rho_attn, rho_mlp):
    return (
        Linear("q", m, hidden, hidden, rho_attn, 20, 1),
        Linear("k", m, hidden, kv, rho_attn, 20, 2),
        Linear("v", m, hidden, kv, rho_attn, 20, 3),
        Linear("o", m, hidden, hidden, rho_attn, 21, 4),
        Linear("up", m, hidden, mlp, rho_mlp, 20, 5),
        Linear("gate", m, hidden, mlp, rho_mlp, 20, 6),
        Linear("down", m, mlp, hidden, rho_mlp, 22, 7),
    )


def _c2_linears():
    out = []
    for rho in (0.5, 0.7, 0.8):
        for lin in _layer(2048, 2048, 512, 8192, rho, rho):
            out.append(Linear(f"{lin.name}@{rho}", lin.m, lin.d, lin.n, rho, lin.tensor_a, lin.tensor_b))
    return tuple(out)


def _c5_linears():
    out = []
    for m in (8192, 16):
        for rho in (0.3, 0.5, 0.7, 0.8, 1.0):
            for lin in _layer(m, 8192, 1024, 28672, rho, rho):
                out.append(Linear(f"{lin.name}@m{m}@{rho}", m, lin.d, lin.n, rho, lin.tensor_a, lin.tensor_b))
    return tuple(out)


WORKLOADS = {
    # Single reduced XW in fp32: A 64x512 (N(0,1) x log-normal(0,1) column scale), W 512x512.
    "xw-fp32-64x512": Workload(1, "xw-fp32-64x512", "f32", "lognormal1",
                               linears=(Linear("xw", 64, 512, 512, 0.5, 20, 1),)),
    # LLaMA-3.2-1B-shaped projections, 2048 tokens.
    "llama3.2-1b-proj-2k": Workload(2, "llama3.2-1b-proj-2k", "bf16", "outlier", act_frac=0.01,
                                    act_factor=20.0, linears=_c2_linears(), silu_down=True),
    # One attention layer, 32 heads x 128, 4096 tokens.
    "attn-32h-4k": Workload(3, "attn-32h-4k", "bf16", "none",
                            attention=Attention(4096, 32, 32, 128, 0.5)),
    # LLaMA-3.1-8B-shaped layer at 16384 tokens; attention side 0.5, MLP 0.8.
    "llama3.1-8b-layer-16k": Workload(4, "llama3.1-8b-layer-16k", "bf16", "outlier", act_frac=0.005,
                                      act_factor=30.0,
                                      linears=_layer(16384, 4096, 1024, 14336, 0.5, 0.8),
                                      attention=Attention(16384, 32, 8, 128, 0.5)),
    # LLaMA-3.1-70B-shaped layer, prefill m=8192 and decode m=16, rho sweep.
    "llama3.1-70b-layer": Workload(5, "llama3.1-70b-layer", "bf16", "lognormal1", act_sigma=1.0,
                                   linears=_c5_linears(),
                                   attention=Attention(8192, 64, 8, 128, 0.5)),
}


def _activation(w: Workload, seed: int, tensor_id: int, m: int, d: int) -> np.ndarray:
    """Activation matrix; the column-level draws (outlier channels, column
    scales) use their own stream, so the first m' rows do not depend on m."""
    rng = stream(seed, w.wid, tensor_id * 100003 + d)
    col_rng = stream(seed, w.wid, tensor_id * 100003 + d + 50000)
    bf16 = w.dtype == "bf16"
    if w.act == "outlier":
        return outlier_activations(rng, m, d, w.act_frac, w.act_factor, bf16=bf16, col_rng=col_rng)
    if w.act == "lognormal1":
        return lognormal_col_activations(rng, m, d, w.act_sigma, bf16=bf16, col_rng=col_rng)
    a = normal(rng, (m, d))
    return bf16_round(a) if bf16 else a


def linear_weight(w: Workload, lin: Linear, seed: int = 0) -> np.ndarray:
    """B [d, n] of one projection (rows are the contraction index)."""
    return weight(stream(seed, w.wid, lin.tensor_b * 100003 + lin.d * 7 + lin.n), lin.d, lin.n,
                  bf16=w.dtype == "bf16")


def linear_weight_int8(w: Workload, lin: Linear, seed: int = 0):
    """(q int8 [d, n], scale float32 [n]): the projection's weight in per-column INT8 form."""
    return int8_per_column(linear_weight(w, lin, seed))


def activation_key(w: Workload, lin: Linear, m: int | None = None):
    """Projections with equal keys read the same activation matrix."""
    m = lin.m if m is None else m
    if lin.name.startswith("down") and w.silu_down:
        return ("silu", m, lin.d)
    return (lin.tensor_a, m, lin.d)


def linear_activation(w: Workload, lin: Linear, seed: int = 0, m: int | None = None) -> np.ndarray:
    """A [m, d] of one projection.  ``m`` overrides the token count (same
    distributions, fewer rows).  For the LLaMA-3.2-1B workload the
    down-projection input is the SiLU-gated MLP activation silu(X Wg) * (X Wu),
    formed in float32 from the workload's bf16 X, Wg and Wu, rounded to bf16."""
    m = lin.m if m is None else m
    if lin.name.startswith("down") and w.silu_down:
        hidden = lin.n
        X = _activation(w, seed, 20, m, hidden)
        Wu = weight(stream(seed, w.wid, 5 * 100003 + hidden * 7 + lin.d), hidden, lin.d)
        Wg = weight(stream(seed, w.wid, 6 * 100003 + hidden * 7 + lin.d), hidden, lin.d)
        g = X @ Wg
        u = X @ Wu
        return bf16_round((g / (1.0 + np.exp(-g))) * u)
    return _activation(w, seed, lin.tensor_a, m, lin.d)


def linear_operands(w: Workload, lin: Linear, seed: int = 0, m: int | None = None):
    """(A [m, d], B [d, n]) for one projection of workload ``w`` (float32 arrays)."""
    return linear_activation(w, lin, seed, m), linear_weight(w, lin, seed)


def attention_operands(w: Workload, seed: int = 0, L: int | None = None, Hq: int | None = None,
                       Hkv: int | None = None):
    """(Q [L][Hq][dh], Kt [Hkv][dh][L], V [L][Hkv][dh]) for workload ``w``'s attention layer."""
    at = w.attention
    L = at.L if L is None else L
    Hq = at.Hq if Hq is None else Hq
    Hkv = at.Hkv if Hkv is None else Hkv
    return attention_qkv(seed, w.wid, L, Hq, Hkv, at.dh)

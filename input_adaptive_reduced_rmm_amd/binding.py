"""ctypes binding of librmm.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module turns torch
tensors into pointers, strides and sizes, allocates outputs and workspace with
torch's device allocator, passes torch's current HIP stream, and raises
``RMMError`` with the library's message when a call is rejected.  The C
declarations and their contracts live in include/rmm.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RMMError", "load", "lib_path",
    "rmm_version", "rmm_k_from_rho", "rmm_k_pad",
    "rmm_colnorm", "rmm_topk", "rmm_gemm", "rmm_gemm_scored", "rmm_gemm_noalloc", "rmm_gemm_w8", "rmm_swiglu_scored", "rmm_rmsnorm_scored", "rmm_attention_decode_batch", "rmm_qk", "rmm_pv",
    "rmm_attention",
    "rmm_colnorm_workspace_bytes", "rmm_topk_workspace_bytes", "rmm_gemm_workspace_bytes",
    "rmm_qk_workspace_bytes", "rmm_pv_workspace_bytes", "rmm_attention_workspace_bytes",
    "rmm_gemm_w8_workspace_bytes", "rmm_swiglu_scored_workspace_bytes", "rmm_rmsnorm_scored_workspace_bytes",
    "rmm_attention_decode_batch_workspace_bytes",
    "rmm_linear", "timing",
]

RMM_BF16, RMM_F32 = 0, 1
RMM_OK, RMM_ERR_INVALID_ARG, RMM_ERR_UNSUPPORTED, RMM_ERR_WORKSPACE, RMM_ERR_HIP = 0, 1, 2, 3, 4
_STATUS = {0: "RMM_OK", 1: "RMM_ERR_INVALID_ARG", 2: "RMM_ERR_UNSUPPORTED", 3: "RMM_ERR_WORKSPACE",
           4: "RMM_ERR_HIP"}

_here = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_here, "librmm.so")
_lib = None


class RMMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_i64, _f64, _sz, _vp = ctypes.c_int64, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p
_PROTOS = {
    "rmm_version": (ctypes.c_int, []),
    "rmm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rmm_last_error": (ctypes.c_char_p, []),
    "rmm_k_from_rho": (ctypes.c_int, [_f64, _i64, ctypes.POINTER(_i64)]),
    "rmm_k_pad": (_i64, [_i64]),
    "rmm_colnorm_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64]),
    "rmm_colnorm": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "rmm_topk_workspace_bytes": (_sz, [_i64, _i64]),
    "rmm_topk": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "rmm_gemm_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64]),
    "rmm_gemm": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp,
                                _i64, _vp, _sz, _vp]),
    "rmm_qk_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "rmm_qk": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                              ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "rmm_pv_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "rmm_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "rmm_timing_set_tag": (ctypes.c_int, [ctypes.c_char_p]),
    "rmm_timing_collect": (ctypes.c_int, []),
    "rmm_timing_count": (ctypes.c_int, []),
    "rmm_timing_entry": (ctypes.c_int, [ctypes.c_int, ctypes.c_char_p, _sz, ctypes.POINTER(_f64),
                                        ctypes.POINTER(_i64)]),
    "rmm_timing_reset": (ctypes.c_int, []),
    "rmm_pv": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                              ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
    "rmm_attention_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "rmm_gemm_w8_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "rmm_swiglu_scored_workspace_bytes": (_sz, [_i64, _i64]),
    "rmm_swiglu_scored": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "rmm_rmsnorm_scored_workspace_bytes": (_sz, [_i64, _i64]),
    "rmm_attention_decode_batch_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "rmm_attention_decode_batch": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                                  _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _i64,
                                                  _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "rmm_rmsnorm_scored": (ctypes.c_int, [_vp, _i64, _vp, ctypes.c_float, _i64, _i64, _vp, _i64, _vp, _vp, _sz,
                                          _vp]),
    "rmm_gemm_scored_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64]),
    "rmm_gemm_scored": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _i64,
                                       _vp, _vp, _sz, _vp]),
    "rmm_gemm_noalloc": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp,
                                        _i64, _vp]),
    "rmm_gemm_w8": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _sz,
                                   _vp]),
    "rmm_attention": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _vp,
                                     _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp,
                                     _vp, _vp, _sz, _vp]),
}


def load():
    """Load librmm.so (built in-tree by __graft_entry__.build()); raise loudly if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"RMM HIP library not built: {lib_path} is missing "
                          "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
    lib = ctypes.CDLL(lib_path)
    for name, (res, args) in _PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise RMMError(status, load().rmm_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RMM_BF16
    if t.dtype == torch.float32:
        return RMM_F32
    raise TypeError(f"unsupported dtype {t.dtype}; RMM takes bfloat16 or float32")


def _dev(*ts: torch.Tensor):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("RMM operands must live on a HIP device")
    for t in ts:
        if t.device != dev:
            raise ValueError("RMM operands must share one device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes: int, dev, ws: torch.Tensor | None):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: need {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ------------------------------------------------------------------ scalars
def rmm_version() -> int:
    return load().rmm_version()


def rmm_k_from_rho(rho: float, d: int) -> int:
    k = _i64(0)
    _check(load().rmm_k_from_rho(float(rho), int(d), ctypes.byref(k)))
    return int(k.value)


def rmm_k_pad(k: int) -> int:
    return int(load().rmm_k_pad(int(k)))


def rmm_colnorm_workspace_bytes(dtype: torch.dtype, m: int, d: int, batch: int = 1) -> int:
    dt = RMM_BF16 if dtype == torch.bfloat16 else RMM_F32
    return int(load().rmm_colnorm_workspace_bytes(dt, m, d, batch))


def rmm_topk_workspace_bytes(batch: int, d: int) -> int:
    return int(load().rmm_topk_workspace_bytes(batch, d))


def rmm_gemm_workspace_bytes(dtype: torch.dtype, m: int, n: int, k: int) -> int:
    dt = RMM_BF16 if dtype == torch.bfloat16 else RMM_F32
    return int(load().rmm_gemm_workspace_bytes(dt, m, n, k))


def rmm_qk_workspace_bytes(Lq: int, Hq: int, dh: int, k: int) -> int:
    return int(load().rmm_qk_workspace_bytes(Lq, Hq, dh, k))


def rmm_pv_workspace_bytes(Hq: int, Lq: int, Lk: int, k: int) -> int:
    return int(load().rmm_pv_workspace_bytes(Hq, Lq, Lk, k))


# ------------------------------------------------------------------ entry points
def rmm_colnorm(A: torch.Tensor, out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Column scores of A [m, d] -> float32 [d], or of A [batch, m, d] -> [batch, d].

    The last dimension must have unit stride; other strides are passed through.
    """
    lib = load()
    dev = _dev(A)
    squeeze = A.dim() == 2
    A3 = A.unsqueeze(0) if squeeze else A
    if A3.dim() != 3 or A3.stride(2) != 1:
        raise ValueError("A must be [m, d] or [batch, m, d] with unit column stride")
    batch, m, d = A3.shape
    if out is None:
        out = torch.empty((batch, d), dtype=torch.float32, device=dev)
    dt = _dt(A)
    ws, wsb = _ws(int(lib.rmm_colnorm_workspace_bytes(dt, m, d, batch)), dev, ws)
    _check(lib.rmm_colnorm(dt, _ptr(A3), m, d, A3.stride(1), batch, A3.stride(0), _ptr(out), _ptr(ws), wsb,
                           _stream(dev)))
    return out[0] if squeeze else out


def rmm_topk(scores: torch.Tensor, k: int, out: torch.Tensor | None = None):
    """Top-k indices of scores [d] or [batch, d] -> int32 [k_pad] or [batch, k_pad]
    (kept indices ascending, then -1)."""
    lib = load()
    dev = _dev(scores)
    squeeze = scores.dim() == 1
    s2 = scores.unsqueeze(0) if squeeze else scores
    if s2.dtype != torch.float32 or not s2.is_contiguous():
        raise ValueError("scores must be contiguous float32")
    batch, d = s2.shape
    kp = rmm_k_pad(k)
    if out is None:
        out = torch.empty((batch, max(kp, 1)), dtype=torch.int32, device=dev)
    _check(lib.rmm_topk(_ptr(s2), batch, d, int(k), _ptr(out), None, 0, _stream(dev)))
    return out[0] if squeeze else out


def rmm_gemm_scored(A: torch.Tensor, B: torch.Tensor, idx: torch.Tensor, k: int, out: torch.Tensor | None = None,
                    scores: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Y = A[:, idx[:k]] @ B[idx[:k], :] and the column scores of Y -> (Y [m, n], scores float32 [n])."""
    lib = load()
    dev = _dev(A, B, idx)
    if A.dim() != 2 or B.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A [m, d] and B [d, n] must be 2-D with unit column stride")
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    m, d = A.shape
    d2, n = B.shape
    if d2 != d:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=A.dtype, device=dev)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=dev)
    dt = _dt(A)
    ws, wsb = _ws(int(lib.rmm_gemm_scored_workspace_bytes(dt, m, n, int(k))), dev, ws)
    _check(lib.rmm_gemm_scored(dt, _ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(idx), m, d, n, int(k),
                               _ptr(out), out.stride(0), _scores_ptr(scores, (n,), dev), _ptr(ws), wsb, _stream(dev)))
    return out, scores


def rmm_gemm_noalloc(A: torch.Tensor, B: torch.Tensor, idx: torch.Tensor, k: int, out: torch.Tensor):
    """rmm_gemm with the library's fixed scratch array instead of a workspace:
    Y = A[:, idx[:k]] @ B[idx[:k], :] written into `out` [m, n]; allocates nothing."""
    lib = load()
    dev = _dev(A, B, idx, out)
    if A.dim() != 2 or B.dim() != 2 or out.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("A [m, d], B [d, n] and out [m, n] must be 2-D with unit column stride")
    if A.dtype != B.dtype or out.dtype != A.dtype:
        raise TypeError("A, B and out must share a dtype")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    m, d = A.shape
    d2, n = B.shape
    if d2 != d or tuple(out.shape) != (m, n):
        raise ValueError("shapes of A, B and out disagree")
    _check(lib.rmm_gemm_noalloc(_dt(A), _ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(idx), m, d, n, int(k),
                                _ptr(out), out.stride(0), _stream(dev)))
    return out


def rmm_gemm(A: torch.Tensor, B: torch.Tensor, idx: torch.Tensor, k: int, out: torch.Tensor | None = None,
             ws: torch.Tensor | None = None):
    """Y = A[:, idx[:k]] @ B[idx[:k], :] for A [m, d], B [d, n] (same dtype)."""
    lib = load()
    dev = _dev(A, B, idx)
    if A.dim() != 2 or B.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A [m, d] and B [d, n] must be 2-D with unit column stride")
    if A.dtype != B.dtype:
        raise TypeError("A and B must share a dtype")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    m, d = A.shape
    d2, n = B.shape
    if d2 != d:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((m, n), dtype=A.dtype, device=dev)
    dt = _dt(A)
    ws, wsb = _ws(int(lib.rmm_gemm_workspace_bytes(dt, m, n, int(k))), dev, ws)
    _check(lib.rmm_gemm(dt, _ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(idx), m, d, n, int(k), _ptr(out),
                        out.stride(0), _ptr(ws), wsb, _stream(dev)))
    return out


def rmm_gemm_w8_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load().rmm_gemm_w8_workspace_bytes(m, n, k))


def rmm_gemm_w8(A: torch.Tensor, Bq: torch.Tensor, scale: torch.Tensor, idx: torch.Tensor, k: int,
                out: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Y = A[:, idx[:k]] @ (Bq[idx[:k], :] * scale) for bf16 A [m, d], int8 Bq [d, n], float32 scale [n]."""
    lib = load()
    dev = _dev(A, Bq, scale, idx)
    if A.dtype != torch.bfloat16 or Bq.dtype != torch.int8 or scale.dtype != torch.float32:
        raise TypeError("rmm_gemm_w8 takes bfloat16 A, int8 Bq and float32 scale")
    if A.dim() != 2 or Bq.dim() != 2 or A.stride(1) != 1 or Bq.stride(1) != 1 or not scale.is_contiguous():
        raise ValueError("A [m, d] and Bq [d, n] must be 2-D with unit column stride, scale contiguous")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    m, d = A.shape
    d2, n = Bq.shape
    if d2 != d or scale.numel() != n:
        raise ValueError("shapes of A, Bq and scale disagree")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws, wsb = _ws(rmm_gemm_w8_workspace_bytes(m, n, int(k)), dev, ws)
    _check(lib.rmm_gemm_w8(_ptr(A), A.stride(0), _ptr(Bq), Bq.stride(0), _ptr(scale), _ptr(idx), m, d, n, int(k),
                           _ptr(out), out.stride(0), _ptr(ws), wsb, _stream(dev)))
    return out


def rmm_swiglu_scored_workspace_bytes(m: int, n: int) -> int:
    return int(load().rmm_swiglu_scored_workspace_bytes(m, n))


def rmm_swiglu_scored(G: torch.Tensor, U: torch.Tensor, H: torch.Tensor | None = None,
                      scores: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """H = silu(G) * U (bf16 [m, n]) and the column scores of H (float32 [n]) in one pass."""
    lib = load()
    dev = _dev(G, U)
    if G.dtype != torch.bfloat16 or U.dtype != torch.bfloat16:
        raise TypeError("rmm_swiglu_scored takes bfloat16 G and U")
    if G.dim() != 2 or G.shape != U.shape or G.stride(1) != 1 or U.stride(1) != 1:
        raise ValueError("G and U must be [m, n] with unit column stride")
    m, n = G.shape
    if H is None:
        H = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=dev)
    ws, wsb = _ws(rmm_swiglu_scored_workspace_bytes(m, n), dev, ws)
    _check(lib.rmm_swiglu_scored(_ptr(G), G.stride(0), _ptr(U), U.stride(0), m, n, _ptr(H), H.stride(0),
                                 _ptr(scores), _ptr(ws), wsb, _stream(dev)))
    return H, scores


def rmm_rmsnorm_scored_workspace_bytes(m: int, d: int) -> int:
    return int(load().rmm_rmsnorm_scored_workspace_bytes(m, d))


def rmm_rmsnorm_scored(X: torch.Tensor, w: torch.Tensor, eps: float = 1e-5, Y: torch.Tensor | None = None,
                       scores: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Y = X * w / sqrt(mean(X^2, row) + eps) (bf16 [m, d]) and the column scores of Y (float32 [d])."""
    lib = load()
    dev = _dev(X, w)
    if X.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("rmm_rmsnorm_scored takes bfloat16 X and w")
    if X.dim() != 2 or X.stride(1) != 1 or w.dim() != 1 or w.shape[0] != X.shape[1] or w.stride(0) != 1:
        raise ValueError("X must be [m, d] with unit column stride and w contiguous [d]")
    m, d = X.shape
    if Y is None:
        Y = torch.empty((m, d), dtype=torch.bfloat16, device=dev)
    if scores is None:
        scores = torch.empty(d, dtype=torch.float32, device=dev)
    ws, wsb = _ws(rmm_rmsnorm_scored_workspace_bytes(m, d), dev, ws)
    _check(lib.rmm_rmsnorm_scored(_ptr(X), X.stride(0), _ptr(w), float(eps), m, d, _ptr(Y), Y.stride(0),
                                  _ptr(scores), _ptr(ws), wsb, _stream(dev)))
    return Y, scores


def _scores_ptr(t: torch.Tensor | None, shape, dev):
    """Pointer of an optional float32 score output of the given shape (None: NULL)."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape) or t.device != dev:
        raise ValueError(f"scores must be contiguous float32 {tuple(shape)} on {dev}")
    return _ptr(t)


def rmm_qk(Q: torch.Tensor, Kt: torch.Tensor, k: int, S: torch.Tensor | None = None,
           idx: torch.Tensor | None = None, ws: torch.Tensor | None = None, causal: bool = False,
           feat_scores: torch.Tensor | None = None):
    """Feature-reduced scores. Q [Lq, Hq, dh], Kt [Hkv, dh, Lk] (bf16) ->
    (S float32 [Hq, Lq, Lk], idx int32 [Hq, k_pad]).  causal=True leaves tiles
    above the causal diagonal unwritten.  feat_scores (optional float32 [Hq, dh])
    receives the column scores the selection used."""
    lib = load()
    dev = _dev(Q, Kt)
    if Q.dtype != torch.bfloat16 or Kt.dtype != torch.bfloat16:
        raise TypeError("rmm_qk takes bfloat16 Q and Kt")
    if Q.dim() != 3 or Kt.dim() != 3 or Q.stride(2) != 1 or Kt.stride(2) != 1:
        raise ValueError("Q [Lq, Hq, dh] and Kt [Hkv, dh, Lk] need unit innermost stride")
    Lq, Hq, dh = Q.shape
    Hkv, dh2, Lk = Kt.shape
    if dh2 != dh:
        raise ValueError("head dims differ")
    kp = rmm_k_pad(k)
    if S is None:
        S = torch.empty((Hq, Lq, Lk), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((Hq, kp), dtype=torch.int32, device=dev)
    ws, wsb = _ws(int(lib.rmm_qk_workspace_bytes(Lq, Hq, dh, int(k))), dev, ws)
    _check(lib.rmm_qk(_ptr(Q), Lq, Hq, dh, Q.stride(0), Q.stride(1), _ptr(Kt), Lk, Hkv, Kt.stride(0),
                      Kt.stride(1), int(k), 1 if causal else 0, _ptr(S), S.stride(0), S.stride(1), _ptr(idx),
                      _scores_ptr(feat_scores, (Hq, dh), dev), _ptr(ws), wsb, _stream(dev)))
    return S, idx


def rmm_pv(P: torch.Tensor, V: torch.Tensor, k: int, O: torch.Tensor | None = None,
           idx: torch.Tensor | None = None, ws: torch.Tensor | None = None, causal: bool = False,
           tok_scores: torch.Tensor | None = None):
    """Token-reduced output. P [Hq, Lq, Lk], V [Lk, Hkv, dh] (bf16) ->
    (O bf16 [Lq, Hq, dh], idx int32 [Hq, k_pad]).  causal=True: P above the
    causal diagonal is taken as zero and never read.  tok_scores (optional
    float32 [Hq, Lk]) receives the token scores the selection used."""
    lib = load()
    dev = _dev(P, V)
    if P.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise TypeError("rmm_pv takes bfloat16 P and V")
    if P.dim() != 3 or V.dim() != 3 or P.stride(2) != 1 or V.stride(2) != 1:
        raise ValueError("P [Hq, Lq, Lk] and V [Lk, Hkv, dh] need unit innermost stride")
    Hq, Lq, Lk = P.shape
    Lk2, Hkv, dh = V.shape
    if Lk2 != Lk:
        raise ValueError("token counts differ")
    kp = rmm_k_pad(k)
    if O is None:
        O = torch.empty((Lq, Hq, dh), dtype=torch.bfloat16, device=dev)
    if idx is None:
        idx = torch.empty((Hq, kp), dtype=torch.int32, device=dev)
    ws, wsb = _ws(int(lib.rmm_pv_workspace_bytes(Hq, Lq, Lk, int(k))), dev, ws)
    _check(lib.rmm_pv(_ptr(P), Hq, Lq, Lk, P.stride(0), P.stride(1), _ptr(V), Hkv, dh, V.stride(0),
                      V.stride(1), int(k), 1 if causal else 0, _ptr(O), O.stride(0), O.stride(1), _ptr(idx),
                      _scores_ptr(tok_scores, (Hq, Lk), dev), _ptr(ws), wsb, _stream(dev)))
    return O, idx


def rmm_attention_workspace_bytes(Lq: int, Lk: int, Hq: int, dh: int, k_feat: int, k_tok: int) -> int:
    return int(load().rmm_attention_workspace_bytes(Lq, Lk, Hq, dh, k_feat, k_tok))


def rmm_attention(Q: torch.Tensor, Kt: torch.Tensor, V: torch.Tensor, k_feat: int, k_tok: int,
                  O: torch.Tensor | None = None, idx_feat: torch.Tensor | None = None,
                  idx_tok: torch.Tensor | None = None, tok_scores: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None, causal: bool = True, o_scores: torch.Tensor | None = None):
    """Fused reduced attention.  Q [Lq, Hq, dh], Kt [Hkv, dh, Lk], V [Lk, Hkv, dh] (bf16)
    -> (O bf16 [Lq, Hq, dh], idx_feat int32 [Hq, k_pad(k_feat)], idx_tok int32 [Hq, k_pad(k_tok)]).
    tok_scores (optional float32 [Hq, Lk]) receives the token scores; o_scores (optional
    float32 [Hq, dh]) the column scores of O for the projection that reads it."""
    lib = load()
    dev = _dev(Q, Kt, V)
    if Q.dtype != torch.bfloat16 or Kt.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise TypeError("rmm_attention takes bfloat16 Q, Kt and V")
    if Q.dim() != 3 or Kt.dim() != 3 or V.dim() != 3 or Q.stride(2) != 1 or Kt.stride(2) != 1 or V.stride(2) != 1:
        raise ValueError("Q [Lq, Hq, dh], Kt [Hkv, dh, Lk], V [Lk, Hkv, dh] need unit innermost stride")
    Lq, Hq, dh = Q.shape
    Hkv, dh2, Lk = Kt.shape
    if dh2 != dh or V.shape[0] != Lk or V.shape[1] != Hkv or V.shape[2] != dh:
        raise ValueError("shapes of Q, Kt and V disagree")
    if O is None:
        O = torch.empty((Lq, Hq, dh), dtype=torch.bfloat16, device=dev)
    if idx_feat is None:
        idx_feat = torch.empty((Hq, rmm_k_pad(k_feat)), dtype=torch.int32, device=dev)
    if idx_tok is None:
        idx_tok = torch.empty((Hq, rmm_k_pad(k_tok)), dtype=torch.int32, device=dev)
    ws, wsb = _ws(int(lib.rmm_attention_workspace_bytes(Lq, Lk, Hq, dh, int(k_feat), int(k_tok))), dev, ws)
    _check(lib.rmm_attention(_ptr(Q), Lq, Hq, dh, Q.stride(0), Q.stride(1), _ptr(Kt), Lk, Hkv, Kt.stride(0),
                             Kt.stride(1), _ptr(V), V.stride(0), V.stride(1), int(k_feat), int(k_tok),
                             1 if causal else 0, _ptr(O), O.stride(0), O.stride(1), _ptr(idx_feat),
                             _ptr(idx_tok), _ptr(tok_scores), _ptr(o_scores), _ptr(ws), wsb, _stream(dev)))
    return O, idx_feat, idx_tok


def rmm_attention_decode_batch_workspace_bytes(nseq: int, Hq: int, dh: int, Lmax: int, kt_max: int) -> int:
    return int(load().rmm_attention_decode_batch_workspace_bytes(nseq, Hq, dh, Lmax, kt_max))


def rmm_attention_decode_batch(Q: torch.Tensor, Kt: torch.Tensor, V: torch.Tensor, lens: torch.Tensor,
                               k_tok: torch.Tensor, k_feat: int, kt_max: int | None = None,
                               O: torch.Tensor | None = None, idx_feat: torch.Tensor | None = None,
                               idx_tok: torch.Tensor | None = None, tok_scores: torch.Tensor | None = None,
                               ws: torch.Tensor | None = None):
    """One decode step of B sequences.  Q [B, Hq, dh] (one new token each), Kt [B, Hkv, dh, Lmax],
    V [B, Lmax, Hkv, dh] (bf16), lens and k_tok int32 [B] on the device ->
    (O bf16 [B, Hq, dh], idx_feat int32 [B*Hq, k_pad(k_feat)], idx_tok int32 [B*Hq, k_pad(kt_max)])."""
    lib = load()
    dev = _dev(Q, Kt, V, lens, k_tok)
    if Q.dtype != torch.bfloat16 or Kt.dtype != torch.bfloat16 or V.dtype != torch.bfloat16:
        raise TypeError("rmm_attention_decode_batch takes bfloat16 Q, Kt and V")
    if lens.dtype != torch.int32 or k_tok.dtype != torch.int32 or not lens.is_contiguous() or not k_tok.is_contiguous():
        raise TypeError("lens and k_tok must be contiguous int32 device tensors")
    if Q.dim() != 3 or Kt.dim() != 4 or V.dim() != 4 or Q.stride(2) != 1 or Kt.stride(3) != 1 or V.stride(3) != 1:
        raise ValueError("Q [B, Hq, dh], Kt [B, Hkv, dh, Lmax], V [B, Lmax, Hkv, dh] with unit innermost stride")
    B, Hq, dh = Q.shape
    Hkv, Lmax = Kt.shape[1], Kt.shape[3]
    if Kt.shape[0] != B or Kt.shape[2] != dh or V.shape[0] != B or V.shape[1] != Lmax or V.shape[2] != Hkv \
            or V.shape[3] != dh or lens.numel() != B or k_tok.numel() != B:
        raise ValueError("inconsistent shapes")
    kt_max = Lmax if kt_max is None else int(kt_max)
    if O is None:
        O = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device=dev)
    if idx_feat is None:
        idx_feat = torch.empty((B * Hq, rmm_k_pad(k_feat)), dtype=torch.int32, device=dev)
    if idx_tok is None:
        idx_tok = torch.empty((B * Hq, rmm_k_pad(kt_max)), dtype=torch.int32, device=dev)
    ws, wsb = _ws(rmm_attention_decode_batch_workspace_bytes(B, Hq, dh, Lmax, kt_max), dev, ws)
    _check(lib.rmm_attention_decode_batch(
        _ptr(Q), Q.stride(0), Q.stride(1), _ptr(Kt), Kt.stride(0), Kt.stride(1), Kt.stride(2),
        _ptr(V), V.stride(0), V.stride(1), V.stride(2), _ptr(lens), _ptr(k_tok), B, Hq, Hkv, dh, Lmax,
        int(k_feat), kt_max, _ptr(O), O.stride(0), O.stride(1), _ptr(idx_feat), _ptr(idx_tok),
        _ptr(tok_scores) if tok_scores is not None else None, _ptr(ws), wsb, _stream(dev)))
    return O, idx_feat, idx_tok


def rmm_linear(A: torch.Tensor, B: torch.Tensor, rho: float):
    """Whole reduced projection: scores -> top-k -> reduced GEMM. Returns (Y, idx, scores, k)."""
    k = rmm_k_from_rho(rho, A.shape[1])
    s = rmm_colnorm(A)
    idx = rmm_topk(s, k)
    return rmm_gemm(A, B, idx, k), idx, s, k


class timing:
    """Per-kernel HIP-event timing inside the library (see rmm_timing_* in rmm.h)."""

    @staticmethod
    def enable(on: bool = True):
        _check(load().rmm_timing_enable(1 if on else 0))

    @staticmethod
    def tag(name: str | None):
        _check(load().rmm_timing_set_tag(name.encode() if name else None))

    @staticmethod
    def reset():
        _check(load().rmm_timing_reset())

    @staticmethod
    def collect() -> dict:
        """Wait for recorded launches; return {"tag/kernel": (total_ms, launches)}."""
        lib = load()
        _check(lib.rmm_timing_collect())
        out = {}
        buf = ctypes.create_string_buffer(256)
        for i in range(lib.rmm_timing_count()):
            ms, n = _f64(0.0), _i64(0)
            _check(lib.rmm_timing_entry(i, buf, 256, ctypes.byref(ms), ctypes.byref(n)))
            out[buf.value.decode()] = (ms.value, n.value)
        return out

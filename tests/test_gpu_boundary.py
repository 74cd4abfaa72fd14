"""The C ABI's error contract on the device: a rejected call enqueues nothing.

Each call below is valid except for one layout the kernels cannot address, and
passes a workspace of the queried size, so the rejection comes from the check
that sits latest in the entry point.  Outputs and index lists are poisoned
before the call; after a device synchronisation they must hold the poison
bit for bit.
"""
import ctypes

import pytest
import torch

from input_adaptive_reduced_rmm_amd import binding as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
POISON_I32 = 0x5A5A5A5A


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_rejected_qk_leaves_outputs_untouched():
    lib = R.load()
    Lq = Lk = 256
    Hq, Hkv, dh, k = 4, 2, 128, 64
    Q = torch.randn(Lq, Hq, dh, device=DEV).to(torch.bfloat16)
    Kt = torch.randn(Hkv, dh, Lk, device=DEV).to(torch.bfloat16)   # small; the claimed ldkt is never read
    ldkt = 1 << 25            # 127 feature rows of one key head span more than 4 GiB
    S = torch.full((Hq, Lq, Lk), float("nan"), device=DEV)
    kp = lib.rmm_k_pad(k)
    idx = torch.full((Hq, kp), POISON_I32, dtype=torch.int32, device=DEV)
    need = lib.rmm_qk_workspace_bytes(Lq, Hq, dh, k)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    S0, idx0 = S.clone(), idx.clone()
    torch.cuda.synchronize()
    for causal in (0, 1):
        st = lib.rmm_qk(_p(Q), Lq, Hq, dh, Hq * dh, dh, _p(Kt), Lk, Hkv, dh * ldkt, ldkt, k, causal, _p(S),
                        Lq * Lk, Lk, _p(idx), None, _p(ws), need, _stream())
        assert st == R.RMM_ERR_UNSUPPORTED, lib.rmm_last_error()
        assert b"4 GiB" in lib.rmm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0)
    assert torch.equal(S.view(torch.int32), S0.view(torch.int32))


def test_rejected_pv_leaves_outputs_untouched():
    lib = R.load()
    Lq = Lk = 256
    Hq, Hkv, dh, k = 4, 2, 128, 128
    P = torch.rand(Hq, Lq, Lk, device=DEV).to(torch.bfloat16)
    V = torch.randn(Lk, Hkv, dh, device=DEV).to(torch.bfloat16)
    ldp = 1 << 24             # 256 rows of P span more than 4 GiB
    O = torch.full((Lq, Hq, dh), float("nan"), device=DEV).to(torch.bfloat16)
    kp = lib.rmm_k_pad(k)
    idx = torch.full((Hq, kp), POISON_I32, dtype=torch.int32, device=DEV)
    need = lib.rmm_pv_workspace_bytes(Hq, Lq, Lk, k)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    O0, idx0 = O.clone(), idx.clone()
    torch.cuda.synchronize()
    st = lib.rmm_pv(_p(P), Hq, Lq, Lk, Lq * ldp, ldp, _p(V), Hkv, dh, Hkv * dh, dh, k, 1, _p(O), Hq * dh, dh,
                    _p(idx), None, _p(ws), need, _stream())
    assert st == R.RMM_ERR_UNSUPPORTED, lib.rmm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0)
    assert torch.equal(O.view(torch.int16), O0.view(torch.int16))


def test_rejected_attention_leaves_outputs_untouched():
    lib = R.load()
    Lq = Lk = 256
    Hq, Hkv, dh, kf, kt = 4, 2, 128, 64, 128
    Q = torch.randn(Lq, Hq, dh, device=DEV).to(torch.bfloat16)
    Kt = torch.randn(Hkv, dh, Lk, device=DEV).to(torch.bfloat16)
    V = torch.randn(Lk, Hkv, dh, device=DEV).to(torch.bfloat16)
    ldkt = 1 << 25            # the feature rows of one key head span more than 4 GiB
    O = torch.full((Lq, Hq, dh), float("nan"), device=DEV).to(torch.bfloat16)
    If = torch.full((Hq, lib.rmm_k_pad(kf)), POISON_I32, dtype=torch.int32, device=DEV)
    It = torch.full((Hq, lib.rmm_k_pad(kt)), POISON_I32, dtype=torch.int32, device=DEV)
    need = lib.rmm_attention_workspace_bytes(Lq, Lk, Hq, dh, kf, kt)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    O0, If0, It0 = O.clone(), If.clone(), It.clone()
    torch.cuda.synchronize()
    st = lib.rmm_attention(_p(Q), Lq, Hq, dh, Hq * dh, dh, _p(Kt), Lk, Hkv, dh * ldkt, ldkt, _p(V), Hkv * dh, dh,
                           kf, kt, 1, _p(O), Hq * dh, dh, _p(If), _p(It), None, None, _p(ws), need, _stream())
    assert st == R.RMM_ERR_UNSUPPORTED, lib.rmm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(If, If0) and torch.equal(It, It0)
    assert torch.equal(O.view(torch.int16), O0.view(torch.int16))


def test_rejected_gemm_w8_leaves_output_untouched():
    lib = R.load()
    m, d, n, k = 16, 256, 200, 100
    A = torch.randn(m, d, device=DEV).to(torch.bfloat16)
    Bq = torch.zeros(d, 208, dtype=torch.int8, device=DEV)
    ldb = 204                 # few-row int8 rows must be 16-byte aligned
    scale = torch.ones(n, device=DEV)
    idx = torch.arange(k, dtype=torch.int32, device=DEV)
    Y = torch.full((m, n), float("nan"), device=DEV).to(torch.bfloat16)
    need = lib.rmm_gemm_w8_workspace_bytes(m, n, k)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    Y0 = Y.clone()
    torch.cuda.synchronize()
    st = lib.rmm_gemm_w8(_p(A), d, _p(Bq), ldb, _p(scale), _p(idx), m, d, n, k, _p(Y), n, _p(ws), need, _stream())
    assert st == R.RMM_ERR_UNSUPPORTED, lib.rmm_last_error()
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y0.view(torch.int16))

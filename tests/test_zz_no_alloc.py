"""rmm_gemm_noalloc (the reduced product with the library's fixed scratch array
instead of a workspace) against rmm_gemm, called through the C ABI.

Two calls in a row on one device, the second with a smaller product, each
compared bit for bit with rmm_gemm on the same operands (the two entry points
run the same kernels, so the outputs are identical); the first call's scratch
contents must not leak into the second.  The products cover the few-row
kernel (m <= 32), the row-gather core and the persistent NT kernel.  A product
whose scratch exceeds the array is rejected before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from input_adaptive_reduced_rmm_amd import binding as R
from _parity import TOL_BF16, dev_tensor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _operands(m, d, n, seed):
    rng = synth.stream(0, 77, seed)
    A = synth.outlier_activations(rng, m, d, 0.01, 20.0)
    B = synth.weight(synth.stream(0, 77, seed + 100), d, n)
    return A, B


def _pair(m, d, n, rho, seed):
    A, B = _operands(m, d, n, seed)
    Ad, Bd = dev_tensor(A, torch.bfloat16), dev_tensor(B, torch.bfloat16)
    k = R.rmm_k_from_rho(rho, d)
    idx = R.rmm_topk(R.rmm_colnorm(Ad), k)
    Y_ws = R.rmm_gemm(Ad, Bd, idx, k)
    Y_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    R.rmm_gemm_noalloc(Ad, Bd, idx, k, Y_na)
    torch.cuda.synchronize()
    I = idx.cpu().numpy()[:k]
    return A, B, I, Y_ws, Y_na


@pytest.mark.parametrize("first,second", [
    ((32, 2048, 3072, 0.5), (16, 1024, 512, 0.7)),        # few-row kernel, then a smaller one
    ((2048, 2048, 6144, 0.5), (512, 1536, 1024, 0.8)),    # NT kernel (m >= 1024, 192 tiles), then the row-gather core
    ((600, 1000, 700, 0.3), (40, 512, 300, 0.5)),         # ragged row-gather core, then a ragged small one
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for j, (m, d, n, rho) in enumerate((first, second)):
        print(f"  noalloc call {j}: m={m} d={d} n={n} rho={rho}", flush=True)
        A, B, I, Y_ws, Y_na = _pair(m, d, n, rho, seed=10 * j + m % 7)
        assert torch.equal(Y_na.view(torch.int16), Y_ws.view(torch.int16)), (m, d, n, rho)
        err = rel_fro(Y_na.float().cpu().numpy(), oracle.reduced_product(A, B, I))
        assert err < TOL_BF16, err


def test_noalloc_rejects_products_beyond_the_array():
    lib = R.load()
    m, d, n, k = 16384, 4096, 28672, 3277        # needs far more than the fixed array
    assert lib.rmm_gemm_workspace_bytes(0, m, n, k) > (64 << 20)
    Y = torch.full((4, 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros((4, 4), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(4, dtype=torch.int32, device=DEV)
    # the huge shape is rejected on the host before any pointer is read
    st = lib.rmm_gemm_noalloc(0, ctypes.c_void_p(A.data_ptr()), d, ctypes.c_void_p(A.data_ptr()), n,
                              ctypes.c_void_p(idx.data_ptr()), m, d, n, k, ctypes.c_void_p(Y.data_ptr()), n,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == R.RMM_ERR_UNSUPPORTED
    assert b"scratch" in lib.rmm_last_error()
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all()


def test_noalloc_f32_path():
    m, d, n = 64, 512, 512
    rng = synth.stream(0, 78, 1)
    A = rng.standard_normal((m, d)).astype(np.float32)
    B = rng.standard_normal((d, n)).astype(np.float32) / np.sqrt(d)
    Ad, Bd = dev_tensor(A, torch.float32), dev_tensor(B, torch.float32)
    k = R.rmm_k_from_rho(0.5, d)
    idx = R.rmm_topk(R.rmm_colnorm(Ad), k)
    Y_ws = R.rmm_gemm(Ad, Bd, idx, k)
    Y_na = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    R.rmm_gemm_noalloc(Ad, Bd, idx, k, Y_na)
    torch.cuda.synchronize()
    assert torch.equal(Y_na.view(torch.int32), Y_ws.view(torch.int32))

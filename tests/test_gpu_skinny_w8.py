"""Few-row (decode) reduced GEMM and the INT8-weight reduced GEMM against the oracle.

`rmm_gemm` with m <= 32 and 16-byte aligned bf16 weight rows runs the split-K
few-row kernel; `rmm_gemm_w8` multiplies by INT8 weights with one float scale
per output column (the few-row kernel for m <= 32, dequantized kept rows and
the bf16 GEMM for more rows).  Products are compared with the float64 oracle
by relative Frobenius error (bf16 bound 1e-2); the INT8 reference is
A[:, I] (q[I, :] * scale) with the weight taken exactly as q * scale.
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


def _acts(m, d, seed):
    return synth.lognormal_col_activations(synth.stream(seed, 78, 1), m, d, 1.0, bf16=True)


def _weight(d, n, seed):
    return synth.weight(synth.stream(seed, 78, 2), d, n)


def _indices(d, k, seed, sort=True):
    rng = np.random.default_rng(seed)
    I = rng.choice(d, size=k, replace=False).astype(np.int32)
    return np.sort(I) if sort else I


# (m, d, n, k): one row to 32 rows; one split and many; ragged n and k; k = 1 and k = d.
SKINNY = [(1, 4096, 4096, 2048), (16, 8192, 1000, 4096), (32, 640, 4096, 640), (7, 300, 136, 77),
          (16, 2048, 64, 1), (32, 28672, 8192, 14336), (5, 4096, 67584 // 8, 3000), (16, 64, 8, 64)]


@pytest.mark.parametrize("m,d,n,k", SKINNY)
def test_skinny_bf16(m, d, n, k):
    A, B, I = _acts(m, d, m + d), _weight(d, n, n + k), _indices(d, k, m * k)
    Y = R.rmm_gemm(dev_tensor(A, BF), dev_tensor(B, BF), dev_tensor(I, torch.int32), k).float().cpu().numpy()
    assert rel_fro(Y, oracle.reduced_product(A, B, I)) < TOL_BF16


def test_skinny_bf16_unsorted_invalid_indices_and_output_stride():
    m, d, n, k = 16, 1000, 520, 700
    A, B = _acts(m, d, 3), _weight(d, n, 4)
    I = _indices(d, k, 5, sort=False)
    I[::9] = -1
    I[4::9] = d + 7                               # contributes zero
    Yfull = torch.zeros((m, n + 8), dtype=BF, device=DEV)
    R.rmm_gemm(dev_tensor(A, BF), dev_tensor(B, BF), dev_tensor(I, torch.int32), k, out=Yfull[:, :n])
    keep = I[(I >= 0) & (I < d)]
    assert rel_fro(Yfull[:, :n].float().cpu().numpy(), oracle.reduced_product(A, B, keep)) < TOL_BF16
    assert torch.all(Yfull[:, n:] == 0)


def test_skinny_is_deterministic():
    m, d, n, k = 16, 8192, 4096, 4096
    A, B, I = (dev_tensor(_acts(m, d, 6), BF), dev_tensor(_weight(d, n, 7), BF),
               dev_tensor(_indices(d, k, 8), torch.int32))
    assert torch.equal(R.rmm_gemm(A, B, I, k), R.rmm_gemm(A, B, I, k))


def _q_dev(q):
    """INT8 weight on the device with rows padded to a multiple of 16 bytes (a [d, n] view)."""
    d, n = q.shape
    ld = (n + 15) // 16 * 16
    buf = torch.zeros((d, ld), dtype=torch.int8, device=DEV)
    buf[:, :n] = torch.from_numpy(q).to(DEV)
    return buf[:, :n]


# INT8 weights: few-row kernel (m <= 32) and the dequantized many-row paths (m > 32, m >= 1024).
W8 = [(1, 4096, 4096, 2048), (16, 8192, 1000, 4096), (32, 640, 4096, 640), (16, 2048, 64, 1),
      (16, 28672, 8192, 14336), (100, 1000, 520, 333), (1500, 2048, 1100, 1024)]


@pytest.mark.parametrize("m,d,n,k", W8)
def test_w8(m, d, n, k):
    A, (q, s), I = _acts(m, d, m + 2 * d), synth.int8_per_column(_weight(d, n, n + 3)), _indices(d, k, k + 9)
    Y = R.rmm_gemm_w8(dev_tensor(A, BF), _q_dev(q), torch.from_numpy(s).to(DEV),
                      dev_tensor(I, torch.int32), k).float().cpu().numpy()
    assert rel_fro(Y, oracle.reduced_product_w8(A, q, s, I)) < TOL_BF16


def test_w8_invalid_indices_and_determinism():
    m, d, n, k = 8, 3000, 4096, 1500
    A, (q, s) = _acts(m, d, 11), synth.int8_per_column(_weight(d, n, 12))
    I = _indices(d, k, 13)
    I[::7] = -1
    Ad, qd, sd, Id = (dev_tensor(A, BF), torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                      dev_tensor(I, torch.int32))
    Y1 = R.rmm_gemm_w8(Ad, qd, sd, Id, k)
    Y2 = R.rmm_gemm_w8(Ad, qd, sd, Id, k)
    assert torch.equal(Y1, Y2)
    keep = I[I >= 0]
    assert rel_fro(Y1.float().cpu().numpy(), oracle.reduced_product_w8(A, q, s, keep)) < TOL_BF16


def test_w8_decode_needs_aligned_rows():
    m, d, n, k = 4, 100, 100, 50                  # 100-byte weight rows
    A, (q, s) = _acts(m, d, 14), synth.int8_per_column(_weight(d, n, 15))
    with pytest.raises(R.RMMError) as e:
        R.rmm_gemm_w8(dev_tensor(A, BF), torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                      dev_tensor(_indices(d, k, 16), torch.int32), k)
    assert e.value.status == R.RMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()


# The LLaMA-3.1-70B decode batch (m = 16) with its projections held as INT8.
W70 = synth.WORKLOADS["llama3.1-70b-layer"]


@pytest.mark.parametrize("name", sorted([l.name for l in W70.linears if "@m16@" in l.name and l.rho == 0.5]))
def test_llama70b_decode_projection_int8(name):
    lin = [l for l in W70.linears if l.name == name][0]
    A = synth.linear_activation(W70, lin)
    q, s = synth.linear_weight_int8(W70, lin)
    Ad = dev_tensor(A, BF)
    k = R.rmm_k_from_rho(lin.rho, lin.d)
    assert k == oracle.retained_count(lin.rho, lin.d)
    sc = R.rmm_colnorm(Ad)
    idx = R.rmm_topk(sc, k)
    Y = R.rmm_gemm_w8(Ad, torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), idx, k)
    s_ora = oracle.column_scores(A)
    check_selection(idx.cpu().numpy(), sc.cpu().numpy(), s_ora, k)
    I = idx.cpu().numpy()[:k]
    assert rel_fro(Y.float().cpu().numpy(), oracle.reduced_product_w8(A, q, s, I)) < TOL_BF16
    torch.cuda.synchronize()


def test_decode_chain_graph_replay_matches_eager():
    """Scores -> top-k -> few-row GEMM captured in a HIP graph: every replay, with
    eager work and synchronisations between them, equals the eager result."""
    m, d, n, rho = 16, 8192, 4096, 0.5
    A = dev_tensor(_acts(m, d, 21), BF)
    B = dev_tensor(_weight(d, n, 22), BF)
    k = R.rmm_k_from_rho(rho, d)
    sc = torch.empty(d, dtype=torch.float32, device=DEV)
    idx = torch.empty(R.rmm_k_pad(k), dtype=torch.int32, device=DEV)
    Y = torch.empty((m, n), dtype=BF, device=DEV)
    ws_c = torch.empty(max(R.rmm_colnorm_workspace_bytes(BF, m, d), 1), dtype=torch.uint8, device=DEV)
    ws_g = torch.empty(R.rmm_gemm_workspace_bytes(BF, m, n, k), dtype=torch.uint8, device=DEV)

    def chain():
        R.rmm_colnorm(A, out=sc, ws=ws_c)
        R.rmm_topk(sc, k, out=idx)
        R.rmm_gemm(A, B, idx, k, out=Y, ws=ws_g)

    chain()
    torch.cuda.synchronize()
    y_ref, i_ref = Y.clone(), idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(4):
        Y.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, i_ref), f"replay {rep}: indices differ"
        assert torch.equal(Y, y_ref), f"replay {rep}: output differs"
        _ = (B[:64].float() * 2).sum().item()                      # unrelated eager work

"""Reduced projections with an operand larger than 4 GiB.

An activation over 4 GiB: one seeded 1024-row block repeated down the rows, so its
column scores have a closed form: s_j over reps copies of the block is
sqrt(reps) times the block's own column norm (float64, from the oracle), and
every output row equals the product of one block row.  A matrix of this size
leaves the 32-bit buffer ranges of the wide-row gather, so the path takes the
generic gather with 64-bit offsets; the reduced GEMM addresses each output
tile from its own base.  With 139264 rows a lane of the column-norm kernel
adds about 136 squares in sequence, so the score tolerances of the smaller
cases still hold (worst case about 5e-6 relative, typically 1e-7).
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


def test_projection_with_activation_over_4gib():
    rows, d, n, reps, rho = 1024, 16384, 512, 136, 0.5
    m = rows * reps
    assert m * d * 2 > 4 * 2**30
    block = synth.lognormal_col_activations(synth.stream(11, 77, 1), rows, d, 1.0, bf16=True)
    B = synth.lognormal_col_activations(synth.stream(12, 77, 1), d, n, 1.0, bf16=True) / math.sqrt(d)
    blk_d = dev_tensor(block, torch.bfloat16)
    block64 = blk_d.double().cpu().numpy()                 # the values the kernels read
    Bd = dev_tensor(B, torch.bfloat16)
    B64 = Bd.double().cpu().numpy()
    A = blk_d.repeat(reps, 1)
    del blk_d
    Y, idx, s, k = R.rmm_linear(A, Bd, rho)
    torch.cuda.synchronize()
    assert k == oracle.retained_count(rho, d)

    s_gpu = s.cpu().numpy()
    s_ora = math.sqrt(reps) * oracle.column_scores(block64)
    print(f"  score rms rel err {check_scores(s_gpu, s_ora):.2e}")
    check_selection(idx.cpu().numpy(), s_gpu, s_ora, k)
    I = idx.cpu().numpy()[:k]

    pick = np.unique(np.concatenate([[0, 1, rows - 1, rows, m // 2, m - rows, m - 2, m - 1],
                                     np.random.default_rng(5).choice(m, size=56, replace=False)]))
    got = Y[torch.from_numpy(pick).to(DEV)].float().cpu().numpy()
    want = oracle.reduced_product(block64[pick % rows], B64, I)
    err = rel_fro(got, want)
    print(f"  m={m} k={k} sampled rows {pick.size} rel_fro={err:.2e}")
    assert err < TOL_BF16
    del A, Y
    torch.cuda.empty_cache()


def test_projection_with_weight_over_4gib():
    """A weight larger than 4 GiB (8192 x 270336 bf16, as a vocabulary-sized
    projection) is beyond the 32-bit buffer ranges of the other GEMM paths;
    the product runs on the row-gather kernel that addresses the kept weight
    rows with 64-bit pointers.  Checked on sampled output columns, the first
    and last included."""
    m, d, n, rho = 48, 8192, 270336, 0.5
    assert d * n * 2 > 4 * 2**30
    A = synth.lognormal_col_activations(synth.stream(13, 77, 1), m, d, 1.0, bf16=True)
    Ad = dev_tensor(A, torch.bfloat16)
    A64 = Ad.double().cpu().numpy()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(14)
    Bd = torch.randn((d, n), generator=gen, device=DEV, dtype=torch.bfloat16)
    Bd.mul_(1.0 / math.sqrt(d))
    Y, idx, s, k = R.rmm_linear(Ad, Bd, rho)
    torch.cuda.synchronize()
    assert k == oracle.retained_count(rho, d)
    s_gpu = s.cpu().numpy()
    s_ora = oracle.column_scores(A64)
    check_scores(s_gpu, s_ora)
    check_selection(idx.cpu().numpy(), s_gpu, s_ora, k)
    I = idx.cpu().numpy()[:k]
    assert int(I.max()) * n * 2 > 4 * 2**30                    # kept rows beyond the first 4 GiB
    cols = np.unique(np.concatenate([[0, 1, n // 2, n - 2, n - 1],
                                     np.random.default_rng(6).choice(n, size=59, replace=False)]))
    cols_d = torch.from_numpy(cols).to(DEV)
    got = Y[:, cols_d].float().cpu().numpy()
    want = oracle.reduced_product(A64, Bd[:, cols_d].double().cpu().numpy(), I)
    err = rel_fro(got, want)
    print(f"  n={n} k={k} sampled columns {cols.size} rel_fro={err:.2e}")
    assert err < TOL_BF16
    del Bd, Y
    torch.cuda.empty_cache()

"""Shared helpers for the GPU parity tests (comparison rules, device transfer)."""
from __future__ import annotations

import numpy as np

import oracle

GAP = 1e-5          # relative gap between the k-th and (k+1)-th oracle scores
TOL_BF16 = 1e-2     # relative Frobenius error, bf16 operands
TOL_F32 = 1e-5      # relative Frobenius error, float32 operands


def dev_tensor(a: np.ndarray, dtype, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def rel_fro(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


# Column scores: every score within SCORE_RTOL of float64 (the worst case of a
# blocked float32 sum of up to 16384 squares), and the root-mean-square
# relative error within SCORE_RMS (the typical error of that sum, about
# sqrt(terms per block) * 2^-24).
SCORE_RTOL = 1e-5
SCORE_RMS = 1e-6


def score_rms(gpu_scores, oracle_scores) -> float:
    """Root-mean-square relative error of the scores whose float64 value is
    above 1e-30 (the per-score check covers the rest)."""
    g = np.asarray(gpu_scores, dtype=np.float64)
    o = np.asarray(oracle_scores, dtype=np.float64)
    nz = o > 1e-30
    if not np.any(nz):
        return 0.0
    rel = (g[nz] - o[nz]) / o[nz]
    return float(np.sqrt(np.mean(rel * rel)))


def check_scores(gpu_scores, oracle_scores, atol=0.0) -> float:
    """Both score rules; returns the root-mean-square relative error."""
    np.testing.assert_allclose(gpu_scores, oracle_scores, rtol=SCORE_RTOL, atol=atol)
    rms = score_rms(gpu_scores, oracle_scores)
    assert rms <= SCORE_RMS, rms
    return rms


def rank_gap(s: np.ndarray, k: int) -> float:
    """(s_(k) - s_(k+1)) / s_(k) for the k-th/(k+1)-th largest scores; inf when k == d."""
    d = s.shape[0]
    if k >= d:
        return float("inf")
    top = np.sort(s)[::-1]
    if top[k - 1] == 0:
        return 0.0
    return float((top[k - 1] - top[k]) / top[k - 1])


def check_selection(idx_row: np.ndarray, gpu_scores: np.ndarray, oracle_scores: np.ndarray, k: int):
    """Index-set rules.  Returns 1 for a near tie (counted), 0 otherwise.

    * Always: the GPU's kept set is exactly the oracle's selection applied to
      the GPU's own float32 scores (no tolerance), ascending, padded with -1.
    * When the oracle's float64 gap at rank k exceeds GAP, the set must also
      equal the oracle's float64 selection.
    """
    kp = idx_row.shape[0]
    I = idx_row[:k].astype(np.int64)
    assert np.all(idx_row[k:kp] == -1), "padding must be -1"
    assert np.array_equal(I, oracle.select_top(gpu_scores.astype(np.float64), k)), "selection differs on GPU scores"
    I_ora = oracle.select_top(oracle_scores, k)
    if rank_gap(oracle_scores, k) > GAP:
        assert np.array_equal(I, I_ora), "selection differs from oracle"
        return 0
    # Near tie: any disagreement with the float64 selection must be a swap of
    # indices whose float64 scores lie within the tie band around the k-th score.
    kth = np.sort(oracle_scores)[::-1][k - 1]
    for j in np.setxor1d(I, I_ora):
        assert abs(oracle_scores[j] - kth) <= GAP * kth, "swap outside the tie band"
    return 1

"""Comparison rules of the parity tests (shared by the GPU tests and smoke()).

* Chunk sets are compared exactly, except at score near-ties: a chunk in the
  symmetric difference of the GPU set and the oracle set is a near-tie when its
  oracle score is within 1e-5 * max(|s_(k)|, rms(row)) of the oracle's k-th
  score s_(k).  Near-ties are counted; any other difference fails.
* Attention outputs: max |out - out_oracle| <= 1e-4 for fp32 K/V and <= 2e-2 for
  bf16 K/V; the same bounds apply to lse.
"""
from __future__ import annotations

import numpy as np

NEAR_TIE_REL = 1e-5
ATOL = {"f32": 1e-4, "bf16": 2e-2}


def compare_topk(gpu_idx: np.ndarray, oracle_idx: np.ndarray, oracle_scores: np.ndarray):
    """Return (#rows that differ, #near-tie chunks, list of hard failures).

    gpu_idx, oracle_idx: [..., k]; oracle_scores: [..., C] (fp64).
    """
    gi = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    oi = oracle_idx.reshape(-1, oracle_idx.shape[-1])
    sc = oracle_scores.reshape(-1, oracle_scores.shape[-1])
    rows_diff, near, hard = 0, 0, []
    for r in range(gi.shape[0]):
        a, b = set(gi[r].tolist()), set(oi[r].tolist())
        if len(a) != gi.shape[1]:
            hard.append((r, "duplicate ids in GPU row"))
            continue
        if not np.all(np.diff(gi[r]) > 0):
            hard.append((r, "GPU row not ascending"))
        if a == b:
            continue
        rows_diff += 1
        row = sc[r]
        sk = row[oi[r]].min()
        tol = NEAR_TIE_REL * max(abs(sk), float(np.sqrt(np.mean(row ** 2))))
        for c in a ^ b:
            if not (0 <= c < row.shape[0]) or abs(row[c] - sk) > tol:
                hard.append((r, c, float(row[c]) if 0 <= c < row.shape[0] else None, float(sk)))
            else:
                near += 1
    return rows_diff, near, hard


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isneginf(a) & np.isneginf(b)
    d = np.abs(np.where(both_inf, 0.0, a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0

"""Metrics reported beside the oracle's outputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* rel-L1: sum |O - O_dense| / sum |O_dense| over the evaluated rows.
* block sparsity: 1 - (kept blocks) / (admissible blocks).
* P.V skip fraction: skipped (tile, group) pairs / all (tile, group) pairs of
  the kept tiles.
* true recall: mean over rows of the exact softmax mass that falls inside the
  row's kept key blocks (how much of the true attention map the mask keeps;
  the DynSparse story argues a fixed recall preserves accuracy).
"""
from __future__ import annotations

from typing import List

import numpy as np


def rel_l1(O: np.ndarray, O_dense: np.ndarray) -> float:
    O = np.asarray(O, dtype=np.float64)
    O_dense = np.asarray(O_dense, dtype=np.float64)
    return float(np.abs(O - O_dense).sum() / np.abs(O_dense).sum())


def block_sparsity(kept_counts, admissible_counts) -> float:
    return float(1.0 - np.sum(kept_counts) / np.sum(admissible_counts))


def skip_fraction(skips: List[np.ndarray]) -> float:
    tot = sum(s.size for s in skips)
    return float(sum(int(s.sum()) for s in skips) / tot) if tot else 0.0


def true_recall(Q, K, kept: List[np.ndarray], BQ: int, BK: int, sm: float,
                causal: bool, blocks=None) -> float:
    """Mean exact attention mass inside the kept key blocks, over the rows
    of ``blocks`` (all query blocks by default)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    N = Q.shape[0]
    if blocks is None:
        blocks = range(len(kept))
    tot, cnt = 0.0, 0
    for i in blocks:
        rows = np.arange(i * BQ, min(N, (i + 1) * BQ))
        S = sm * (Q[rows] @ K.T)
        if causal:
            S = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, S)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        E /= E.sum(axis=1, keepdims=True)
        keep = np.zeros(N, dtype=bool)
        for j in kept[i]:
            keep[j * BK:min(N, (j + 1) * BK)] = True
        tot += float(E[:, keep].sum())
        cnt += len(rows)
    return tot / cnt

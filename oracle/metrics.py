"""Metrics reported beside the oracle's outputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Each metric is the
plain definition, for one head at a time unless stated:

* rel-L1: sum |O - O_dense| / sum |O_dense| over the evaluated rows (the
  relative error of the sparse result against exact dense attention).
* max-abs: max |A - B| over all elements.
* admissible counts |A_i|: key blocks a query block may attend to (all of
  them; under causality those whose first key is not after the block's last
  row).
* block sparsity: 1 - (kept blocks) / (admissible blocks), summed over every
  query block given.
* P.V skip fraction: skipped (tile, group) pairs / all (tile, group) pairs of
  the kept tiles, where query block i has ceil(|R_i| / G) real row groups;
  group slots past the last row of a partial block are not counted.
* predicted kept mass: sum of P-hat over the kept blocks of each query block
  (the cut guarantees it reaches tau under the cumulative-mass rule).
* true recall: mean over rows of the exact softmax mass that falls inside the
  row's kept key blocks -- how much of the true attention map the mask keeps
  (the DynSparse story argues that a fixed recall preserves accuracy).
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import numpy as np


def rel_l1(O: np.ndarray, O_dense: np.ndarray) -> float:
    """sum |O - O_dense| / sum |O_dense|."""
    O = np.asarray(O, dtype=np.float64)
    O_dense = np.asarray(O_dense, dtype=np.float64)
    return float(np.abs(O - O_dense).sum() / np.abs(O_dense).sum())


def max_abs(A: np.ndarray, B: np.ndarray) -> float:
    """max |A - B| (0 for empty inputs)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    return float(np.abs(A - B).max()) if A.size else 0.0


def admissible_counts(N: int, BQ: int, BK: int, causal: bool) -> np.ndarray:
    """|A_i| per query block: every key block, or under causality the key
    blocks j with j * BK <= last row of R_i."""
    nqb, nkb = (N + BQ - 1) // BQ, (N + BK - 1) // BK
    if not causal:
        return np.full(nqb, nkb, dtype=np.int64)
    last_rows = np.minimum(N, (np.arange(nqb) + 1) * BQ) - 1
    return (last_rows // BK + 1).astype(np.int64)


def block_sparsity(kept_counts, admissible) -> float:
    """1 - sum(kept) / sum(admissible) over the query blocks given."""
    return float(1.0 - np.sum(kept_counts, dtype=np.float64) /
                 np.sum(admissible, dtype=np.float64))


def real_groups(rows: int, G: int) -> int:
    """Row groups of G rows that hold at least one real row."""
    return (int(rows) + G - 1) // G


def skip_fraction(skips: Sequence[np.ndarray], row_counts: Iterable[int], G: int) -> float:
    """``skips[i]``: bool [k_i, n_slots] skip decisions of query block i (one
    column per group slot); ``row_counts[i]`` = |R_i|.  Only the first
    ceil(|R_i| / G) columns are groups of real rows."""
    skipped = total = 0
    for s, r in zip(skips, row_counts):
        s = np.asarray(s, dtype=bool)
        ng = real_groups(r, G)
        skipped += int(s[:, :ng].sum())
        total += s.shape[0] * ng
    return float(skipped / total) if total else 0.0


def predicted_kept_mass(P: np.ndarray, kept: Sequence[np.ndarray],
                        blocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """sum over j in L_i of P-hat_ij, for each query block i of ``blocks``
    (all by default)."""
    P = np.asarray(P, dtype=np.float64)
    if blocks is None:
        blocks = range(len(kept))
    return np.array([float(P[i, np.asarray(kept[i], dtype=np.int64)].sum()) for i in blocks])


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

"""Comparison rules between the GPU path and the fp64 oracle.

Masks: bit-exact kept lists, except where floating point cannot decide:
  * set differences are excused when the oracle's cumulative mass at the cut
    is within 1e-6 of tau (|c(k) - tau| or |c(k-1) - tau| <= 1e-6), or every
    differing block's P-hat is within 1e-6 of the last kept block's P-hat;
  * order differences are excused between blocks of the same forced class
    whose scores are within 1e-6 * max(1, |s|) of each other.
Skip bits: exact, except groups whose delta is within `tol` of lambda.
Outputs: max |O_gpu - O_oracle| with the oracle run under the GPU's own
mask and skip decisions.
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-6
MASS_TOL = 1e-6


def order_key_ok(lst, s, forced):
    """The list must be sorted by (forced first, s desc, j asc) up to score
    near-ties.  Returns the first offending position or -1."""
    for t in range(len(lst) - 1):
        a, b = lst[t], lst[t + 1]
        fa, fb = bool(forced[a]), bool(forced[b])
        if fa != fb:
            if fb and not fa:
                return t
            continue
        if s[a] > s[b] or (s[a] == s[b] and a < b):
            continue
        if abs(s[a] - s[b]) <= REL_TIE * max(1.0, abs(s[a])):
            continue
        return t
    return -1


def compare_mask_row(gpu_list, pred, i, tau):
    """Returns (ok, exact, reason) for query block i of one head."""
    o_list = pred["kept"][i]
    if len(gpu_list) == len(o_list) and np.array_equal(gpu_list, o_list):
        return True, True, ""
    s, P, F, adm = pred["s"][i], pred["P"][i], pred["forced"][i], pred["adm"][i]
    g = list(int(x) for x in gpu_list)
    if any(not adm[j] for j in g) or len(set(g)) != len(g):
        return False, False, "inadmissible or repeated block"
    if not all(F[j] for j in g[:int(F.sum())]) or not set(np.flatnonzero(F)).issubset(g):
        return False, False, "forced blocks missing or not first"
    bad = order_key_ok(g, s, F)
    if bad >= 0:
        return False, False, f"order violated at {bad}: {g[bad]} before {g[bad+1]}"
    diff = set(g) ^ set(int(x) for x in o_list)
    if diff:
        order = pred["order"][i]
        k = len(o_list)
        c = np.cumsum(P[order])
        near_cut = (abs(c[k - 1] - tau) <= MASS_TOL) or (k >= 2 and abs(c[k - 2] - tau) <= MASS_TOL)
        pk = P[order[k - 1]]
        near_mass = all(abs(P[j] - pk) <= MASS_TOL for j in diff)
        if not (near_cut or near_mass):
            return False, False, f"kept sets differ by {sorted(diff)} (cut mass {c[k-1]:.9f})"
    return True, False, "excused"


def compare_masks(gpu_kept, preds, tau):
    """gpu_kept / preds: per head.  Returns (n_rows, n_exact, failures)."""
    n = exact = 0
    fails = []
    for hidx, (gl, pr) in enumerate(zip(gpu_kept, preds)):
        for i in range(len(pr["kept"])):
            ok, ex, why = compare_mask_row(gl[i], pr, i, tau)
            n += 1
            exact += ex
            if not ok:
                fails.append((hidx, i, why))
    return n, exact, fails


def out_tol(mode, V=None):
    """Max-abs bar for the fp32 output against the oracle run under the GPU's
    own mask and skip bits: 1e-2 for bf16 and fp32 inputs, 5e-2 for
    INT8/FP8 (the stated tolerances; the 4-bit Q/K codes take the quantised
    bar too)."""
    return {"bf16": 1e-2, "f32": 1e-2, "i8fp8": 5e-2, "i4fp8": 5e-2}[mode]


def compare_recall_skips(gpu_skips, stats, tol):
    """Recall rule.  ``stats`` are the oracle's group statistics (relative
    slack) computed along the GPU's own skip history (the oracle run with
    force_skip = the GPU's bits), so an earlier near-threshold difference
    does not cascade; the oracle would skip where stat >= 0.  A differing bit
    is excused when |stat| <= tol."""
    n = mism = 0
    fails = []
    for i, (g, st) in enumerate(zip(gpu_skips, stats)):
        ng = st.shape[1]
        gg = g[:, :ng]
        n += gg.size
        diff = gg != (st >= 0)
        if diff.any():
            mism += int(diff.sum())
            bad = diff & ~(np.abs(st) <= tol)
            if bad.any():
                t, gi = np.argwhere(bad)[0]
                fails.append((i, int(t), int(gi), float(st[t, gi])))
    return n, mism, fails


def compare_skips(gpu_skips, oracle_skips, oracle_deltas, lam, tol):
    """All lists are per query block: bool/float [cnt, n_groups]."""
    n = mism = 0
    fails = []
    for i, (g, o, d) in enumerate(zip(gpu_skips, oracle_skips, oracle_deltas)):
        ng = o.shape[1]
        gg = g[:, :ng]
        n += gg.size
        diff = gg != o
        if diff.any():
            mism += int(diff.sum())
            near = np.abs(d - lam) <= tol
            if np.any(diff & ~near):
                t, gi = np.argwhere(diff & ~near)[0]
                fails.append((i, int(t), int(gi), float(d[t, gi])))
    return n, mism, fails

"""Comparison rules between the GPU path and the fp64 oracle.

Masks.  Bit-exact kept lists, except where floating point cannot decide.
The GPU scores blocks from fp32 block means; the oracle from fp64 ones (the
scores then differ by about 1e-8 at the video shapes).  So:
  * position t of the GPU list must hold the oracle's block at position t of
    its processing order, or a block tied with it: consecutive blocks of
    that order in the same forced class whose scores lie within
    REL_TIE * max(1, |s|) of each other form one tie class, and the GPU may
    order a tie class differently (at the cut, keep another subset of it);
  * the length may differ from the oracle's only where the oracle's
    cumulative P-hat along the GPU's list is within MASS_TOL of tau at the
    boundary (a longer GPU list stopped no later than the mass tau + MASS_TOL,
    a shorter one reached tau - MASS_TOL); never when tau >= 1 (keep all) or
    for the top-k rule (callers pass tau = 2 there).
With ``means_preds`` (the oracle's steps after pooling run on the GPU's own
block means) every row must also match that prediction with the ties and
mass tolerance at 1e-12: the GPU's scoring, sort and cut are then checked on
their own, exactly up to fp64 rounding.
Skip bits: exact, except groups whose delta is within `tol` of lambda.
Outputs: max |O_gpu - O_oracle| with the oracle run under the GPU's own
mask and skip decisions.
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-6
MASS_TOL = 1e-6
EXACT_TIE = 1e-12


def tie_classes(order, s, forced, rel):
    """Class id of each position of ``order``: a new class starts where the
    forced class changes or the score gap to the previous entry exceeds
    rel * max(1, |s|)."""
    cls = np.zeros(len(order), dtype=np.int64)
    c = 0
    for t in range(1, len(order)):
        a, b = order[t - 1], order[t]
        if bool(forced[a]) != bool(forced[b]) or \
                abs(s[a] - s[b]) > rel * max(1.0, abs(s[a]), abs(s[b])):
            c += 1
        cls[t] = c
    return cls


def compare_mask_row(gpu_list, pred, i, tau, rel=REL_TIE, mass_tol=MASS_TOL):
    """Returns (ok, exact, reason) for query block i of one head."""
    o_list = pred["kept"][i]
    if len(gpu_list) == len(o_list) and np.array_equal(gpu_list, o_list):
        return True, True, ""
    s, P, F, adm = pred["s"][i], pred["P"][i], pred["forced"][i], pred["adm"][i]
    g = [int(x) for x in gpu_list]
    if any(not (0 <= j < len(adm)) or not adm[j] for j in g) or len(set(g)) != len(g):
        return False, False, "inadmissible or repeated block"
    if not all(F[j] for j in g[:int(F.sum())]) or not set(np.flatnonzero(F)).issubset(g):
        return False, False, "forced blocks missing or not first"
    order = [int(x) for x in pred["order"][i]]
    cls = tie_classes(order, s, F, rel)
    cls_of = {j: cls[t] for t, j in enumerate(order)}
    for t, j in enumerate(g):
        if cls_of[j] != cls[t]:
            return False, False, (f"position {t}: block {j} where the oracle has {order[t]} "
                                  f"(scores {s[j]:.9g} vs {s[order[t]]:.9g})")
    kg, ko = len(g), len(o_list)
    if kg != ko:
        if tau >= 1.0:
            return False, False, f"{kg} blocks where tau >= 1 keeps all {ko}"
        cum = np.cumsum(P[np.array(g, dtype=np.int64)])
        if kg > ko and not (kg >= 2 and cum[kg - 2] <= tau + mass_tol):
            return False, False, (f"{kg} blocks where the oracle keeps {ko}: mass "
                                  f"{cum[kg - 2]:.9f} before the last one")
        if kg < ko and not cum[kg - 1] >= tau - mass_tol:
            return False, False, (f"{kg} blocks where the oracle keeps {ko}: mass "
                                  f"{cum[kg - 1]:.9f}")
    return True, False, "excused"


def compare_masks(gpu_kept, preds, tau, means_preds=None):
    """gpu_kept / preds (/ means_preds): per head.  Returns (n_rows, n_exact,
    failures)."""
    n = exact = 0
    fails = []
    for hidx, (gl, pr) in enumerate(zip(gpu_kept, preds)):
        for i in range(len(pr["kept"])):
            ok, ex, why = compare_mask_row(gl[i], pr, i, tau)
            n += 1
            exact += ex
            if not ok:
                fails.append((hidx, i, why))
            if means_preds is not None:
                ok, _, why = compare_mask_row(gl[i], means_preds[hidx], i, tau, rel=EXACT_TIE,
                                              mass_tol=EXACT_TIE)
                if not ok:
                    fails.append((hidx, i, "on the GPU's own means: " + why))
    return n, exact, fails


def out_tol(mode, V=None):
    """Max-abs bar for the fp32 output against the oracle run under the GPU's
    own mask and skip bits: 1e-2 for bf16 and fp32 inputs, 5e-2 for
    INT8/FP8 (the stated tolerances; the 4-bit Q/K codes and the
    power-of-two V scales take the quantised bar too)."""
    return {"bf16": 1e-2, "f32": 1e-2, "i8fp8": 5e-2, "i4fp8": 5e-2, "i8mxfp8": 5e-2}[mode]


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

"""CPU checks of the GPU-vs-oracle mask comparison (tests/compare.py).

The comparison must accept the oracle's own lists and the differences
floating point can make (a near-tie swapped, the cut moved where the mass at
the boundary is within the tolerance of tau), and reject the mistakes a
kernel could plausibly make: a list with a gap (a higher-ranked block
skipped), a swap of blocks whose scores are far apart, a list cut early or
late away from tau, an inadmissible or repeated block, forced blocks not
first.
"""
import numpy as np

import compare
import oracle as O


def _pred(tau=0.8):
    rng = np.random.default_rng(5)
    Q, K = (rng.standard_normal((512, 16)) for _ in range(2))
    return O.predict_head(Q, K, O.Params(tau=tau))


def _row(pred):
    # the query block with the longest kept list
    return int(np.argmax([len(k) for k in pred["kept"]]))


def test_accepts_the_oracle_lists():
    pred = _pred()
    n, ex, fails = compare.compare_masks([pred["kept"]], [pred], 0.8)
    assert not fails and ex == n == len(pred["kept"])


def test_rejects_a_gap_and_a_far_swap():
    pred = _pred()
    i = _row(pred)
    order, k = pred["order"][i], len(pred["kept"][i])
    assert k >= 3
    gap = np.concatenate([order[:1], order[2:k + 1]])  # skips the second-ranked block
    ok, _, why = compare.compare_mask_row(gap, pred, i, 0.8)
    assert not ok and "position 1" in why
    swap = order[:k].copy()
    swap[0], swap[k - 1] = swap[k - 1], swap[0]
    ok, _, _ = compare.compare_mask_row(swap, pred, i, 0.8)
    assert not ok


def test_rejects_wrong_lengths_away_from_tau():
    pred = _pred()
    i = _row(pred)
    order, k = pred["order"][i], len(pred["kept"][i])
    ok, _, why = compare.compare_mask_row(order[:k - 1], pred, i, 0.8)
    assert not ok and "mass" in why
    ok, _, why = compare.compare_mask_row(order[:k + 1], pred, i, 0.8)
    assert not ok and "mass" in why
    # tau >= 1 and the top-k rule (tau = 2) allow no length difference
    full = O.predict_head(*(np.random.default_rng(5).standard_normal((512, 16))
                            for _ in range(2)), O.Params(tau=1.0))
    ok, _, _ = compare.compare_mask_row(full["order"][i][:-1], full, i, 1.0)
    assert not ok


def test_rejects_structural_mistakes():
    pred = _pred()
    i = _row(pred)
    lst = list(pred["kept"][i])
    ok, _, why = compare.compare_mask_row(lst[:-1] + [lst[0]], pred, i, 0.8)
    assert not ok and "repeated" in why
    ok, _, _ = compare.compare_mask_row(lst[:-1] + [10_000], pred, i, 0.8)
    assert not ok
    # causal: the forced diagonal blocks must come first
    rng = np.random.default_rng(6)
    Q, K = (rng.standard_normal((512, 16)) for _ in range(2))
    cp = O.predict_head(Q, K, O.Params(tau=0.9, causal=True))
    j = 3
    lst = list(cp["kept"][j])
    nf = int(cp["forced"][j].sum())
    assert nf == 2 and len(lst) > nf
    bad = lst[nf:nf + 1] + lst[:nf] + lst[nf + 1:]
    ok, _, why = compare.compare_mask_row(bad, cp, j, 0.9)
    assert not ok and "forced" in why


def test_excuses_a_near_tie_and_a_cut_at_tau():
    pred = _pred()
    i = _row(pred)
    order, k = pred["order"][i], len(pred["kept"][i])
    s = pred["s"][i].copy()
    # make the blocks at positions 1 and 2 tie within 1e-7: a swap is excused
    s[order[2]] = s[order[1]] - 1e-7
    tied = dict(pred, s=[s if r == i else pred["s"][r] for r in range(len(pred["s"]))])
    lst = order[:k].copy()
    lst[1], lst[2] = lst[2], lst[1]
    ok, ex, _ = compare.compare_mask_row(lst, tied, i, 0.8)
    assert ok and not ex
    # ...but not on the GPU's own means, where ties are held to 1e-12
    ok, _, _ = compare.compare_mask_row(lst, tied, i, 0.8, rel=compare.EXACT_TIE,
                                        mass_tol=compare.EXACT_TIE)
    assert not ok
    # tau placed exactly at the cumulative mass of the first k - 1 blocks:
    # a list one block longer or shorter is within the mass tolerance
    c = np.cumsum(pred["P"][i][order])
    tau = float(c[k - 2]) + 5e-7
    ok, _, _ = compare.compare_mask_row(order[:k - 1], pred, i, tau)
    assert ok
    ok, _, _ = compare.compare_mask_row(order[:k - 1], pred, i, tau + 1e-5)
    assert not ok

"""CPU pins of the oracle's metrics (oracle/metrics.py).

Each metric is checked against something other than its own code: values
worked by hand, the token-level brute force in tests/brute.py, and closed
forms (a mask that keeps every admissible block has true recall 1 and
predicted kept mass 1; lambda = -inf skips no real group, lambda > 0 skips
all of them).  The cases are chosen so that the plausible slips fail: a
dropped absolute value in rel-L1, the admissible count under causality
taken as NKB or off by one block, phantom group slots of a partial query
block counted as skipped groups, a row-normalisation or causal-mask slip in
the recall.
"""
import math

import numpy as np
import pytest

import brute
import oracle as O


# ------------------------------------------------------------------ rel-L1
def test_rel_l1_hand_values():
    Od = np.array([[1.0, 1.0], [1.0, 1.0]])
    # |0| + |1| + |2| + |3| = 6 over |Od| = 4
    assert O.rel_l1(np.array([[1.0, 2.0], [3.0, 4.0]]), Od) == 1.5
    # sign errors count in absolute value: |-2| * 4 / 4
    assert O.rel_l1(-Od, Od) == 2.0
    assert O.rel_l1(Od, Od) == 0.0
    # the denominator takes |O_dense|: (0.5 + 0.5) / (1 + 3)
    assert O.rel_l1(np.array([0.5, -2.5]), np.array([1.0, -3.0])) == 0.25


def test_max_abs_hand_values():
    assert O.max_abs(np.array([1.0, -2.0, 3.0]), np.array([1.5, 2.0, 3.0])) == 4.0
    assert O.max_abs(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


# -------------------------------------------------------- block sparsity
@pytest.mark.parametrize("n", [1, 63, 64, 200, 256, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_admissible_counts_match_token_level_brute_force(n, causal):
    got = O.admissible_counts(n, 128, 64, causal)
    assert got.tolist() == brute.admissible(n, 128, 64, causal)
    # and the oracle's own admissible set (O2) agrees
    assert got.tolist() == O.admissible_blocks(n, 128, 64, causal).sum(axis=1).tolist()


def test_admissible_counts_hand_values():
    # N = 256 causal: rows 0..127 see key blocks 0, 1; rows 128..255 see 0..3
    assert O.admissible_counts(256, 128, 64, True).tolist() == [2, 4]
    # N = 1000 causal: last rows 127, 255, ..., 999 -> 2, 4, ..., 14, 16
    assert O.admissible_counts(1000, 128, 64, True).tolist() == [2, 4, 6, 8, 10, 12, 14, 16]
    assert O.admissible_counts(1000, 128, 64, False).tolist() == [16] * 8


def test_block_sparsity_hand_values():
    adm = O.admissible_counts(256, 128, 64, True)
    assert O.block_sparsity([2, 3], adm) == pytest.approx(1.0 - 5.0 / 6.0, abs=1e-15)
    assert O.block_sparsity([2, 4], adm) == 0.0
    # against the non-causal count the same lists would read sparser
    assert O.block_sparsity([2, 3], O.admissible_counts(256, 128, 64, False)) == \
        pytest.approx(1.0 - 5.0 / 8.0, abs=1e-15)


# ------------------------------------------------------ P.V skip fraction
def test_skip_fraction_counts_only_real_groups():
    # N = 160, G = 32: query block 0 has 128 rows (4 groups), block 1 has 32
    # rows (1 real group, 3 empty slots that kernels and oracle mark skipped)
    skips = [np.array([[1, 0, 0, 0], [1, 1, 0, 0]], dtype=bool),
             np.array([[0, 1, 1, 1]], dtype=bool)]
    rows = [128, 32]
    assert O.skip_fraction(skips, rows, 32) == pytest.approx(3.0 / 9.0, abs=1e-15)
    # counting the empty slots would give 6 / 12
    assert O.real_groups(32, 32) == 1 and O.real_groups(120, 32) == 4
    assert O.real_groups(16, 32) == 1 and O.real_groups(33, 32) == 2
    assert O.skip_fraction([], [], 32) == 0.0


@pytest.mark.parametrize("lam,expect", [(-math.inf, 0.0), (0.5, 1.0)])
def test_skip_fraction_closed_forms_on_a_partial_block(lam, expect):
    # lambda = -inf never skips a real group; lambda > 0 skips every group
    # (delta <= 0 < lambda); the oracle marks the slots past the last row
    # skipped either way, so only the real-group count gives 0 and 1
    rng = np.random.default_rng(11)
    n, d = 160, 8
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    p = O.Params(tau=0.9, lam=lam)
    pred = O.predict_head(Q, K, p)
    _, _, skips = O.sparse_attention_head(Q, K, V, pred["kept"], p)
    rows = [min(n, (i + 1) * 128) - i * 128 for i in range(len(skips))]
    assert rows == [128, 32]
    assert O.skip_fraction(skips, rows, p.G) == expect


# ------------------------------------------------- predicted kept mass
def test_predicted_kept_mass_hand_values():
    P = np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]])
    got = O.predicted_kept_mass(P, [np.array([0, 2]), np.array([2])])
    np.testing.assert_allclose(got, [0.7, 0.8], atol=1e-15)
    got = O.predicted_kept_mass(P, [np.array([0, 2]), np.array([2])], blocks=[1])
    np.testing.assert_allclose(got, [0.8], atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_predicted_kept_mass_reaches_tau_and_one(causal):
    rng = np.random.default_rng(12)
    Q, K = (rng.standard_normal((600, 16)) for _ in range(2))
    for tau in (0.3, 0.8, 0.95):
        pred = O.predict_head(Q, K, O.Params(causal=causal, tau=tau))
        assert np.all(O.predicted_kept_mass(pred["P"], pred["kept"]) >= tau)
    pred = O.predict_head(Q, K, O.Params(causal=causal, tau=1.0))
    np.testing.assert_allclose(O.predicted_kept_mass(pred["P"], pred["kept"]), 1.0, atol=1e-12)


# ------------------------------------------------------------ true recall
def test_true_recall_hand_values():
    # sm = 1, one-dimensional tokens: row 0 has logits (0, ln 3) -> masses
    # (1/4, 3/4); row 1 has logits (0, 0) -> (1/2, 1/2).  Keeping key block 1
    # (key 1) only: recall = (3/4 + 1/2) / 2
    Q = np.array([[1.0], [0.0]])
    K = np.array([[0.0], [math.log(3.0)]])
    kept = [np.array([1])]
    assert O.true_recall(Q, K, kept, 2, 1, 1.0, False) == pytest.approx(0.625, abs=1e-15)
    # causal: row 0 sees key 0 alone (mass 0 on key 1), row 1 as before
    assert O.true_recall(Q, K, kept, 2, 1, 1.0, True) == pytest.approx(0.25, abs=1e-15)
    assert O.true_recall(Q, K, [np.array([0, 1])], 2, 1, 1.0, True) == pytest.approx(1.0)
    assert O.true_recall(Q, K, [np.array([], dtype=np.int64)], 2, 1, 1.0, False) == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_true_recall_matches_scalar_brute_force(causal):
    rng = np.random.default_rng(13)
    n, d = 90, 4
    Q, K = (rng.standard_normal((n, d)) for _ in range(2))
    p = O.Params(BQ=16, BK=8, causal=causal, tau=0.7)
    kept = O.predict_head(Q, K, p)["kept"]
    sm = 1.0 / math.sqrt(d)
    for blocks in (None, [0, 3, 5]):
        got = O.true_recall(Q, K, kept, 16, 8, sm, causal, blocks=blocks)
        exp = brute.true_recall(Q.tolist(), K.tolist(), [k.tolist() for k in kept], 16, 8,
                                causal, sm=sm, blocks=blocks)
        assert got == pytest.approx(exp, abs=1e-12)
        assert 0.0 < got < 1.0


@pytest.mark.parametrize("causal", [False, True])
def test_true_recall_is_one_when_every_admissible_block_is_kept(causal):
    rng = np.random.default_rng(14)
    Q, K = (rng.standard_normal((300, 8)) for _ in range(2))
    p = O.Params(causal=causal, tau=1.0)
    kept = O.predict_head(Q, K, p)["kept"]
    assert O.true_recall(Q, K, kept, 128, 64, p.sm(8), causal) == pytest.approx(1.0, abs=1e-12)

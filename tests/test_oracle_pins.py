"""CPU pins of the fp64 oracle against things other than itself.

* scalar brute force (tests/brute.py) on tiny inputs, every branch;
* closed forms: tau = 1, lambda = -inf reproduces dense softmax attention;
  lambda > 0 skips every P.V product so O = 0; a constant block pools to its
  constant; energy weights equal top-cdf weights when all key blocks are full;
* invariants: weight rows sum to 1, kept mass >= tau, minimality of the cut,
  tau -> 0+ keeps max(1, |F|) blocks, |O| <= max |V|;
* subset enumeration of the cut for small NKB;
* special case: blockwise-constant Q/K make the pooled scores the exact
  logits, so the mask is top-cdf over the exact block masses;
* an independent library routine: torch's scaled_dot_product_attention in
  float64 for the dense reference.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import brute
import oracle as O


def rand_qkv(seed, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((n, d)), scale * rng.standard_normal((n, d)),
            rng.standard_normal((n, d)))


# ----------------------------------------------------------------- pooling
def test_pool_matches_brute_and_partial_block():
    q, _, _ = rand_qkv(1, 37, 5)
    got = O.pool_means(q, 8)
    exp = np.array(brute.pool(q.tolist(), 8))
    assert got.shape == (5, 5)
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-14)
    # the partial last block (5 rows) averages only its own rows
    np.testing.assert_allclose(got[-1], q[32:].mean(axis=0), atol=1e-15)


def test_pool_linearity_and_constant_block():
    a, b, _ = rand_qkv(2, 50, 4)
    np.testing.assert_allclose(O.pool_means(2.5 * a - 3.0 * b, 16),
                               2.5 * O.pool_means(a, 16) - 3.0 * O.pool_means(b, 16),
                               atol=1e-13)
    c = np.tile(np.array([[1.5, -2.0, 0.25]]), (20, 1))
    np.testing.assert_array_equal(O.pool_means(c, 8), np.tile(c[:1], (3, 1)))


# ------------------------------------------------------- weights and mask
@pytest.mark.parametrize("rule", ["topcdf", "energy"])
@pytest.mark.parametrize("causal", [False, True])
def test_weights_rows_sum_to_one(rule, causal):
    q, k, _ = rand_qkv(3, 203, 8)
    p = O.Params(BQ=16, BK=8, causal=causal, rule=rule, tau=0.9)
    pr = O.predict_head(q, k, p)
    sums = pr["P"].sum(axis=1)
    assert np.all(np.abs(sums - 1.0) <= 1e-12)
    assert np.all(pr["P"][~pr["adm"]] == 0)


def test_energy_equals_topcdf_on_full_blocks():
    q, k, _ = rand_qkv(4, 256, 8)
    pt = O.predict_head(q, k, O.Params(BQ=32, BK=16, tau=0.8))
    pe = O.predict_head(q, k, O.Params(BQ=32, BK=16, tau=0.8, rule="energy"))
    np.testing.assert_allclose(pt["P"], pe["P"], atol=1e-15)
    assert all(np.array_equal(a, b) for a, b in zip(pt["kept"], pe["kept"]))


def test_energy_weights_follow_block_sizes():
    # a partial last key block with equal scores gets proportionally less mass
    s = np.zeros((1, 3))
    adm = np.ones((1, 3), dtype=bool)
    P = O.block_weights(s, adm, "energy", np.array([64.0, 64.0, 32.0]))
    np.testing.assert_allclose(P[0], [0.4, 0.4, 0.2], atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rule", ["topcdf", "energy"])
@pytest.mark.parametrize("keep_prefix", [0, 2])
@pytest.mark.parametrize("tau", [0.3, 0.9, 0.999, 1.0])
def test_predict_matches_brute(causal, rule, keep_prefix, tau):
    q, k, _ = rand_qkv(5, 45, 4, scale=2.0)
    p = O.Params(BQ=8, BK=4, causal=causal, rule=rule, tau=tau,
                 keep_prefix_kblocks=keep_prefix)
    got = O.predict_head(q, k, p)["kept"]
    exp = brute.predict(q.tolist(), k.tolist(), 8, 4, causal, tau, rule, keep_prefix)
    assert [list(x) for x in got] == exp


def test_cut_invariants_and_minimality():
    q, k, _ = rand_qkv(6, 400, 8, scale=1.5)
    for tau in (0.2, 0.5, 0.9, 0.97):
        p = O.Params(BQ=32, BK=16, tau=tau, keep_prefix_kblocks=1)
        pr = O.predict_head(q, k, p)
        for i, lst in enumerate(pr["kept"]):
            mass = pr["P"][i, lst].sum()
            nf = int(pr["forced"][i].sum())
            assert mass >= tau - 1e-15
            assert np.all(pr["forced"][i, lst[:nf]])
            if len(lst) > nf:  # dropping the last kept block falls below tau
                assert pr["P"][i, lst[:-1]].sum() < tau


def test_cut_extremes():
    q, k, _ = rand_qkv(7, 300, 8)
    for causal, kp in ((False, 0), (False, 3), (True, 0)):
        adm = O.admissible_blocks(300, 32, 16, causal)
        pr = O.predict_head(q, k, O.Params(BQ=32, BK=16, causal=causal, tau=1e-12,
                                           keep_prefix_kblocks=kp))
        F = pr["forced"]
        for i, lst in enumerate(pr["kept"]):
            assert len(lst) == max(1, int(F[i].sum()))
        pr1 = O.predict_head(q, k, O.Params(BQ=32, BK=16, causal=causal, tau=1.0,
                                            keep_prefix_kblocks=kp))
        for i, lst in enumerate(pr1["kept"]):
            assert sorted(lst) == list(np.flatnonzero(adm[i]))


def test_cut_is_minimum_cardinality_by_subset_enumeration():
    """NKB <= 12: among all subsets that contain the forced blocks and reach
    tau, the greedy prefix has the minimum size and, at that size, the
    maximum mass (top-cdf weights are monotone in the score)."""
    rng = np.random.default_rng(8)
    for trial in range(30):
        nkb = int(rng.integers(3, 12))
        s = rng.normal(0, 1.5, size=(1, nkb))
        adm = np.ones((1, nkb), dtype=bool)
        P = O.block_weights(s, adm, "topcdf", np.full(nkb, 64.0))[0]
        F = np.zeros(nkb, dtype=bool)
        F[: int(rng.integers(0, 3))] = True
        tau = float(rng.uniform(0.05, 0.99))
        order = O.processing_order(s[0], adm[0], F)
        k = O.cut_length(P[order], int(F.sum()), tau)
        kept = set(order[:k].tolist())
        best = None
        for r in range(nkb + 1):
            for sub in itertools.combinations(range(nkb), r):
                if not set(np.flatnonzero(F)).issubset(sub):
                    continue
                if P[list(sub)].sum() >= tau:
                    mass = P[list(sub)].sum()
                    if best is None or mass > best[1]:
                        best = (set(sub), mass)
            if best is not None:
                break
        assert len(kept) == len(best[0]), (trial, kept, best)
        assert kept == best[0]


def test_blockwise_constant_inputs_predict_exactly():
    """Q and K constant over each block: pooled logits are the exact logits,
    so the kept set is top-cdf over the exact block masses."""
    rng = np.random.default_rng(9)
    d, BQ, BK = 8, 32, 16
    qc = rng.standard_normal((8, d)) * 1.5
    kc = rng.standard_normal((16, d)) * 1.5
    q = np.repeat(qc, BQ, axis=0)
    k = np.repeat(kc, BK, axis=0)
    tau = 0.9
    pr = O.predict_head(q, k, O.Params(BQ=BQ, BK=BK, tau=tau))
    sm = 1 / math.sqrt(d)
    for i in range(8):
        logits = sm * (q[i * BQ] @ k.T)
        e = np.exp(logits - logits.max())
        mass = np.add.reduceat(e, np.arange(0, len(e), BK)) / e.sum()
        order = np.argsort(-mass, kind="stable")
        cum = np.cumsum(mass[order])
        kk = int(np.searchsorted(cum, tau) + 1)
        assert set(pr["kept"][i].tolist()) == set(order[:kk].tolist())


def test_hand_worked_cut():
    """Scores ln 4, ln 3, ln 2, ln 1 over four blocks give masses 0.4, 0.3,
    0.2, 0.1; tau = 0.65 keeps the first two, tau = 0.85 the first three."""
    s = np.log(np.array([[2.0, 4.0, 1.0, 3.0]]))
    adm = np.ones((1, 4), dtype=bool)
    P = O.block_weights(s, adm, "topcdf", np.full(4, 64.0))[0]
    np.testing.assert_allclose(P, [0.2, 0.4, 0.1, 0.3], atol=1e-15)
    order = O.processing_order(s[0], adm[0], np.zeros(4, dtype=bool))
    assert order.tolist() == [1, 3, 0, 2]
    assert O.cut_length(P[order], 0, 0.65) == 2
    assert O.cut_length(P[order], 0, 0.85) == 3
    # a forced block goes first and counts toward tau
    F = np.array([False, False, True, False])
    order = O.processing_order(s[0], adm[0], F)
    assert order.tolist() == [2, 1, 3, 0]
    assert O.cut_length(P[order], 1, 0.65) == 3


def test_cut_boundary_is_inclusive():
    """Masses that are exact binary fractions reach tau exactly: the prefix
    that lands on tau is kept as is (sum >= tau, not > tau)."""
    assert O.cut_length(np.array([0.5, 0.25, 0.25]), 0, 0.75) == 2
    assert O.cut_length(np.array([0.5, 0.25, 0.25]), 0, 0.5) == 1
    assert O.cut_length(np.array([0.5, 0.25, 0.25]), 0, 0.75000001) == 3
    # rounding can leave the total below tau < 1: keep everything
    assert O.cut_length(np.array([0.3, 0.3, 0.3]), 0, 0.95) == 3


# ------------------------------------------------------- sparse attention
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lam", [-math.inf, -3.0, -0.5, 0.0, 0.7])
def test_sparse_attention_matches_brute(causal, lam):
    q, k, v = rand_qkv(10, 38, 3, scale=2.0)
    p = O.Params(BQ=8, BK=4, causal=causal, tau=0.8, lam=lam, G=4,
                 keep_prefix_kblocks=1)
    pr = O.predict_head(q, k, p)
    got, _, sk = O.sparse_attention_head(q, k, v, pr["kept"], p)
    lists = [list(x) for x in pr["kept"]]
    exp, esk = brute.attention(q.tolist(), k.tolist(), v.tolist(), lists, 8, 4,
                               causal, lam, 4)
    np.testing.assert_allclose(got, np.array(exp), atol=1e-12, rtol=0)
    assert [s.tolist() for s in sk] == esk


@pytest.mark.parametrize("G", [2, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_attention_groups_match_brute(G, causal):
    """Skip groups of a quarter, the whole and twice the query block (the last
    is one group per block, as G = 128 with 128-row blocks), against the
    scalar brute force, on a ragged N."""
    q, k, v = rand_qkv(12, 37, 3, scale=2.0)
    p = O.Params(BQ=8, BK=4, causal=causal, tau=0.8, lam=-0.5, G=G)
    pr = O.predict_head(q, k, p)
    got, _, sk = O.sparse_attention_head(q, k, v, pr["kept"], p)
    exp, esk = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                               [list(x) for x in pr["kept"]], 8, 4, causal, -0.5, G)
    np.testing.assert_allclose(got, np.array(exp), atol=1e-12, rtol=0)
    assert [s.tolist() for s in sk] == esk
    assert all(s.shape[1] == (8 + G - 1) // G for s in sk)


def test_sparse_attention_force_skip_matches_brute():
    q, k, v = rand_qkv(11, 40, 3, scale=2.0)
    p = O.Params(BQ=8, BK=4, tau=0.9, lam=-math.inf, G=4)
    pr = O.predict_head(q, k, p)
    rng = np.random.default_rng(0)
    fs = [rng.random((len(x), 2)) < 0.4 for x in pr["kept"]]
    got, _, sk = O.sparse_attention_head(q, k, v, pr["kept"], p, force_skip=fs)
    exp, _ = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                             [list(x) for x in pr["kept"]], 8, 4, False, -math.inf, 4,
                             force_skip=[f.tolist() for f in fs])
    np.testing.assert_allclose(got, np.array(exp), atol=1e-12)
    assert all(np.array_equal(a, b) for a, b in zip(sk, fs))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [256, 300])
def test_dense_identity_tau1_lambda_neginf(causal, n):
    q, k, v = rand_qkv(12, n, 16, scale=1.5)
    p = O.Params(BQ=32, BK=16, causal=causal, tau=1.0, lam=-math.inf, G=8)
    r = O.oracle_head(q, k, v, p)
    od, lse_d = O.dense_attention_head(q, k, v, p.sm(16), causal)
    assert np.abs(r["O"] - od).max() <= 1e-12 * max(1.0, np.abs(od).max())
    np.testing.assert_allclose(r["lse"], lse_d, atol=1e-12)
    assert not any(s.any() for s in r["skips"])


def test_positive_lambda_skips_everything():
    q, k, v = rand_qkv(13, 200, 8)
    for causal in (False, True):
        p = O.Params(BQ=32, BK=16, causal=causal, tau=0.9, lam=1e-9, G=8)
        r = O.oracle_head(q, k, v, p)
        assert np.all(r["O"] == 0.0)
        assert all(s.all() for s in r["skips"])


def test_output_bounded_by_v():
    q, k, v = rand_qkv(14, 333, 8, scale=3.0)
    for lam in (-math.inf, -2.0, 0.0):
        r = O.oracle_head(q, k, v, O.Params(BQ=32, BK=16, tau=0.7, lam=lam, G=8))
        assert np.abs(r["O"]).max() <= np.abs(v).max() + 1e-12


def test_dense_matches_torch_sdpa_and_brute():
    q, k, v = rand_qkv(15, 70, 6)
    for causal in (False, True):
        od, _ = O.dense_attention_head(q, k, v, 1 / math.sqrt(6), causal, chunk=16)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None],
            torch.from_numpy(v)[None], is_causal=causal)[0].numpy()
        np.testing.assert_allclose(od, t, atol=1e-13)
        b = np.array(brute.dense(q.tolist(), k.tolist(), v.tolist(), causal))
        np.testing.assert_allclose(od, b, atol=1e-13)


def test_lambda_zero_keeps_only_max_raising_tiles():
    """lambda = 0: a group multiplies P.V only for tiles whose local max
    reaches the new running max in some row of the group."""
    q, k, v = rand_qkv(16, 64, 4, scale=2.0)
    p = O.Params(BQ=16, BK=8, tau=1.0, lam=0.0, G=4)
    r = O.oracle_head(q, k, v, p)
    sm = p.sm(4)
    for i, lst in enumerate(r["kept"]):
        m = np.full(16, -np.inf)
        for t, j in enumerate(lst):
            S = sm * q[i * 16:(i + 1) * 16] @ k[j * 8:(j + 1) * 8].T
            mloc = S.max(axis=1)
            raises = mloc >= np.maximum(m, mloc)
            for g in range(4):
                assert r["skips"][i][t, g] == (not raises[g * 4:(g + 1) * 4].any())
            m = np.maximum(m, mloc)


# ------------------------------------------------------------ top-k rule
@pytest.mark.parametrize("causal", [False, True])
def test_topk_rule_keeps_the_k_highest_scores(causal):
    """The top-k cut against an independent selection: forced blocks, then
    the k - |F| highest pooled scores (ties by index) via a stable argsort."""
    q, k, _ = rand_qkv(41, 300, 8, scale=2.0)
    for kk in (1, 3, 7, 100):
        p = O.Params(BQ=32, BK=16, causal=causal, rule="topk", topk_blocks=kk,
                     keep_prefix_kblocks=1)
        pr = O.predict_head(q, k, p)
        for i, lst in enumerate(pr["kept"]):
            adm = np.flatnonzero(pr["adm"][i])
            F = set(np.flatnonzero(pr["forced"][i]).tolist())
            want_n = min(len(adm), max(len(F), kk))
            assert len(lst) == want_n
            assert set(lst[:len(F)].tolist()) == F
            rest = [j for j in adm if j not in F]
            s = pr["s"][i, rest]
            top = [rest[t] for t in np.argsort(-s, kind="stable")[:want_n - len(F)]]
            assert lst[len(F):].tolist() == top
        # P-hat is the top-cdf softmax whatever the budget
        p2 = O.Params(BQ=32, BK=16, causal=causal, rule="topcdf", keep_prefix_kblocks=1)
        np.testing.assert_array_equal(pr["P"], O.predict_head(q, k, p2)["P"])


def test_topk_budget_covering_everything_is_dense():
    q, k, v = rand_qkv(42, 200, 8)
    p = O.Params(BQ=32, BK=16, rule="topk", topk_blocks=1000, lam=-math.inf)
    pr = O.predict_head(q, k, p)
    Oo, _, _ = O.sparse_attention_head(q, k, v, pr["kept"], p)
    od, _ = O.dense_attention_head(q, k, v, 1 / math.sqrt(8), False)
    np.testing.assert_allclose(Oo, od, atol=1e-12)

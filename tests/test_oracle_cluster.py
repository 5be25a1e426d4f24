"""CPU pins of the token reordering oracle (oracle/cluster.py, C1..C5).

Pinned against things other than the oracle's own code:
* the quadratic form is the mean squared logit change of replacing a token
  by a representative, evaluated by brute force over the other side's
  tokens (C1);
* quad_dist equals the direct (x - c)^T M (x - c) on small inputs;
* the feature metric reproduces scipy's Lloyd iteration
  (scipy.cluster.vq.kmeans2 from given centroids); the interaction metric
  reproduces the same routine on whitened data X L, M = L L^T (C3);
* Lloyd's objective never increases, neither at an update nor at an
  assignment;
* hand-computed passes, including an exact tie, on 1-d examples;
* token_order is the unique stable sort by cluster (properties, C4);
* reordering is exact at tau = 1, lambda = -inf (attention is permutation
  equivariant, so the result is dense attention), and one cluster per side
  is the identity order (C5).
"""
import math
import warnings

import numpy as np
import pytest

import oracle as O

scipy_vq = pytest.importorskip("scipy.cluster.vq")


def rand(seed, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return scale * rng.standard_normal((n, d))


def blobs(seed, n, d, k, spread=0.3):
    rng = np.random.default_rng(seed)
    centres = 2.0 * rng.standard_normal((k, d))
    lab = rng.integers(0, k, n)
    return centres[lab] + spread * rng.standard_normal((n, d))


def test_quadratic_form_is_the_mean_logit_change():
    Q, K = rand(1, 40, 6), rand(2, 70, 6)
    sm = 1.0 / math.sqrt(6)
    Mk = O.metric_matrix(Q, K, "q", "interaction")
    Mq = O.metric_matrix(Q, K, "k", "interaction")
    rng = np.random.default_rng(3)
    for _ in range(5):
        x, c = Q[rng.integers(40)], rng.standard_normal(6)
        brute = np.mean([(sm * (x - c) @ k) ** 2 for k in K])
        assert abs(brute - sm * sm * (x - c) @ Mk @ (x - c)) < 1e-12
        y, e = K[rng.integers(70)], rng.standard_normal(6)
        brute = np.mean([(sm * q @ (y - e)) ** 2 for q in Q])
        assert abs(brute - sm * sm * (y - e) @ Mq @ (y - e)) < 1e-12
    assert np.array_equal(O.metric_matrix(Q, K, "q", "feature"), np.eye(6))


def test_quad_dist_direct():
    X, c = rand(4, 30, 5), rand(5, 7, 5)
    A = rand(6, 5, 5)
    M = A @ A.T + 0.1 * np.eye(5)
    D = O.quad_dist(X, c, M)
    for n in range(30):
        for m in range(7):
            r = X[n] - c[m]
            assert abs(D[n, m] - r @ M @ r) <= 1e-12 * (1 + abs(r @ M @ r))


@pytest.mark.parametrize("seed,n,d,C,T", [(7, 300, 4, 6, 1), (8, 500, 8, 10, 5),
                                          (9, 257, 3, 17, 8), (10, 64, 2, 64, 3)])
def test_feature_metric_is_lloyd(seed, n, d, C, T):
    X = blobs(seed, n, d, max(2, C // 2))
    ours = O.cluster_tokens(X, C, T, np.eye(d))
    init = X[O.seeds(n, C)].copy()
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        _, ref = scipy_vq.kmeans2(X, init, iter=T, minit="matrix", missing="warn")
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("seed,n,d,C,T", [(11, 400, 6, 8, 4), (12, 333, 5, 12, 6)])
def test_interaction_metric_is_lloyd_on_whitened_tokens(seed, n, d, C, T):
    Q = blobs(seed, n, d, 5)
    K = blobs(seed + 100, n, d, 5) @ np.diag(np.linspace(0.3, 2.0, d))
    for side, X in (("q", Q), ("k", K)):
        M = O.metric_matrix(Q, K, side, "interaction")
        L = np.linalg.cholesky(M)
        ours = O.cluster_tokens(X, C, T, M)
        Xw = X @ L
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            _, ref = scipy_vq.kmeans2(Xw, Xw[O.seeds(n, C)].copy(), iter=T, minit="matrix",
                                      missing="warn")
        assert np.array_equal(ours, ref), side


def test_lloyd_objective_never_increases():
    Q, K = blobs(13, 600, 8, 6), rand(14, 600, 8)
    for metric in ("feature", "interaction"):
        M = O.metric_matrix(Q, K, "q", metric)
        _, hist = O.cluster_tokens(Q, 20, 6, M, history=True)
        prev = None
        for c, lab in hist:
            D = O.quad_dist(Q, c, M)
            J = D[np.arange(600), lab].sum()
            if prev is not None:
                c_prev, lab_prev = prev
                J_before = O.quad_dist(Q, c_prev, M)[np.arange(600), lab_prev].sum()
                J_upd = D[np.arange(600), lab_prev].sum()   # new centroids, old labels
                assert J_upd <= J_before * (1 + 1e-12)
                assert J <= J_upd * (1 + 1e-12)
            prev = (c, lab)


def test_hand_example():
    """d = 1, C = 2.  Seeds: tokens floor(6/4) = 1 and floor(18/4) = 4, the
    values 0.1 and 0.2.  Pass 1: 0 and 0.1 go to 0.1, the rest to 0.2.  Means
    0.05 and (5 + 5.2 + 0.2 + 5.1) / 4 = 3.875.  Pass 2 moves 0.2 to cluster
    0."""
    X = np.array([[0.0], [0.1], [5.0], [5.2], [0.2], [5.1]])
    assert list(O.seeds(6, 2)) == [1, 4]
    l1, hist = O.cluster_tokens(X, 2, 1, np.eye(1), history=True)
    assert list(l1) == [0, 0, 1, 1, 1, 1]
    l2, hist = O.cluster_tokens(X, 2, 2, np.eye(1), history=True)
    assert np.allclose(hist[1][0][:, 0], [0.05, 3.875])
    assert list(l2) == [0, 0, 1, 1, 0, 1]
    assert list(O.token_order(l2)) == [0, 1, 4, 2, 3, 5]
    # a positive scalar metric scales every distance alike: same labels
    assert list(O.cluster_tokens(X, 2, 2, np.array([[3.7]]))) == [0, 0, 1, 1, 0, 1]


def test_exact_tie_goes_to_the_smaller_cluster():
    X = np.array([[0.0], [1.0], [2.0]])      # seed tokens 0 and 2: centroids 0 and 2
    assert list(O.seeds(3, 2)) == [0, 2]
    assert list(O.cluster_tokens(X, 2, 1, np.eye(1))) == [0, 0, 1]
    assert list(O.cluster_tokens(X, 2, 1, np.array([[0.5]]))) == [0, 0, 1]


def test_token_order_is_the_stable_sort():
    rng = np.random.default_rng(15)
    for C in (1, 3, 50):
        lab = rng.integers(0, C, 777)
        perm = O.token_order(lab, C)
        assert sorted(perm.tolist()) == list(range(777))
        sl = lab[perm]
        assert np.all(np.diff(sl) >= 0)
        same = np.diff(sl) == 0
        assert np.all(np.diff(perm)[same] > 0)
    # an empty cluster in the middle leaves no gap
    assert list(O.token_order(np.array([2, 0, 2, 0]), 3)) == [1, 3, 0, 2]


@pytest.mark.parametrize("metric", ["feature", "interaction"])
def test_reordered_dense_is_dense_attention(metric):
    rng = np.random.default_rng(16)
    N, d = 300, 16
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    p = O.Params(BQ=32, BK=16, G=8, tau=1.0, lam=-math.inf)
    cp = O.ClusterParams(clusters_q=5, clusters_k=9, iters=3, metric=metric)
    r = O.reordered_head(Q, K, V, p, cp)
    assert not np.array_equal(r["perm_q"], np.arange(N))
    Od, lsed = O.dense_attention_head(Q, K, V, p.sm(d), False)
    np.testing.assert_allclose(r["O"], Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lsed, rtol=0, atol=1e-12)


def test_one_cluster_is_the_identity_order():
    rng = np.random.default_rng(17)
    N, d = 200, 8
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    p = O.Params(BQ=32, BK=16, G=8, tau=0.8, lam=-2.0)
    cp = O.ClusterParams(clusters_q=1, clusters_k=1, iters=2)
    r = O.reordered_head(Q, K, V, p, cp)
    assert np.array_equal(r["perm_q"], np.arange(N))
    ref = O.oracle_head(Q, K, V, p)
    assert np.array_equal(r["O"], ref["O"])
    assert all(np.array_equal(a, b) for a, b in zip(r["kept"], ref["kept"]))


def test_reordered_sparse_moves_rows_back():
    """Under a sparse mask the reordered result is the plain pipeline on the
    permuted tokens, scattered back: check on rows the pipeline itself
    computes, by running the plain oracle on explicitly permuted inputs."""
    rng = np.random.default_rng(18)
    N, d = 256, 8
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    p = O.Params(BQ=32, BK=16, G=8, tau=0.7, lam=-3.0)
    pq, pk = rng.permutation(N), rng.permutation(N)
    Or, lser, sk, kept = O.reordered_attention_head(Q, K, V, p, pq, pk)
    ref = O.oracle_head(Q[pq], K[pk], V[pk], p)
    for r in range(N):
        assert np.array_equal(Or[pq[r]], ref["O"][r])
        assert lser[pq[r]] == ref["lse"][r]
    with pytest.raises(ValueError):
        O.reordered_attention_head(Q, K, V, O.Params(causal=True), pq, pk)

"""CPU pins of the oracle's recall skip rule (skip_rule = "recall").

The rule (oracle O8'): per row, d = energy dropped so far and l = energy
seen so far over the kept tiles, both relative to the running max; a group
skips tile t's P.V when every row has d + E_t <= (1 - rho) l_t.

Pinned against things other than the oracle's online bookkeeping:
* a scale-free re-statement: every energy taken relative to the row's
  maximum over all its kept tiles (no running max, no rescaling of d or l),
  the decisions made on those sums -- decisions and outputs must agree;
* the recall guarantee it is built for: for every row, dropped / seen
  <= 1 - rho over the kept tiles;
* a closed-form bound on the output: dropping a share s of the energy moves
  O by at most s * max|V| from the no-skip result;
* rho = 1 drops only groups with no visible key in the tile, so the output
  equals lambda = -inf exactly;
* a hand-computed two-tile example (one query, logits 0, 0 | -1, -1).
"""
import math

import numpy as np
import pytest

import oracle as O


def rand_qkv(seed, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((n, d)), scale * rng.standard_normal((n, d)),
            rng.standard_normal((n, d)))


def scale_free(Q, K, V, kept, p):
    """The recall rule restated without a running max: for row r, every
    logit is taken relative to M_r = its maximum over all kept tiles."""
    N, d = Q.shape
    sm = p.sm(d)
    ng = (p.BQ + p.G - 1) // p.G
    Oout = np.zeros((N, d))
    skips, shares = [], np.zeros(N)
    for i, lst in enumerate(kept):
        rows = np.arange(i * p.BQ, min(N, (i + 1) * p.BQ))
        nr = len(rows)
        tiles = []
        for j in lst:
            cols = np.arange(j * p.BK, min(N, (j + 1) * p.BK))
            S = sm * (Q[rows] @ K[cols].T)
            if p.causal:
                S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
            tiles.append((cols, S))
        M = np.full(nr, -np.inf)
        for _, S in tiles:
            M = np.maximum(M, S.max(axis=1))
        Ms = np.where(np.isfinite(M), M, 0.0)
        seen = np.zeros(nr)
        dropped = np.zeros(nr)
        num = np.zeros((nr, d))
        sk = np.zeros((len(lst), ng), dtype=bool)
        for t, (cols, S) in enumerate(tiles):
            e = np.where(np.isfinite(S), np.exp(S - Ms[:, None]), 0.0)
            E = e.sum(axis=1)
            seen = seen + E
            for g in range(ng):
                gr = slice(g * p.G, min(nr, (g + 1) * p.G))
                if gr.start >= nr:
                    sk[t, g] = True
                    continue
                ok = dropped[gr] + E[gr] <= (1.0 - p.recall) * seen[gr]
                sk[t, g] = bool(ok.all())
                if sk[t, g]:
                    dropped[gr] += E[gr]
                else:
                    num[gr] += e[gr] @ V[cols]
        skips.append(sk)
        good = seen > 0
        Oout[rows[good]] = num[good] / seen[good, None]
        shares[rows[good]] = dropped[good] / seen[good]
    return Oout, skips, shares


CASES = [
    # seed, N, d, BQ, BK, G, causal, tau, rho
    (11, 150, 8, 32, 16, 8, False, 0.9, 0.95),
    (12, 200, 6, 32, 8, 16, True, 0.95, 0.9),
    (13, 97, 4, 16, 8, 4, False, 1.0, 0.8),
    (14, 256, 8, 64, 16, 32, True, 0.85, 0.99),
    (15, 120, 5, 32, 16, 32, False, 0.9, 0.5),
]


@pytest.mark.parametrize("case", CASES)
def test_recall_rule_matches_scale_free_statement(case):
    seed, N, d, BQ, BK, G, causal, tau, rho = case
    q, k, v = rand_qkv(seed, N, d, scale=1.5)
    p = O.Params(BQ=BQ, BK=BK, G=G, causal=causal, tau=tau, skip_rule="recall", recall=rho)
    kept = O.predict_head(q, k, p)["kept"]
    stats = []
    Oo, _, sko = O.sparse_attention_head(q, k, v, kept, p, deltas=stats)
    Ob, skb, shares = scale_free(q, k, v, kept, p)
    n_skip = 0
    for i in range(len(kept)):
        near = np.abs(stats[i]) <= 1e-9
        assert np.array_equal(sko[i][~near], skb[i][~near]), f"block {i}"
        assert not near.any()          # no decision this close to the boundary here
        n_skip += int(sko[i].sum())
    np.testing.assert_allclose(Oo, Ob, rtol=0, atol=1e-12)
    # the guarantee: recall >= rho on every row
    assert np.all(shares <= 1.0 - rho + 1e-12)
    if rho < 1.0:
        assert n_skip > 0              # the cases exercise the rule


@pytest.mark.parametrize("case", CASES)
def test_recall_output_bound(case):
    seed, N, d, BQ, BK, G, causal, tau, rho = case
    q, k, v = rand_qkv(seed, N, d, scale=1.5)
    p = O.Params(BQ=BQ, BK=BK, G=G, causal=causal, tau=tau, skip_rule="recall", recall=rho)
    p0 = O.Params(BQ=BQ, BK=BK, G=G, causal=causal, tau=tau, lam=-math.inf)
    kept = O.predict_head(q, k, p)["kept"]
    Or, _, _ = O.sparse_attention_head(q, k, v, kept, p)
    On, _, _ = O.sparse_attention_head(q, k, v, kept, p0)
    _, _, shares = scale_free(q, k, v, kept, p)
    vmax = np.abs(v).max()
    # O_skip - O_full = -(sum over dropped P V) / l, |.| <= share * max|V|
    dev = np.abs(Or - On).max(axis=1)
    assert np.all(dev <= shares * vmax + 1e-12)
    assert np.all(dev <= (1.0 - rho) * vmax + 1e-12)


def test_recall_one_drops_nothing_visible():
    for causal in (False, True):
        q, k, v = rand_qkv(21, 180, 8)
        p = O.Params(BQ=32, BK=16, G=8, causal=causal, tau=0.9, skip_rule="recall", recall=1.0)
        p0 = O.Params(BQ=32, BK=16, G=8, causal=causal, tau=0.9, lam=-math.inf)
        kept = O.predict_head(q, k, p)["kept"]
        Or, lr, skr = O.sparse_attention_head(q, k, v, kept, p)
        On, ln, _ = O.sparse_attention_head(q, k, v, kept, p0)
        np.testing.assert_array_equal(Or, On)
        np.testing.assert_array_equal(lr, ln)
        # a skip at rho = 1 only where the whole group sees no key of the tile
        N = 180
        for i, lst in enumerate(kept):
            rows = np.arange(i * 32, min(N, (i + 1) * 32))
            for t, j in enumerate(lst):
                cols = np.arange(j * 16, min(N, (j + 1) * 16))
                for g in range(4):
                    gr = rows[g * 8:(g + 1) * 8]
                    visible = len(gr) > 0 and (not causal or (cols[None, :] <= gr[:, None]).any())
                    assert skr[i][t, g] == (not visible)


def test_recall_hand_example():
    """One query (d = 1, sm = 1), keys 0, 0 | -1, -1 in two tiles of 2: the
    first tile holds energy 2, the second 2/e, a share (2/e) / (2 + 2/e) =
    0.26894 of the total.  rho = 0.75 keeps it, rho = 0.7 drops it."""
    Q = np.array([[1.0]])
    K = np.array([[0.0], [0.0], [-1.0], [-1.0]])
    V = np.array([[1.0], [3.0], [10.0], [20.0]])
    Qp = np.vstack([Q, np.zeros((3, 1))])       # 4 rows: the query + 3 padding rows
    share = (2 / math.e) / (2 + 2 / math.e)
    assert abs(share - 0.2689414) < 1e-6
    for rho, dropped in ((0.75, False), (0.7, True)):
        p = O.Params(BQ=1, BK=2, G=1, causal=False, tau=1.0, skip_rule="recall", recall=rho)
        kept = [np.array([0, 1])] + [np.array([0, 1])] * 3
        Oo, lse, sk = O.sparse_attention_head(Qp, K, V, kept, p)
        assert not sk[0][0, 0]                      # the first tile is always kept
        assert sk[0][1, 0] == dropped
        total = 2 + 2 / math.e
        if dropped:
            want = (1.0 + 3.0) / total              # l still counts the dropped energy
        else:
            want = (1.0 + 3.0 + (10.0 + 20.0) / math.e) / total
        assert abs(Oo[0, 0] - want) < 1e-14
        assert abs(lse[0] - math.log(total)) < 1e-14


def test_recall_rule_in_the_quantised_oracle():
    """The quantised stage two applies the same rule: with its own logits
    and P, its decisions must match a scale-free pass over those logits."""
    q, k, v = rand_qkv(31, 160, 16, scale=2.0)
    p = O.Params(BQ=32, BK=16, G=8, tau=0.9, skip_rule="recall", recall=0.9)
    kept = O.predict_head(q, k, p)["kept"]
    stats = []
    _, _, sk = O.sparse_attention_quant_head(q, k, v, kept, p, deltas=stats)
    # logits of the quantised path, rebuilt from the quantisers
    qc, qs = O.int8_quantize_blocks(q, 32)
    kc, ks = O.int8_quantize_blocks(k, 16)
    sm = p.sm(16)
    n_skip = 0
    for i, lst in enumerate(kept):
        rows = np.arange(i * 32, min(160, (i + 1) * 32))
        Ss = []
        for j in lst:
            cols = np.arange(j * 16, min(160, (j + 1) * 16))
            Ss.append(sm * float(qs[i]) * float(ks[j]) *
                      (qc[rows].astype(np.int64) @ kc[cols].astype(np.int64).T))
        M = np.max([S.max(axis=1) for S in Ss], axis=0)
        seen = np.zeros(len(rows))
        dropped = np.zeros(len(rows))
        for t, S in enumerate(Ss):
            E = np.exp(S - M[:, None]).sum(axis=1)
            seen += E
            for g in range(4):
                gr = slice(8 * g, 8 * g + 8)
                want = bool((dropped[gr] + E[gr] <= 0.1 * seen[gr]).all())
                if abs(stats[i][t, g]) > 1e-9:
                    assert sk[i][t, g] == want
                if sk[i][t, g]:
                    dropped[gr] += E[gr]
                    n_skip += 1
    assert n_skip > 0

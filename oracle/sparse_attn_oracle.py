"""fp64 CPU oracle: block-mean pooled predictor, cumulative-mass mask and
block-sparse attention with the softmax-aware skip.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain, slow, step by
step, in float64, for one (batch, head) at a time.  Inputs are the exact
values the GPU sees (bf16- or fp32-representable), widened to float64.

Notation: N tokens, head dimension d, query blocks of BQ rows (R_i), key
blocks of BK rows (C_j, n_j = |C_j|), sm the softmax scale, tau the
cumulative-mass target, lambda the skip threshold, G the rows per skip
group.

Steps and the passages they follow
----------------------------------
O1 pool          SpargeAttn abstract, stage one ("predict the attention map"
                 quickly); iCATS abstract (prior work groups query and key
                 tokens independently to estimate scores).  Reading: a group
                 is a contiguous block; its representative is the mean of its
                 valid rows (a partial last block averages only real rows).
O2 admissible    Reading: non-causal keeps every key block; causal drops key
                 blocks that lie wholly in the future of the query block
                 before anything is normalised.
O3 scores        Reading: s_ij = sm * <qbar_i, kbar_j>, sm = 1/sqrt(d) unless
                 given; the same scale as the attention logits.
O4 weights       iCATS abstract ("top-p rule"); DynSparse story (cumulative
                 energy).  Reading: top-cdf = softmax of s_i. over the
                 admissible blocks; energy = n_j * exp(s_ij - max) normalised
                 (each block weighted by its estimated total energy).
O5 forced        Reading: the first ``keep_prefix_kblocks`` key blocks, and
                 under causality the key blocks that touch the query block's
                 diagonal, are always kept (every row then sees a key).
O6 order         Reading: forced first, then s descending, then j ascending
                 (a total order on the admissible blocks).
O7 cut           DynSparse story (recall target); iCATS abstract (top-p).
                 Reading: keep the shortest prefix of that order whose fp64
                 cumulative weight reaches tau (inclusive), never fewer than
                 the forced blocks; tau >= 1, or a prefix that never reaches
                 tau by rounding, keeps every admissible block.  The kept
                 list keeps this order; attention processes it in this order.
O7' top-k        DynSparse story (top-k fixes a computational budget but
                 relaxes accuracy, the comparator of top-p).  Reading (rule =
                 "topk"): keep the first min(|A_i|, max(|F_i|, k)) blocks of
                 the same processing order; P-hat is the top-cdf softmax.
O8 attention     SpargeAttn abstract, stage two (an online softmax-aware
                 filter that costs nothing extra and skips more products).
                 Reading: flash-attention online softmax over the kept list;
                 for each group of G consecutive rows of the query block,
                 delta_g = max over its rows of (local max - new running
                 max); the P.V product of that tile is skipped for the group
                 when delta_g < lambda (natural-log units, strict).  A
                 skipped tile still updates m and l.  Rows with no visible
                 key in the tile contribute -inf to delta_g.
O8' recall skip  DynSparse story ("training-free sparse attention based on
                 cumulative energy filtering": a fixed recall suffices for
                 accuracy, a static threshold is suboptimal, and the dynamic
                 threshold comes from the cumulative energy of the selected
                 tokens, which the flash-attention operator already holds).
                 Reading (skip_rule = "recall", target recall rho): each row
                 keeps, next to l, the energy d it has dropped so far, both
                 relative to the same running max.  For tile t with energy
                 E_r = sum_c exp(S_rc - m_r) and l_r already updated with it,
                 row r may drop the tile when d_r + E_r <= (1 - rho) l_r; the
                 group skips P.V when every row may, and then d_r += E_r.  So
                 for every row the dropped share of the energy over the kept
                 tiles stays <= 1 - rho at every step (recall >= rho).  Rows
                 with no visible key in the tile (E_r = 0) never block a skip.
O10 dense        Plain softmax(sm * Q K^T [+ causal mask]) V, the exact
                 reference for rel-L1 and for the tau=1, lambda=-inf identity.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np


@dataclasses.dataclass
class Params:
    """Problem parameters, mirroring the C-ABI parameter block.

    ``tau``, ``lam`` and ``sm_scale`` are the float32 values the library
    receives; the oracle widens them to float64 exactly.
    """
    BQ: int = 128
    BK: int = 64
    causal: bool = False
    tau: float = 0.95
    lam: float = -math.inf
    sm_scale: float = 0.0          # 0 -> 1/sqrt(d)
    rule: str = "topcdf"           # "topcdf" | "energy" | "topk"
    keep_prefix_kblocks: int = 0
    G: int = 32                    # rows per skip group
    skip_rule: str = "lambda"      # "lambda" (O8) | "recall" (O8')
    recall: float = 1.0            # rho of the recall rule
    topk_blocks: int = 0           # budget of the "topk" rule

    def sm(self, d: int) -> float:
        return float(self.sm_scale) if self.sm_scale else 1.0 / math.sqrt(d)


def n_blocks(N: int, bs: int) -> int:
    return (N + bs - 1) // bs


def _rows(i: int, bs: int, N: int) -> range:
    return range(i * bs, min(N, (i + 1) * bs))


# --------------------------------------------------------------------- O1
def pool_means(X: np.ndarray, bs: int) -> np.ndarray:
    """O1: mean of each contiguous block of ``bs`` rows (valid rows only)."""
    X = np.asarray(X, dtype=np.float64)
    N, d = X.shape
    nb = n_blocks(N, bs)
    out = np.empty((nb, d), dtype=np.float64)
    for b in range(nb):
        r = _rows(b, bs, N)
        out[b] = X[r.start:r.stop].sum(axis=0) / len(r)
    return out


# --------------------------------------------------------------------- O2
def admissible_blocks(N: int, BQ: int, BK: int, causal: bool) -> np.ndarray:
    """O2: bool [NQB, NKB]; causal keeps key blocks whose first key is not
    after the query block's last row."""
    nqb, nkb = n_blocks(N, BQ), n_blocks(N, BK)
    adm = np.ones((nqb, nkb), dtype=bool)
    if causal:
        for i in range(nqb):
            last_row = _rows(i, BQ, N)[-1]
            for j in range(nkb):
                adm[i, j] = j * BK <= last_row
    return adm


# --------------------------------------------------------------------- O3
def block_scores(qbar: np.ndarray, kbar: np.ndarray, sm: float) -> np.ndarray:
    """O3: s_ij = sm * qbar_i . kbar_j  (all pairs; callers mask)."""
    return sm * (qbar @ kbar.T)


# --------------------------------------------------------------------- O4
def block_weights(s: np.ndarray, adm: np.ndarray, rule: str,
                  n_k: np.ndarray) -> np.ndarray:
    """O4: predicted block mass P-hat [NQB, NKB], 0 outside the admissible
    set.  top-cdf (and top-k, which only changes the cut): softmax of s over
    admissible j.  energy: weights n_j * exp(s_ij - max) normalised."""
    P = np.zeros_like(s)
    for i in range(s.shape[0]):
        a = adm[i]
        si = s[i, a]
        w = np.exp(si - si.max())
        if rule == "energy":
            w = w * n_k[a]
        elif rule not in ("topcdf", "topk"):
            raise ValueError(rule)
        P[i, a] = w / w.sum()
    return P


# --------------------------------------------------------------------- O5
def forced_blocks(N: int, BQ: int, BK: int, causal: bool, keep_prefix: int,
                  adm: np.ndarray) -> np.ndarray:
    """O5: bool [NQB, NKB] of always-kept blocks (a subset of adm)."""
    nqb, nkb = adm.shape
    F = np.zeros_like(adm)
    F[:, :min(keep_prefix, nkb)] = True
    if causal:
        for i in range(nqb):
            first_row = _rows(i, BQ, N)[0]
            for j in range(nkb):
                last_key = _rows(j, BK, N)[-1]
                if last_key >= first_row:
                    F[i, j] = True
    return F & adm


# --------------------------------------------------------------------- O6
def processing_order(s_row: np.ndarray, adm_row: np.ndarray,
                     forced_row: np.ndarray) -> np.ndarray:
    """O6: admissible j sorted by (forced first, s descending, j ascending)."""
    js = [j for j in range(len(s_row)) if adm_row[j]]
    js.sort(key=lambda j: (0 if forced_row[j] else 1, -s_row[j], j))
    return np.array(js, dtype=np.int64)


# --------------------------------------------------------------------- O7
def cut_length(p_in_order: np.ndarray, n_forced: int, tau: float) -> int:
    """O7: number of kept blocks: the shortest prefix whose running fp64 sum
    reaches tau, at least n_forced; tau >= 1 or no such prefix keeps all."""
    n = len(p_in_order)
    if tau >= 1.0:
        return n
    c = 0.0
    for k in range(n):
        c += float(p_in_order[k])
        if c >= tau:
            return max(n_forced, k + 1)
    return n


def predict_head(Q: np.ndarray, K: np.ndarray, p: Params) -> dict:
    """Stage one for one head: O1..O7.  Returns the kept lists (in
    processing order), the predicted map, scores and sets."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return predict_from_means(pool_means(Q, p.BQ), pool_means(K, p.BK), Q.shape[0], p)


def predict_from_means(qbar: np.ndarray, kbar: np.ndarray, N: int, p: Params) -> dict:
    """Stage one after pooling, O2..O7, for block means given as input (the
    oracle's own, or another implementation's, to check the later steps on
    their own)."""
    qbar = np.asarray(qbar, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    d = qbar.shape[1]
    adm = admissible_blocks(N, p.BQ, p.BK, p.causal)
    s = block_scores(qbar, kbar, p.sm(d))
    nkb = kbar.shape[0]
    n_k = np.array([len(_rows(j, p.BK, N)) for j in range(nkb)], dtype=np.float64)
    P = block_weights(s, adm, p.rule, n_k)
    F = forced_blocks(N, p.BQ, p.BK, p.causal, p.keep_prefix_kblocks, adm)
    kept: List[np.ndarray] = []
    orders: List[np.ndarray] = []
    for i in range(s.shape[0]):
        order = processing_order(s[i], adm[i], F[i])
        if p.rule == "topk":        # O7': a fixed budget in the same order
            k = min(len(order), max(int(F[i].sum()), int(p.topk_blocks)))
        else:
            k = cut_length(P[i, order], int(F[i].sum()), float(p.tau))
        orders.append(order)
        kept.append(order[:k])
    return dict(qbar=qbar, kbar=kbar, s=s, P=P, adm=adm, forced=F,
                order=orders, kept=kept)


# --------------------------------------------------------------------- O8
def group_skip(p: Params, gr: slice, nr: int, delta_r: np.ndarray, E: np.ndarray,
               l: np.ndarray, drop: np.ndarray):
    """The skip decision of one row group for one tile, and its statistic.

    lambda (O8): stat = delta_g = max over the group's rows of
    (local max - new running max); skip when stat < lambda.
    recall (O8'): stat = min over the group's rows of the relative slack
    ((1 - rho) l_r - d_r - E_r) / l_r (+inf for a row with l_r = 0); skip
    when stat >= 0.  ``drop`` holds d_r, already rescaled to the new max.
    """
    if p.skip_rule == "lambda":
        dg = float(delta_r[gr].max()) if gr.start < nr else -np.inf
        return bool(dg < float(p.lam)), dg
    if gr.start >= nr:
        return True, np.inf
    if p.skip_rule != "recall":
        raise ValueError(p.skip_rule)
    omr = 1.0 - float(p.recall)
    lg, dg, eg = l[gr], drop[gr], E[gr]
    slack = np.where(lg > 0, (omr * lg - dg - eg) / np.where(lg > 0, lg, 1.0), np.inf)
    st = float(slack.min())
    return bool(st >= 0.0), st


def sparse_attention_head(Q, K, V, kept: List[np.ndarray], p: Params,
                          force_skip: Optional[List[np.ndarray]] = None,
                          deltas: Optional[list] = None):
    """O8: block-sparse online-softmax attention with the per-group skip.

    ``kept[i]`` lists key blocks for query block i in processing order.
    ``force_skip[i]`` (bool [len(kept[i]), n_groups]) replaces the skip
    decision when given (and the recall rule's dropped energy follows the
    forced decisions).  If ``deltas`` is a list, the group statistics of
    ``group_skip`` (float [len(kept[i]), n_groups]) are appended to it.  Returns
    (O [N,d], lse [N] natural log, skips: list of bool
    [len(kept[i]), n_groups]).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    sm = p.sm(d)
    n_groups = (p.BQ + p.G - 1) // p.G
    O = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    skips = []
    for i, lst in enumerate(kept):
        rows = np.arange(i * p.BQ, min(N, (i + 1) * p.BQ))
        nr = len(rows)
        m = np.full(nr, -np.inf)
        l = np.zeros(nr)
        acc = np.zeros((nr, d))
        drop = np.zeros(nr)
        sk = np.zeros((len(lst), n_groups), dtype=bool)
        dl = np.full((len(lst), n_groups), -np.inf)
        for t, j in enumerate(lst):
            cols = np.arange(j * p.BK, min(N, (j + 1) * p.BK))
            S = sm * (Q[rows] @ K[cols].T)
            if p.causal:
                S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
            mloc = S.max(axis=1)
            mnew = np.maximum(m, mloc)
            alpha = np.ones(nr)
            moved = np.isfinite(mnew) & (m != mnew)
            alpha[moved] = np.exp(m[moved] - mnew[moved])   # exp(-inf) = 0
            safe = np.where(np.isfinite(mnew), mnew, 0.0)
            P = np.where(np.isfinite(S), np.exp(S - safe[:, None]), 0.0)
            E = P.sum(axis=1)
            l = alpha * l + E
            drop = alpha * drop
            acc = alpha[:, None] * acc
            delta_r = np.where(np.isfinite(mloc), mloc - safe, -np.inf)
            for g in range(n_groups):
                gr = slice(g * p.G, min(nr, (g + 1) * p.G))
                skip, dl[t, g] = group_skip(p, gr, nr, delta_r, E, l, drop)
                if force_skip is not None:
                    skip = bool(force_skip[i][t, g])
                sk[t, g] = skip
                if gr.start < nr:
                    if skip:
                        drop[gr] += E[gr]
                    else:
                        acc[gr] += P[gr] @ V[cols]
            m = mnew
        skips.append(sk)
        if deltas is not None:
            deltas.append(dl)
        ok = l > 0
        O[rows[ok]] = acc[ok] / l[ok, None]
        lse[rows[ok]] = m[ok] + np.log(l[ok])
    return O, lse, skips


# -------------------------------------------------------------------- O10
def dense_attention_head(Q, K, V, sm: float, causal: bool,
                         rows: Optional[np.ndarray] = None, chunk: int = 128):
    """O10: softmax(sm * Q K^T, causal mask) V in float64, for ``rows`` (all
    rows by default), computed in row chunks.  Returns (O, lse)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    if rows is None:
        rows = np.arange(N)
    O = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for c0 in range(0, len(rows), chunk):
        r = rows[c0:c0 + chunk]
        S = sm * (Q[r] @ K.T)
        if causal:
            S = np.where(np.arange(N)[None, :] > r[:, None], -np.inf, S)
        mx = S.max(axis=1, keepdims=True)
        E = np.exp(S - mx)
        den = E.sum(axis=1, keepdims=True)
        O[c0:c0 + chunk] = (E @ V) / den
        lse[c0:c0 + chunk] = mx[:, 0] + np.log(den[:, 0])
    return O, lse


def oracle_head(Q, K, V, p: Params, force_kept=None, force_skip=None):
    """Stage one then stage two for one head.  ``force_kept`` replaces the
    oracle's own kept lists (to evaluate stage two under another mask)."""
    pred = predict_head(Q, K, p)
    kept = pred["kept"] if force_kept is None else force_kept
    O, lse, skips = sparse_attention_head(Q, K, V, kept, p, force_skip)
    return dict(pred=pred, O=O, lse=lse, skips=skips, kept=kept)

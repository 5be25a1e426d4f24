"""Token reordering predictor -- TEST INFRASTRUCTURE ONLY (see the package
docstring): fp64, plain, one (batch, head) at a time.

Query and key tokens are clustered, each side is reordered so that a
cluster's tokens sit next to each other, and the block-sparse pipeline (O1 to
O8) runs unchanged on the reordered tokens; the output rows go back to their
original positions.

Steps and the passages they follow
----------------------------------
C1 metric    iCATS abstract (arxivdaily.com page): scores are estimated from
             groups of tokens; grouping query and key tokens independently by
             feature similarity (prior work) is less accurate than grouping
             by the query-key dot-product interaction, and that objective
             reduces to a simple quadratic form.  Reading: replacing a query
             x by a representative c moves its logit with key k by
             sm * (x - c) . k; over the N keys the mean squared move is
             sm^2 (x - c)^T M_K (x - c) with M_K = K^T K / N, the keys'
             second-moment matrix.  So queries cluster under the quadratic
             form of M_K and keys under that of M_Q = Q^T Q / N
             ("interaction"); "feature" uses M = I, the prior-work baseline.
C2 seeds     Reading: centroid m of C starts at the token floor((2m+1) N /
             (2C)), evenly spaced over the sequence (deterministic).
C3 passes    Reading: T assignment passes of Lloyd's iteration.  A pass gives
             every token the cluster m minimising (x - c_m)^T M (x - c_m),
             ties to the smaller m.  Between passes every centroid becomes
             the mean of its members; a cluster without members keeps its
             centroid.
C4 order     iCATS abstract (a tail-merging strategy against the padding
             that irregular cluster sizes would cost); PARO abstract on the
             huggingface-mirror search page (reordering tokens turns the
             attention pattern block-wise).  Reading: tokens sorted by
             (cluster, position); the clusters are packed back to back with
             no padding, and the fixed BQ / BK blocks are cut from the
             reordered sequence, so the tail of one cluster shares a block
             with the head of the next.
C5 attention Reading: stage one and stage two run unchanged on Q[perm_q],
             K[perm_k], V[perm_k]; row r of their output is row perm_q[r] of
             O.  Causal attention is not reordered: its mask is defined on the
             original positions.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .sparse_attn_oracle import Params, predict_head, sparse_attention_head


@dataclasses.dataclass
class ClusterParams:
    """Mirrors the C-ABI cluster parameter block."""
    clusters_q: int = 256
    clusters_k: int = 512
    iters: int = 4
    metric: str = "interaction"    # "interaction" | "feature"


# --------------------------------------------------------------------- C1
def second_moment(X: np.ndarray) -> np.ndarray:
    """X^T X / N in float64."""
    X = np.asarray(X, dtype=np.float64)
    return (X.T @ X) / X.shape[0]


def metric_matrix(Q: np.ndarray, K: np.ndarray, side: str, metric: str) -> np.ndarray:
    """The matrix of the quadratic form that clusters ``side`` ("q" or "k")."""
    d = np.asarray(Q).shape[1]
    if metric == "feature":
        return np.eye(d)
    if metric != "interaction":
        raise ValueError(metric)
    return second_moment(K if side == "q" else Q)


def quad_dist(X: np.ndarray, c: np.ndarray, M: np.ndarray) -> np.ndarray:
    """D[x, m] = (x - c_m)^T M (x - c_m) for every token and centroid,
    through the expansion x^T M x - 2 x^T M c_m + c_m^T M c_m."""
    X = np.asarray(X, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    xm = ((X @ M) * X).sum(axis=1)
    cm = ((c @ M) * c).sum(axis=1)
    return xm[:, None] - 2.0 * (X @ M @ c.T) + cm[None, :]


# --------------------------------------------------------------------- C2
def seeds(N: int, C: int) -> np.ndarray:
    """Token index of each initial centroid."""
    return np.array([((2 * m + 1) * N) // (2 * C) for m in range(C)], dtype=np.int64)


# --------------------------------------------------------------------- C3
def assign(X: np.ndarray, c: np.ndarray, M: np.ndarray):
    """One assignment: (labels, D).  np.argmin takes the first minimum, so
    ties go to the smaller cluster index."""
    D = quad_dist(X, c, M)
    return np.argmin(D, axis=1).astype(np.int64), D


def update(X: np.ndarray, labels: np.ndarray, c_prev: np.ndarray) -> np.ndarray:
    """Centroids after a pass: the mean of each cluster's members; a cluster
    without members keeps its previous centroid."""
    X = np.asarray(X, dtype=np.float64)
    c = np.array(c_prev, dtype=np.float64, copy=True)
    for m in range(c.shape[0]):
        members = X[labels == m]
        if len(members):
            c[m] = members.mean(axis=0)
    return c


def cluster_tokens(X: np.ndarray, C: int, T: int, M: np.ndarray, history: bool = False):
    """C2 + C3: the labels of the last of T passes (and, with ``history``,
    the list of (centroids used, labels) of every pass)."""
    if T < 1:
        raise ValueError("at least one pass")
    X = np.asarray(X, dtype=np.float64)
    c = X[seeds(X.shape[0], C)].copy()
    hist = []
    labels = None
    for t in range(T):
        if t > 0:
            c = update(X, labels, c)
        labels, _ = assign(X, c, M)
        hist.append((c.copy(), labels.copy()))
    return (labels, hist) if history else labels


# --------------------------------------------------------------------- C4
def token_order(labels: np.ndarray, C: Optional[int] = None) -> np.ndarray:
    """perm[r] = the token at reordered position r: cluster 0's tokens in
    position order, then cluster 1's, and so on, with no padding."""
    labels = np.asarray(labels)
    C = int(labels.max()) + 1 if C is None else C
    parts = [np.nonzero(labels == m)[0] for m in range(C)]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


# --------------------------------------------------------------------- C5
def reorder_perms(Q: np.ndarray, K: np.ndarray, cp: ClusterParams):
    """(perm_q, perm_k, labels_q, labels_k) of C1..C4 for one head."""
    Mq = metric_matrix(Q, K, "q", cp.metric)
    Mk = metric_matrix(Q, K, "k", cp.metric)
    lq = cluster_tokens(Q, cp.clusters_q, cp.iters, Mq)
    lk = cluster_tokens(K, cp.clusters_k, cp.iters, Mk)
    return token_order(lq, cp.clusters_q), token_order(lk, cp.clusters_k), lq, lk


def reordered_attention_head(Q, K, V, p: Params, perm_q: np.ndarray, perm_k: np.ndarray,
                             force_kept: Optional[List[np.ndarray]] = None,
                             force_skip: Optional[List[np.ndarray]] = None,
                             deltas: Optional[list] = None):
    """C5 under given permutations: returns (O, lse, skips, kept) with O and
    lse in the original row order; kept and skips refer to the reordered
    blocks."""
    if p.causal:
        raise ValueError("causal attention is not reordered")
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Qp, Kp, Vp = Q[perm_q], K[perm_k], V[perm_k]
    kept = predict_head(Qp, Kp, p)["kept"] if force_kept is None else force_kept
    Op, lsep, skips = sparse_attention_head(Qp, Kp, Vp, kept, p, force_skip, deltas)
    O = np.empty_like(Op)
    lse = np.empty_like(lsep)
    O[perm_q] = Op
    lse[perm_q] = lsep
    return O, lse, skips, kept


def reordered_head(Q, K, V, p: Params, cp: ClusterParams):
    """C1..C5 for one head."""
    pq, pk, lq, lk = reorder_perms(Q, K, cp)
    O, lse, skips, kept = reordered_attention_head(Q, K, V, p, pq, pk)
    return dict(O=O, lse=lse, skips=skips, kept=kept, perm_q=pq, perm_k=pk,
                labels_q=lq, labels_k=lk)

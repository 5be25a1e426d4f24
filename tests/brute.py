"""Scalar brute-force reference for tiny inputs (pure Python loops).

Written independently of ``oracle/``: it imports nothing from there and uses
only ``math``.  It restates the same readings of the pages (block-mean
pooling, top-cdf / energy weights, forced-first order, shortest prefix
reaching tau, per-group skip of P.V when max(local max - new max) < lambda),
one scalar at a time, so that a slip in the vectorised oracle (an index, a
sign, a dropped term) shows up as a mismatch.
"""
from __future__ import annotations

import math


def nblk(n, b):
    return (n + b - 1) // b


def pool(X, bs):
    n, d = len(X), len(X[0])
    out = []
    for b in range(nblk(n, bs)):
        lo, hi = b * bs, min(n, (b + 1) * bs)
        row = []
        for c in range(d):
            s = 0.0
            for r in range(lo, hi):
                s += float(X[r][c])
            row.append(s / (hi - lo))
        out.append(row)
    return out


def predict(Q, K, BQ, BK, causal, tau, rule="topcdf", keep_prefix=0, sm=None):
    """Kept key-block lists, in processing order, for every query block."""
    n, d = len(Q), len(Q[0])
    if sm is None:
        sm = 1.0 / math.sqrt(d)
    qb, kb = pool(Q, BQ), pool(K, BK)
    nq, nk = len(qb), len(kb)
    lists = []
    for i in range(nq):
        first_row, last_row = i * BQ, min(n, (i + 1) * BQ) - 1
        cand = []
        for j in range(nk):
            first_key, last_key = j * BK, min(n, (j + 1) * BK) - 1
            if causal and first_key > last_row:
                continue
            s = 0.0
            for c in range(d):
                s += qb[i][c] * kb[j][c]
            s *= sm
            forced = j < keep_prefix or (causal and last_key >= first_row)
            cand.append([j, s, forced, last_key - first_key + 1])
        smax = max(c[1] for c in cand)
        tot = 0.0
        for c in cand:
            w = math.exp(c[1] - smax)
            if rule == "energy":
                w *= c[3]
            c.append(w)
            tot += w
        for c in cand:
            c[4] = c[4] / tot
        # selection sort with the explicit comparison rule
        rest = list(cand)
        order = []
        while rest:
            best = rest[0]
            for c in rest[1:]:
                if c[2] != best[2]:
                    better = c[2]
                elif c[1] != best[1]:
                    better = c[1] > best[1]
                else:
                    better = c[0] < best[0]
                if better:
                    best = c
            order.append(best)
            rest.remove(best)
        nf = sum(1 for c in cand if c[2])
        if tau >= 1.0:
            k = len(order)
        else:
            k = len(order)
            run = 0.0
            for t, c in enumerate(order):
                run += c[4]
                if run >= tau:
                    k = max(nf, t + 1)
                    break
        lists.append([c[0] for c in order[:k]])
    return lists


def attention(Q, K, V, lists, BQ, BK, causal, lam, G, sm=None,
              score=None, pv=None, force_skip=None, weight=None):
    """Online-softmax attention over each query block's list, one row and
    one key at a time.  ``score(r, c)`` and ``pv(r, c, p)`` may override the
    logit and the P.V contribution (vector over d); ``weight(p)`` what a
    probability adds to the normaliser of O (p itself by default; the skip
    rule always sees the plain running sum)."""
    n, d = len(Q), len(Q[0])
    if sm is None:
        sm = 1.0 / math.sqrt(d)
    if score is None:
        def score(r, c):
            return sm * sum(float(Q[r][e]) * float(K[c][e]) for e in range(d))
    if pv is None:
        def pv(r, c, p):
            return [p * float(V[c][e]) for e in range(d)]
    O = [[0.0] * d for _ in range(n)]
    skips = []
    for i, lst in enumerate(lists):
        rows = list(range(i * BQ, min(n, (i + 1) * BQ)))
        m = {r: -math.inf for r in rows}
        l = {r: 0.0 for r in rows}
        ln = {r: 0.0 for r in rows}   # the normaliser of O
        acc = {r: [0.0] * d for r in rows}
        ngroups = nblk(BQ, G)
        sk_i = []
        for t, j in enumerate(lst):
            cols = list(range(j * BK, min(n, (j + 1) * BK)))
            S, mloc, mnew, P = {}, {}, {}, {}
            for r in rows:
                S[r] = {}
                for c in cols:
                    S[r][c] = -math.inf if (causal and c > r) else score(r, c)
                mloc[r] = max(S[r].values())
                mnew[r] = max(m[r], mloc[r])
                if mnew[r] == -math.inf:
                    alpha = 1.0
                elif m[r] == -math.inf:
                    alpha = 0.0
                else:
                    alpha = math.exp(m[r] - mnew[r])
                P[r] = {c: (0.0 if S[r][c] == -math.inf else
                            math.exp(S[r][c] - mnew[r])) for c in cols}
                l[r] = alpha * l[r] + sum(P[r].values())
                ln[r] = alpha * ln[r] + sum((weight(x) if weight else x) for x in P[r].values())
                acc[r] = [alpha * a for a in acc[r]]
            flags = []
            for g in range(ngroups):
                grows = [r for r in rows if g * G <= r - rows[0] < (g + 1) * G]
                delta = -math.inf
                for r in grows:
                    if mloc[r] != -math.inf:
                        delta = max(delta, mloc[r] - mnew[r])
                skip = delta < lam
                if force_skip is not None:
                    skip = bool(force_skip[i][t][g])
                flags.append(skip)
                if not skip:
                    for r in grows:
                        for c in cols:
                            add = pv(r, c, P[r][c])
                            acc[r] = [a + b for a, b in zip(acc[r], add)]
            for r in rows:
                m[r] = mnew[r]
            sk_i.append(flags)
        skips.append(sk_i)
        for r in rows:
            O[r] = [a / ln[r] for a in acc[r]] if ln[r] > 0 else [0.0] * d
    return O, skips


def dense(Q, K, V, causal, sm=None):
    n, d = len(Q), len(Q[0])
    if sm is None:
        sm = 1.0 / math.sqrt(d)
    O = []
    for r in range(n):
        s = []
        for c in range(n):
            if causal and c > r:
                continue
            s.append((c, sm * sum(float(Q[r][e]) * float(K[c][e]) for e in range(d))))
        mx = max(v for _, v in s)
        w = [(c, math.exp(v - mx)) for c, v in s]
        den = sum(x for _, x in w)
        O.append([sum(x * float(V[c][e]) for c, x in w) / den for e in range(d)])
    return O


def true_recall(Q, K, lists, BQ, BK, causal, sm=None, blocks=None):
    """Mean over the rows of ``blocks`` of the exact softmax mass on the keys
    of the row's kept key blocks, one row and one key at a time."""
    n, d = len(Q), len(Q[0])
    if sm is None:
        sm = 1.0 / math.sqrt(d)
    if blocks is None:
        blocks = range(len(lists))
    tot, cnt = 0.0, 0
    for i in blocks:
        kept_keys = set()
        for j in lists[i]:
            for c in range(j * BK, min(n, (j + 1) * BK)):
                kept_keys.add(c)
        for r in range(i * BQ, min(n, (i + 1) * BQ)):
            s = {}
            for c in range(n):
                if causal and c > r:
                    continue
                s[c] = sm * sum(float(Q[r][e]) * float(K[c][e]) for e in range(d))
            mx = max(s.values())
            den = sum(math.exp(v - mx) for v in s.values())
            num = sum(math.exp(v - mx) for c, v in s.items() if c in kept_keys)
            tot += num / den
            cnt += 1
    return tot / cnt


def admissible(n, BQ, BK, causal):
    """|A_i| per query block, from the token-level definition: key block j
    is admissible when some key of it is visible to some row of block i."""
    out = []
    for i in range(nblk(n, BQ)):
        rows = range(i * BQ, min(n, (i + 1) * BQ))
        cnt = 0
        for j in range(nblk(n, BK)):
            keys = range(j * BK, min(n, (j + 1) * BK))
            if any((not causal) or c <= r for r in rows for c in keys):
                cnt += 1
        out.append(cnt)
    return out

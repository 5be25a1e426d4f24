"""Mask reuse across a sequence of calls -- TEST INFRASTRUCTURE ONLY.

Search-page abstracts (SparseD, LiteAttention) and the DynSparse story: the
sparse patterns of a head stay similar across denoising steps, so a mask can
be computed once and reused; early steps matter most (SparseD runs them
with full attention).  Reading: a sequence of calls with a schedule
(refresh_every >= 1, dense_steps >= 0).  Call s < dense_steps keeps every
admissible block (whatever the mask rule) and skips nothing; later calls
predict a fresh mask on call dense_steps and every refresh_every-th call
after it, and otherwise reuse the last mask, evaluated on the call's own
Q, K, V.

iCATS abstract: the tolerance to sparse approximation error varies across
denoising timesteps, so the sparsity follows a schedule guided by the
signal-to-noise ratio.  Reading: an optional per-call tau table supplied by
the caller (who owns the noise schedule; the pages give no formula); a
predicting call s uses tau_by_step[min(s, len - 1)], a reused mask keeps
the tau it was predicted with.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Tuple

from .sparse_attn_oracle import Params, predict_head, sparse_attention_head


def step_plan(n_steps: int, refresh_every: int, dense_steps: int) -> List[Tuple[str, int]]:
    """For each call: ("dense", s), ("refresh", s) or ("reuse", s0), where
    s0 is the call whose inputs produced the mask in use."""
    if refresh_every < 1 or dense_steps < 0:
        raise ValueError("refresh_every >= 1 and dense_steps >= 0")
    plan, src = [], None
    for s in range(n_steps):
        if s < dense_steps:
            plan.append(("dense", s))
        elif (s - dense_steps) % refresh_every == 0:
            src = s
            plan.append(("refresh", s))
        else:
            plan.append(("reuse", src))
    return plan


def call_tau(p: Params, s: int, tau_by_step=None) -> float:
    """The tau a predicting call s uses."""
    if tau_by_step is None or len(tau_by_step) == 0:
        return float(p.tau)
    return float(tau_by_step[min(s, len(tau_by_step) - 1)])


def dense_params(p: Params) -> Params:
    """The parameters of a dense call: every admissible block kept (tau = 1
    under a cumulative-mass rule; a top-k budget would still cut, so a
    dense call reads the top-k rule as top-cdf) and no P.V product
    skipped (lambda = -inf)."""
    rule = "topcdf" if p.rule == "topk" else p.rule
    return dataclasses.replace(p, tau=1.0, rule=rule, topk_blocks=0, skip_rule="lambda",
                               lam=-math.inf)


def sequence_head(steps, p: Params, refresh_every: int, dense_steps: int, attention=None,
                  tau_by_step=None):
    """``steps``: list of (Q, K, V) for one head.  Returns per call
    (O, lse, kept lists used, plan entry).  ``attention`` is the stage-two
    oracle (the unquantised one by default); ``tau_by_step`` the optional
    per-call tau table."""
    attention = attention or sparse_attention_head
    dense_p = dense_params(p)
    out, kept = [], None
    plan = step_plan(len(steps), refresh_every, dense_steps)
    for s, ((kind, src), (Q, K, V)) in enumerate(zip(plan, steps)):
        if kind == "dense":
            lists = predict_head(Q, K, dense_p)["kept"]
            O, lse, _ = attention(Q, K, V, lists, dense_p)
        else:
            if kind == "refresh":
                kept = predict_head(Q, K, dataclasses.replace(p, tau=call_tau(p, s, tau_by_step)))["kept"]
            lists = kept
            O, lse, _ = attention(Q, K, V, lists, p)
        out.append((O, lse, lists, (kind, src)))
    return out

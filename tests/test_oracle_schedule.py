"""CPU pins of the mask-reuse schedule (oracle/schedule.py).

* the call plan against hand-written tables;
* dense calls reproduce dense softmax attention (a closed form);
* refresh calls equal stage one + stage two on that call's own inputs;
* reuse calls use the mask of the call that refreshed it, evaluated on
  their own inputs (checked against a direct oracle call with that mask);
* the drift generator's step 0 is the workload's own head.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import Workload


@pytest.mark.parametrize("n,k,d,want", [
    (5, 1, 0, [("refresh", 0), ("refresh", 1), ("refresh", 2), ("refresh", 3), ("refresh", 4)]),
    (6, 2, 1, [("dense", 0), ("refresh", 1), ("reuse", 1), ("refresh", 3), ("reuse", 3),
               ("refresh", 5)]),
    (7, 3, 2, [("dense", 0), ("dense", 1), ("refresh", 2), ("reuse", 2), ("reuse", 2),
               ("refresh", 5), ("reuse", 5)]),
    (3, 10, 0, [("refresh", 0), ("reuse", 0), ("reuse", 0)]),
    (2, 1, 5, [("dense", 0), ("dense", 1)]),
])
def test_step_plan_tables(n, k, d, want):
    assert O.step_plan(n, k, d) == want


def test_step_plan_rejects_bad_schedules():
    for k, d in ((0, 0), (-1, 2), (2, -1)):
        with pytest.raises(ValueError):
            O.step_plan(3, k, d)


def test_sequence_head_against_direct_calls():
    w = Workload("seq", 201, 1, 1, 300, 32, "f32", structure="lm", causal=True, tau=0.9)
    steps = w.drift_head(0, 0, 5, dtheta=0.2)
    q0, k0, v0 = w.head(0, 0)
    np.testing.assert_array_equal(steps[0][0], q0)
    np.testing.assert_array_equal(steps[0][2], v0)
    p = O.Params(BQ=64, BK=32, G=16, causal=True, tau=0.9, lam=-2.0)
    out = O.sequence_head(steps, p, refresh_every=2, dense_steps=1)
    sm = 1.0 / math.sqrt(32)
    # call 0: dense
    od, lsed = O.dense_attention_head(*steps[0], sm, True)
    np.testing.assert_allclose(out[0][0], od, atol=1e-12)
    np.testing.assert_allclose(out[0][1], lsed, atol=1e-12)
    # call 1: refresh on its own inputs; call 2: that mask on call 2's inputs
    kept1 = O.predict_head(steps[1][0], steps[1][1], p)["kept"]
    o1, _, _ = O.sparse_attention_head(*steps[1], kept1, p)
    o2, _, _ = O.sparse_attention_head(*steps[2], kept1, p)
    np.testing.assert_array_equal(out[1][0], o1)
    np.testing.assert_array_equal(out[2][0], o2)
    assert all(np.array_equal(a, b) for a, b in zip(out[2][2], kept1))
    # the drifted inputs change the mask: a fresh one at call 3 differs
    kept3 = O.predict_head(steps[3][0], steps[3][1], p)["kept"]
    assert any(not np.array_equal(a, b) for a, b in zip(kept1, kept3))
    assert out[3][3] == ("refresh", 3) and out[4][3] == ("reuse", 3)


def test_tau_table():
    """A per-call tau table: a predicting call s uses tau_by_step[min(s, n-1)]
    (so a short table's last entry holds for later calls), a reused mask
    keeps the tau it was predicted with, dense calls ignore the table, and a
    table of the parameter's own tau changes nothing."""
    assert O.call_tau(O.Params(tau=0.9), 3, None) == 0.9
    assert O.call_tau(O.Params(tau=0.9), 1, [0.5, 0.7]) == 0.7
    assert O.call_tau(O.Params(tau=0.9), 7, [0.5, 0.7]) == 0.7
    w = Workload("seq_tau", 202, 1, 1, 256, 16, "f32", structure="gauss", tau=0.9)
    steps = w.drift_head(0, 0, 5, dtheta=0.3)
    p = O.Params(BQ=32, BK=16, G=8, tau=0.9, lam=-2.0)
    table = [0.6, 0.75, 0.95]
    out = O.sequence_head(steps, p, refresh_every=2, dense_steps=1, tau_by_step=table)
    # plan: dense 0, refresh 1 (tau 0.75), reuse 2, refresh 3 (tau 0.95: last entry), reuse 4
    for s, tau in ((1, 0.75), (3, 0.95)):
        kept = O.predict_head(steps[s][0], steps[s][1], O.Params(BQ=32, BK=16, G=8, tau=tau,
                                                                 lam=-2.0))["kept"]
        assert all(np.array_equal(a, b) for a, b in zip(out[s][2], kept))
        assert all(np.array_equal(a, b) for a, b in zip(out[s + 1][2], kept))
    # the two refreshes keep different numbers of blocks (the table acts)
    assert sum(map(len, out[1][2])) < sum(map(len, out[3][2]))
    same = O.sequence_head(steps, p, 2, 1, tau_by_step=[0.9])
    base = O.sequence_head(steps, p, 2, 1)
    for a, b in zip(same, base):
        np.testing.assert_array_equal(a[0], b[0])


@pytest.mark.parametrize("causal", [False, True])
def test_dense_calls_keep_everything_under_the_topk_rule(causal):
    """A dense call keeps every admissible block and skips nothing, whatever
    the mask rule: under a small top-k budget the dense call must still equal
    dense softmax attention (a closed form), while the sparse calls keep the
    budget."""
    w = Workload("seq_topk", 203, 1, 1, 400, 16, "f32", structure="gauss", causal=causal)
    steps = w.drift_head(0, 0, 3, dtheta=0.2)
    p = O.Params(BQ=64, BK=32, G=16, causal=causal, rule="topk", topk_blocks=2, lam=-1.0)
    dp = O.dense_params(p)
    assert (dp.rule, dp.tau, dp.lam, dp.skip_rule) == ("topcdf", 1.0, -math.inf, "lambda")
    out = O.sequence_head(steps, p, refresh_every=1, dense_steps=1)
    adm = O.admissible_blocks(400, 64, 32, causal).sum(axis=1)
    assert [len(x) for x in out[0][2]] == adm.tolist()
    od, _ = O.dense_attention_head(*steps[0], 1.0 / math.sqrt(16), causal)
    np.testing.assert_allclose(out[0][0], od, atol=1e-12)
    forced = O.forced_blocks(400, 64, 32, causal, 0, O.admissible_blocks(400, 64, 32, causal))
    for s in (1, 2):
        want = [min(a, max(f, 2)) for a, f in zip(adm, forced.sum(axis=1))]
        assert [len(x) for x in out[s][2]] == want

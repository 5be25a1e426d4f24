"""GPU parity of sparse_attn_step (mask reuse across a sequence of calls)
through the C ABI, against the oracle's schedule (oracle/schedule.py) on a
seeded drifting sequence (synth Workload.drift_head).

Per call: the refreshed flag equals the plan; a dense or refresh call's
mask matches the oracle's stage one on that call's inputs (bit-exact up to
the near-threshold rules), a reuse call leaves the mask untouched; the
skip bits match the oracle under that mask; the fp32 output matches the
oracle run under the GPU's own mask and skip bits (compare.out_tol).
"""
import dataclasses
import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_mean_pool_amd as sa  # noqa: E402
import oracle as O  # noqa: E402
from synth import Workload  # noqa: E402
import compare  # noqa: E402


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def decode(idx, cnt, bits, h):
    nqb = cnt.shape[2]
    kept = [idx[0, h, i, :cnt[0, h, i]].astype(np.int64) for i in range(nqb)]
    sk = []
    for i in range(nqb):
        t = np.arange(cnt[0, h, i])
        sk.append(((bits[0, h, i][:, t // 32] >> (t % 32).astype(np.uint32)) & 1).T.astype(bool))
    return kept, sk


@pytest.mark.parametrize("w,refresh_every,dense_steps,taus", [
    (Workload("step_field", 301, 1, 2, 1000, 128, "bf16", grid=(10, 10, 10), tau=0.9, lam=-5.0),
     2, 1, None),
    (Workload("step_lm_recall", 302, 1, 2, 700, 128, "bf16", structure="lm", causal=True,
              tau=0.95, skip_rule="recall", recall=0.95), 3, 0, None),
    (Workload("step_quant", 303, 1, 1, 800, 128, "bf16", grid=(8, 10, 10), tau=0.9, lam=-5.0,
              prec="i8fp8"), 2, 1, None),
    (Workload("step_tau_table", 304, 1, 2, 1000, 128, "bf16", grid=(10, 10, 10), tau=0.9,
              lam=-5.0), 1, 1, [1.0, 0.7, 0.8, 0.95]),
    # a dense call keeps every admissible block under the top-k rule too
    (Workload("step_topk", 305, 1, 2, 1000, 128, "bf16", structure="lm", causal=True,
              tau=0.9, lam=-5.0, rule="topk", topk_blocks=3), 2, 1, None),
], ids=["field_k2_d1", "lm_recall_k3", "quant_k2_d1", "field_tau_table", "topk_causal_d1"])
def test_step_sequence(w, refresh_every, dense_steps, taus):
    n_steps = 5
    log(f"[case] {w.name} steps={n_steps} refresh_every={refresh_every} dense={dense_steps} "
        f"taus={taus}")
    seqs = [w.drift_head(0, h, n_steps, dtheta=0.1) for h in range(w.H)]
    dev = torch.device("cuda:0")
    kw = dict(dtype="bf16", causal=w.causal, tau=w.tau, lam=w.lam, rule=w.rule, prec=w.prec,
              keep_prefix_kblocks=w.keep_prefix_kblocks, skip_rule=w.skip_rule, recall=w.recall,
              topk_blocks=w.topk_blocks, o_fp32=True)
    p = sa.make_params(w.B, w.H, w.N, w.D, **kw)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    pws, fws = sa.sparse_attn_workspace_size(p)
    idx = torch.full((1, w.H, nqb, nkb), -1, dtype=torch.int32, device=dev)
    cnt = torch.full((1, w.H, nqb), -1, dtype=torch.int32, device=dev)
    mask = sa.make_mask(idx, cnt)
    ws_p = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
    nw = (nkb + 31) // 32
    skips = torch.zeros((1, w.H, nqb, 4, nw), dtype=torch.int32, device=dev)
    o = torch.empty((1, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    sched = sa.make_schedule(refresh_every, dense_steps, tau_by_step=taus)
    op = O.Params(causal=w.causal, tau=float(np.float32(w.tau)), lam=float(np.float32(w.lam)),
                  rule=w.rule, keep_prefix_kblocks=w.keep_prefix_kblocks,
                  sm_scale=float(np.float32(1.0 / math.sqrt(w.D))), skip_rule=w.skip_rule,
                  recall=float(np.float32(w.recall)), topk_blocks=w.topk_blocks)
    dense_op = O.dense_params(op)
    n_adm = O.admissible_counts(w.N, 128, 64, w.causal)
    fn = O.sparse_attention_quant_head if w.prec == "i8fp8" else O.sparse_attention_head
    plan = O.step_plan(n_steps, refresh_every, dense_steps)
    prev = None
    for s in range(n_steps):
        Q, K, V = (np.stack([seqs[h][s][t] for h in range(w.H)])[None] for t in range(3))
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (Q, K, V))
        skips.zero_()
        sa.sparse_attn_step(p, sched, q, k, v, mask, o, None, skips, predict_ws=ws_p,
                            forward_ws=ws_f)
        torch.cuda.synchronize()
        kind, src = plan[s]
        assert sched.step == s + 1
        assert sched.refreshed == (0 if kind == "reuse" else 1), (s, kind)
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        bits = skips.cpu().numpy().view(np.uint32)
        og = o.cpu().numpy()
        if kind == "reuse":
            assert np.array_equal(cnt_h, prev[1])
            for h in range(w.H):
                for i in range(nqb):
                    c = cnt_h[0, h, i]
                    assert np.array_equal(idx_h[0, h, i, :c], prev[0][0, h, i, :c])
        prev = (idx_h, cnt_h)
        pr = dense_op if kind == "dense" else op
        if kind == "refresh":
            # the call's tau (the table's entry, as float32 like the library's)
            pr = dataclasses.replace(op, tau=float(np.float32(O.call_tau(op, s, taus))))
        worst = 0.0
        for h in range(w.H):
            qh, kh, vh = Q[0, h], K[0, h], V[0, h]
            gk, gs = decode(idx_h, cnt_h, bits, h)
            if kind != "reuse":
                pred = O.predict_head(qh, kh, pr)
                _, ex, fails = compare.compare_masks([gk], [pred], float(pr.tau))
                assert not fails, f"step {s} head {h}: {fails[:3]}"
            if kind == "dense":
                assert not any(x.any() for x in gs)
                assert cnt_h[0, h].tolist() == n_adm.tolist(), f"step {s} head {h}: not dense"
            stats = []
            if pr.skip_rule == "recall":
                Oref, _, _ = fn(qh, kh, vh, gk, pr, force_skip=gs, deltas=stats)
                _, _, sf = compare.compare_recall_skips(gs, stats, 1e-4)
            else:
                _, _, osk = fn(qh, kh, vh, gk, pr, deltas=stats)
                _, _, sf = compare.compare_skips(gs, osk, stats, float(pr.lam), 1e-3)
                Oref, _, _ = fn(qh, kh, vh, gk, pr, force_skip=gs)
            assert not sf, f"step {s} head {h}: skip mismatch {sf[:3]}"
            err = float(np.abs(og[0, h] - Oref).max())
            worst = max(worst, err)
            tol = compare.out_tol("i8fp8" if w.prec == "i8fp8" else "bf16", vh)
            assert err <= tol, f"step {s} head {h}: max-abs {err}"
        log(f"   step {s}: {kind} (mask of call {src}), max-abs {worst:.3g}")

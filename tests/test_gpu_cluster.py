"""GPU parity of token reordering (sparse_attn_cluster, sparse_attn_permute)
through the C ABI against the oracle's C1..C5 (oracle/cluster.py).

Bars:
  * every Lloyd pass: the GPU's labels of pass t against the oracle's pass
    run in fp64 from the GPU's own labels of pass t-1 (so an earlier
    near-tie does not cascade).  A label may differ only where the fp64
    quadratic form of the GPU's cluster is within 1e-4 * (x^T M x + the two
    centroids' c^T M c) of the minimum (the GPU decides in fp32), and such
    near-ties must stay rare;
  * the order: exactly the stable sort of the GPU's labels (integer work,
    bit-exact); the same inputs give the same outputs bit for bit;
  * permute: bit-exact gather and scatter;
  * the reordered attention: masks and skip bits on the permuted tokens by
    the rules of tests/compare.py, the fp32 output in the original order
    within compare.out_tol of the oracle run under the GPU's permutations,
    mask and skip bits.
"""
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
from synth import Workload, make_workload  # noqa: E402
import compare  # noqa: E402
from gpu_harness import to_device  # noqa: E402

TIE_REL = 1e-4
MAX_TIE_SHARE = 0.01


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def heads_of(w: Workload, heads):
    qs, ks, vs = zip(*(w.head(0, h) for h in heads))
    shape = (1, len(heads), w.N, w.D)
    return (np.stack(qs).reshape(shape), np.stack(ks).reshape(shape),
            np.stack(vs).reshape(shape))


def gpu_cluster(q, k, cq, ck, iters, metric):
    B, H, N, D = q.shape
    p = sa.make_params(B, H, N, D)
    cp = sa.make_cluster_params(cq, ck, iters, metric)
    ws = torch.empty(max(1, sa.sparse_attn_cluster_workspace_size(p, cp)), dtype=torch.uint8,
                     device=q.device)
    outs = [torch.full((B, H, N), -7, dtype=torch.int32, device=q.device) for _ in range(4)]
    sa.sparse_attn_cluster(p, cp, q, k, sa.make_reorder(*outs), ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.int64) for t in outs]


def check_pass(X, M, labels, c, tag):
    """labels: the GPU's labels of this pass; c: the centroids the oracle
    derives for it.  Returns the number of excused near-ties."""
    D = O.quad_dist(X, c, M)
    n = X.shape[0]
    o = np.argmin(D, axis=1)
    diff = np.flatnonzero(labels != o)
    if len(diff):
        xm = ((X[diff] @ M) * X[diff]).sum(axis=1)
        cm = ((c @ M) * c).sum(axis=1)
        gap = D[diff, labels[diff]] - D[diff, o[diff]]
        tol = TIE_REL * (np.abs(xm) + np.abs(cm[labels[diff]]) + np.abs(cm[o[diff]]))
        bad = gap > tol
        assert not bad.any(), (f"{tag}: token {diff[bad][0]} GPU cluster "
                               f"{labels[diff[bad][0]]} vs {o[diff[bad][0]]}, "
                               f"gap {gap[bad][0]:.3g} > {tol[bad][0]:.3g}")
        assert len(diff) <= MAX_TIE_SHARE * n + 1, f"{tag}: {len(diff)} near-ties of {n}"
    return len(diff)


def check_passes(Q, K, q, k, cq, ck, iters, metric):
    """Runs the GPU with 1..iters passes and checks each pass."""
    B, H, N, D = Q.shape
    prev = None
    cents = {}
    ties = 0
    for t in range(1, iters + 1):
        pq, pk, lq, lk = gpu_cluster(q, k, cq, ck, t, metric)
        for h in range(H):
            for side, X, lab, perm, C in (("q", Q[0, h], lq[0, h], pq[0, h], cq),
                                          ("k", K[0, h], lk[0, h], pk[0, h], ck)):
                X = X.astype(np.float64)
                assert lab.min() >= 0 and lab.max() < C
                assert np.array_equal(perm, O.token_order(lab, C)), f"pass {t} {side}{h} order"
                M = O.metric_matrix(Q[0, h], K[0, h], side, metric)
                key = (h, side)
                if t == 1:
                    c = X[O.seeds(N, C)].copy()
                else:
                    c = O.update(X, prev[key], cents[key])
                cents[key] = c
                ties += check_pass(X, M, lab, c, f"pass {t} {side}{h}")
        prev = {(h, s): (lq if s == "q" else lk)[0, h] for h in range(H) for s in ("q", "k")}
    return ties, (pq, pk, lq, lk)


@pytest.mark.parametrize("metric", ["interaction", "feature"])
@pytest.mark.parametrize("D,grid,cq,ck", [(128, (10, 15, 20), 24, 40), (64, (10, 10, 25), 19, 33)])
def test_cluster_passes(metric, D, grid, cq, ck):
    N = int(np.prod(grid))
    w = Workload("cluster_field", 401 + D, 1, 2, N, D, "bf16", grid=grid)
    log(f"[case] cluster N={N} D={D} C={cq}/{ck} metric={metric}")
    Q, K, _ = heads_of(w, [0, 1])
    q, k = to_device(Q, "bf16"), to_device(K, "bf16")
    ties, first = check_passes(Q, K, q, k, cq, ck, 4, metric)
    log(f"   4 passes checked, {ties} excused near-ties")
    again = gpu_cluster(q, k, cq, ck, 4, metric)
    assert all(np.array_equal(a, b) for a, b in zip(first, again))


def test_cluster_edge_cases():
    """One cluster (identity order), C = N (every token its own cluster:
    the order is the identity too), a ragged N and an empty cluster."""
    rng = np.random.default_rng(5)
    N, D = 333, 64
    Q = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    K = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    from synth import round_to_bf16
    Q, K = round_to_bf16(Q), round_to_bf16(K)
    q, k = to_device(Q, "bf16"), to_device(K, "bf16")
    pq, pk, lq, lk = gpu_cluster(q, k, 1, 1, 3, "interaction")
    assert np.array_equal(pq[0, 0], np.arange(N)) and np.array_equal(pk[0, 0], np.arange(N))
    assert not lq.any() and not lk.any()
    pq, pk, lq, lk = gpu_cluster(q, k, N, N, 1, "feature")
    assert np.array_equal(lq[0, 0], np.arange(N))
    assert np.array_equal(pq[0, 0], np.arange(N))
    # duplicated tokens: two seeds on equal rows tie, the smaller cluster wins
    # and the other stays empty (keeps its centroid) on the next pass
    Q2 = Q.copy()
    Q2[0, 0, :] = Q[0, 0, :1]
    q2 = to_device(Q2, "bf16")
    ties, _ = check_passes(Q2, K, q2, k, 7, 5, 3, "feature")
    pq, _, lq, _ = gpu_cluster(q2, k, 7, 5, 3, "feature")
    assert not lq.any()
    # tiny sequences: one token, and fewer tokens than one sort chunk
    for n, c in ((1, 1), (50, 6)):
        qn, kn = to_device(Q[:, :, :n].copy(), "bf16"), to_device(K[:, :, :n].copy(), "bf16")
        ties, out = check_passes(Q[:, :, :n], K[:, :, :n], qn, kn, c, c, 2, "interaction")
        assert sorted(out[0][0, 0].tolist()) == list(range(n))


def test_permute_roundtrip():
    rng = np.random.default_rng(6)
    B, H, N, D = 2, 3, 777, 128
    x = torch.randn(B, H, N, D, device="cuda").to(torch.bfloat16)
    perm = torch.stack([torch.randperm(N) for _ in range(B * H)]).reshape(B, H, N)
    perm = perm.to(torch.int32).cuda()
    p = sa.make_params(B, H, N, D)
    y = torch.empty_like(x)
    sa.sparse_attn_permute(p, x, perm, 0, y)
    want = torch.gather(x, 2, perm.long()[..., None].expand(B, H, N, D))
    torch.cuda.synchronize()
    assert torch.equal(y, want)
    back = torch.empty_like(x)
    sa.sparse_attn_permute(p, y, perm, 1, back)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    # fp32 rows (an fp32 O with bf16 inputs) and a strided [B, N, H, D] layout
    x32 = torch.randn(B, N, H, D, device="cuda")
    ps = sa.make_params(B, H, N, D, strides=(N * H * D, D, H * D))
    y32 = torch.empty_like(x32)
    sa.sparse_attn_permute(ps, x32, perm, 0, y32, elem_bytes=4)
    want32 = torch.gather(x32.permute(0, 2, 1, 3), 2,
                          perm.long()[..., None].expand(B, H, N, D))
    torch.cuda.synchronize()
    assert torch.equal(y32.permute(0, 2, 1, 3), want32)
    del rng


def reordered_run(Q, K, V, p_kw, cq, ck, iters, metric):
    """cluster -> permute Q, K, V -> predict -> forward (fp32 O) -> scatter O
    back, all through the C ABI on the device."""
    B, H, N, D = Q.shape
    q, k, v = (to_device(x, "bf16") for x in (Q, K, V))
    pq, pk, lq, lk = (torch.empty((B, H, N), dtype=torch.int32, device="cuda")
                      for _ in range(4))
    p = sa.make_params(B, H, N, D, **p_kw)
    p32 = sa.make_params(B, H, N, D, o_fp32=True, **p_kw)
    cp = sa.make_cluster_params(cq, ck, iters, metric)
    ws = torch.empty(max(1, sa.sparse_attn_cluster_workspace_size(p, cp)), dtype=torch.uint8,
                     device="cuda")
    sa.sparse_attn_cluster(p, cp, q, k, sa.make_reorder(pq, pk, lq, lk), ws)
    qp, kp, vp = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sa.sparse_attn_permute(p, q, pq, 0, qp)
    sa.sparse_attn_permute(p, k, pk, 0, kp)
    sa.sparse_attn_permute(p, v, pk, 0, vp)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    pws, _ = sa.sparse_attn_workspace_size(p)
    idx = torch.full((B, H, nqb, nkb), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, H, nqb), -1, dtype=torch.int32, device="cuda")
    mask = sa.make_mask(idx, cnt)
    sa.sparse_attn_predict(p, qp, kp, mask, torch.empty(pws, dtype=torch.uint8, device="cuda"))
    nw = (nkb + 31) // 32
    skips = torch.zeros((B, H, nqb, 4, nw), dtype=torch.int32, device="cuda")
    op = torch.empty((B, H, N, D), dtype=torch.float32, device="cuda")
    sa.sparse_attn_forward(p32, qp, kp, vp, mask, op, None, skips)
    o = torch.empty_like(op)
    sa.sparse_attn_permute(p, op, pq, 1, o, elem_bytes=4)
    torch.cuda.synchronize()
    c, ix = cnt.cpu().numpy(), idx.cpu().numpy()
    sb = skips.cpu().numpy().view(np.uint32)
    kept, sk = [], []
    for h in range(H):
        kh, sh = [], []
        for i in range(nqb):
            n = c[0, h, i]
            kh.append(ix[0, h, i, :n].astype(np.int64))
            t = np.arange(n)
            sh.append(((sb[0, h, i][:, t // 32] >> (t % 32).astype(np.uint32)) & 1).T.astype(bool))
        kept.append(kh)
        sk.append(sh)
    return dict(O=o.cpu().numpy(), perm_q=pq.cpu().numpy(), perm_k=pk.cpu().numpy(),
                kept=kept, skips=sk)


@pytest.mark.parametrize("metric", ["interaction", "feature"])
def test_reordered_attention(metric):
    w = Workload("reorder_field", 411, 1, 2, 2000, 128, "bf16", grid=(8, 10, 25), tau=0.9,
                 lam=-5.0)
    log(f"[case] reordered attention {w.name} N={w.N} metric={metric}")
    Q, K, V = heads_of(w, [0, 1])
    tau32, lam32 = float(np.float32(w.tau)), float(np.float32(w.lam))
    r = reordered_run(Q, K, V, dict(tau=w.tau, lam=w.lam), 16, 32, 4, metric)
    p = O.Params(tau=tau32, lam=lam32, sm_scale=float(np.float32(1 / math.sqrt(w.D))))
    worst = 0.0
    for h in range(w.H):
        pq, pk = r["perm_q"][0, h], r["perm_k"][0, h]
        assert sorted(pq.tolist()) == list(range(w.N)) and sorted(pk.tolist()) == list(range(w.N))
        Qp, Kp, Vp = Q[0, h][pq], K[0, h][pk], V[0, h][pk]
        pred = O.predict_head(Qp, Kp, p)
        _, _, fails = compare.compare_masks([r["kept"][h]], [pred], tau32)
        assert not fails, fails[:3]
        stats = []
        _, _, osk = O.sparse_attention_head(Qp, Kp, Vp, r["kept"][h], p, deltas=stats)
        _, _, sf = compare.compare_skips(r["skips"][h], osk, stats, lam32, 1e-3)
        assert not sf, sf[:3]
        Oref, _, _, _ = O.reordered_attention_head(Q[0, h], K[0, h], V[0, h], p, pq, pk,
                                                   force_kept=r["kept"][h],
                                                   force_skip=r["skips"][h])
        err = float(np.abs(r["O"][0, h] - Oref).max())
        worst = max(worst, err)
        assert err <= compare.out_tol("bf16"), f"head {h}: max-abs {err}"
    log(f"   max-abs {worst:.3g}")


def test_reordered_attention_full_size():
    """The reordered pipeline at the video workload's N = 32760 with the
    bench's cluster counts (256 / 512, 4 passes), on two of its heads: the
    mask of every query block of the reordered tokens against the oracle's
    stage one, and skip bits and fp32 output of sampled query blocks (first,
    last, seeded random ones) against the oracle under the GPU's own mask and
    skips, compared in the original row order."""
    w = make_workload("wan_video")
    heads = [0, 21]
    log(f"[case] reordered attention full size N={w.N} heads {heads}")
    Q, K, V = heads_of(w, heads)
    tau32, lam32 = float(np.float32(w.tau)), float(np.float32(w.lam))
    r = reordered_run(Q, K, V, dict(tau=w.tau, lam=w.lam), 256, 512, 4, "interaction")
    p = O.Params(tau=tau32, lam=lam32, sm_scale=float(np.float32(1 / math.sqrt(w.D))))
    nqb = (w.N + 127) // 128
    rng = np.random.default_rng(17)
    worst = 0.0
    for h in range(len(heads)):
        pq, pk = r["perm_q"][0, h], r["perm_k"][0, h]
        assert sorted(pq.tolist()) == list(range(w.N)) and sorted(pk.tolist()) == list(range(w.N))
        Qp, Kp, Vp = Q[0, h][pq], K[0, h][pk], V[0, h][pk]
        pred = O.predict_head(Qp, Kp, p)
        _, ex, fails = compare.compare_masks([r["kept"][h]], [pred], tau32)
        assert not fails, fails[:3]
        blocks = sorted({0, nqb - 1, *rng.choice(nqb, size=4, replace=False).tolist()})
        sub_kept = [r["kept"][h][i] if i in blocks else np.zeros(0, dtype=np.int64)
                    for i in range(nqb)]
        sub_skip = [r["skips"][h][i] if i in blocks else np.zeros((0, 4), dtype=bool)
                    for i in range(nqb)]
        stats = []
        _, _, osk = O.sparse_attention_head(Qp, Kp, Vp, sub_kept, p, deltas=stats)
        _, mis, sf = compare.compare_skips([sub_skip[i] for i in blocks],
                                           [osk[i] for i in blocks],
                                           [stats[i] for i in blocks], lam32, 1e-3)
        assert not sf, sf[:3]
        Op, _, _ = O.sparse_attention_head(Qp, Kp, Vp, sub_kept, p, force_skip=sub_skip)
        rows = np.concatenate([np.arange(i * 128, min(w.N, (i + 1) * 128)) for i in blocks])
        err = float(np.abs(r["O"][0, h][pq[rows]] - Op[rows]).max())
        worst = max(worst, err)
        assert err <= compare.out_tol("bf16"), f"head {heads[h]}: max-abs {err}"
        log(f"   head {heads[h]}: masks {ex}/{nqb} exact, {mis} near-lambda skips, blocks "
            f"{blocks}, max-abs {err:.3g}")
    log(f"   max-abs {worst:.3g}")


def test_cluster_full_size():
    """The video workload's shape (N = 32760, D = 128) with the cluster counts
    the bench uses (NQB and NKB: 256 / 512, 4 passes), on two of its heads;
    every pass checked."""
    w = make_workload("wan_video")
    log(f"[case] cluster full size N={w.N} heads 0, 39")
    Q, K, _ = heads_of(w, [0, 39])
    q, k = to_device(Q, "bf16"), to_device(K, "bf16")
    ties, _ = check_passes(Q, K, q, k, 256, 512, 4, "interaction")
    log(f"   {ties} excused near-ties over 4 passes x 2 heads x 2 sides")


def test_cluster_strided_batch():
    """B = 2 with Q, K stored [B, N, H, D] (caller strides): the same orders
    as the packed layout, and every pass checked on one (b, h)."""
    w = Workload("cluster_strided", 421, 2, 2, 1500, 128, "bf16", grid=(6, 10, 25))
    log("[case] cluster B=2 H=2 N=1500 strided")
    qs, ks = [], []
    for b in range(2):
        for h in range(2):
            q_, k_, _ = w.head(b, h)
            qs.append(q_)
            ks.append(k_)
    Q = np.stack(qs).reshape(2, 2, w.N, w.D)
    K = np.stack(ks).reshape(2, 2, w.N, w.D)
    q, k = to_device(Q, "bf16"), to_device(K, "bf16")
    packed = gpu_cluster(q, k, 12, 23, 3, "interaction")
    qt = q.permute(0, 2, 1, 3).contiguous()
    kt = k.permute(0, 2, 1, 3).contiguous()
    p = sa.make_params(2, 2, w.N, w.D, strides=(w.N * 2 * w.D, w.D, 2 * w.D))
    cp = sa.make_cluster_params(12, 23, 3, "interaction")
    ws = torch.empty(sa.sparse_attn_cluster_workspace_size(p, cp), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.full((2, 2, w.N), -7, dtype=torch.int32, device="cuda") for _ in range(4)]
    sa.sparse_attn_cluster(p, cp, qt, kt, sa.make_reorder(*outs), ws)
    torch.cuda.synchronize()
    strided = [t.cpu().numpy().astype(np.int64) for t in outs]
    assert all(np.array_equal(a, b) for a, b in zip(packed, strided))
    # the passes of one (b, h) = (1, 0) against the oracle
    sub_q, sub_k = Q[1:2, 0:1], K[1:2, 0:1]
    ties, _ = check_passes(sub_q, sub_k, to_device(sub_q, "bf16"), to_device(sub_k, "bf16"),
                           12, 23, 3, "interaction")
    pq, pk, lq, lk = (x[1:2, 0:1] for x in packed)
    one = gpu_cluster(to_device(sub_q, "bf16"), to_device(sub_k, "bf16"), 12, 23, 3,
                      "interaction")
    assert np.array_equal(one[0], pq) and np.array_equal(one[2], lq)

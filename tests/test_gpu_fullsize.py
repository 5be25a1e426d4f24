"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (one predict + one forward over all heads).

The oracle cannot redo whole workloads in seconds, so:
  * every head: properties that hold at any size -- kept lists are
    repetition-free admissible subsets that start with the forced blocks,
    counts lie in [max(1, |F|), |A|], the skip words past each list are 0;
  * sampled heads: block means, the whole head's mask against the oracle
    (bit-exact up to the near-threshold rules);
  * sampled query blocks of those heads (first, last -- ragged when N is
    not a multiple of 128 -- and seeded random ones): skip bits and the fp32
    output against the oracle run under the GPU's own mask and skip bits,
    and the bf16 output as that result rounded.
"""
import dataclasses
import math
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_mean_pool_amd as sa  # noqa: E402
import oracle as O  # noqa: E402
from synth import make_workload, round_to_bf16  # noqa: E402
import compare  # noqa: E402

SKIP_TOL = {"bf16": 1e-3, "f32": 1e-4, "i8fp8": 1e-3, "i8mxfp8": 1e-3}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def generate(w):
    with ThreadPoolExecutor(16) as ex:
        heads = list(ex.map(lambda bh: w.head(bh // w.H, bh % w.H), range(w.B * w.H)))
    shape = (w.B, w.H, w.N, w.D)
    return tuple(np.stack([x[t] for x in heads]).reshape(shape) for t in range(3))


def decode_skips(bits, cnt):
    t = np.arange(cnt)
    return ((bits[:, t // 32] >> (t % 32).astype(np.uint32)) & 1).T.astype(bool)


@pytest.mark.parametrize("name,heads,nblocks,over", [
    ("tiny_fp32", None, None, {}),
    ("wan_video", [0, 23], 5, {}),
    # the rest of the video workload's tau sweep, and top-k budgets the bench
    # reports beside it (the mean kept count at tau = 0.9, and half the keys)
    ("wan_video", [17], 4, dict(tau=0.95)),
    ("wan_video", [29], 4, dict(tau=0.99)),
    ("wan_video", [5], 4, dict(rule="topk", topk_blocks=443)),
    ("wan_video", [36], 4, dict(rule="topk", topk_blocks=256)),
    # the same masks with the skip switched off (lambda = -inf), which the
    # bench times beside the headline: no group may skip
    ("wan_video", [21], 4, dict(lam=-math.inf)),
    ("quant_long", [9], 4, dict(lam=-math.inf)),
    ("quant_long", [14], 4, dict(prec="i8mxfp8", lam=-math.inf)),
    ("hunyuan_video", [7, 19], 8, {}),
    ("lm_causal", [0, 31], 5, {}),
    ("quant_long", [5], 4, {}),
    ("quant_long", [12], 4, dict(prec="i8mxfp8")),
    ("wan_video", [11], 4, dict(skip_rule="recall", recall=0.95)),
    ("lm_causal", [9], 4, dict(skip_rule="recall", recall=0.9)),
    # K and V of eight heads (270 MB) exceed the Infinity Cache: the forward
    # runs its V-vote schedule in the windowed workgroup order, whose
    # 512-block windows straddle the heads' 516 query blocks
    ("wan_video", [0, 7], 4, dict(H=8, N=66000, grid=(22, 50, 60))),
    ("wan_video", [3], 4, dict(H=8, N=66000, grid=(22, 50, 60), skip_rule="recall",
                               recall=0.95)),
    # skip groups of two wavefronts in the V-vote schedule, and the recall rule
    # over the whole block (which the host runs in the plain schedule)
    ("wan_video", [2], 4, dict(H=8, N=66000, grid=(22, 50, 60), group_rows=64)),
    ("wan_video", [6], 4, dict(H=8, N=66000, grid=(22, 50, 60), skip_rule="recall",
                               recall=0.95, group_rows=128)),
    ("wan_video", [13], 4, dict(group_rows=16)),
    # the longest sequence the library takes (N = 262144: 4096 key blocks,
    # the mask kernel's largest sort), three heads, so the V-vote schedule
    ("wan_video", [0, 2], 3, dict(H=3, N=262144, grid=(16, 128, 128))),
    # half-wavefront groups and four-wavefront groups in the V-vote schedule
    ("wan_video", [4], 4, dict(H=8, N=66000, grid=(22, 50, 60), group_rows=16)),
    ("wan_video", [1], 4, dict(H=8, N=66000, grid=(22, 50, 60), group_rows=128)),
])
def test_fullsize_parity(name, heads, nblocks, over):
    w = dataclasses.replace(make_workload(name), **over)
    t0 = time.perf_counter()
    Q, K, V = generate(w)
    log(f"[fullsize] {name} B={w.B} H={w.H} N={w.N} D={w.D} generated in "
        f"{time.perf_counter() - t0:.1f}s")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(tdt).to(dev) for x in (Q, K, V))
    kw = dict(dtype=w.dtype, causal=w.causal, tau=w.tau, lam=w.lam, rule=w.rule, prec=w.prec,
              keep_prefix_kblocks=w.keep_prefix_kblocks, skip_rule=w.skip_rule,
              recall=w.recall, topk_blocks=w.topk_blocks, lambda_group_rows=w.group_rows)
    p = sa.make_params(w.B, w.H, w.N, w.D, **kw)
    p32 = sa.make_params(w.B, w.H, w.N, w.D, o_fp32=True, **kw)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    pws, fws = sa.sparse_attn_workspace_size(p)
    idx = torch.full((w.B, w.H, nqb, nkb), -1, dtype=torch.int32, device=dev)
    cnt = torch.full((w.B, w.H, nqb), -1, dtype=torch.int32, device=dev)
    ws_p = torch.empty(pws, dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
    nw = (nkb + 31) // 32
    skips = torch.zeros((w.B, w.H, nqb, 128 // w.group_rows, nw), dtype=torch.int32,
                        device=dev)
    o32 = torch.empty((w.B, w.H, w.N, w.D), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    mask = sa.make_mask(idx, cnt)
    sa.sparse_attn_predict(p, q, k, mask, ws_p)
    sa.sparse_attn_forward(p32, q, k, v, mask, o32, None, skips, ws_f)
    sa.sparse_attn_forward(p, q, k, v, mask, o, None, None, ws_f)
    torch.cuda.synchronize()
    log(f"   GPU done at {time.perf_counter() - t0:.1f}s")
    idx_h = idx.cpu().numpy()
    cnt_h = cnt.cpu().numpy()
    bits_h = skips.cpu().numpy().view(np.uint32)
    ws_h = ws_p.cpu().numpy()
    nq_bytes = w.B * w.H * nqb * w.D * 4
    qbar = ws_h[:nq_bytes].view(np.float32).reshape(w.B, w.H, nqb, w.D)
    koff = (nq_bytes + 255) // 256 * 256
    kbar = ws_h[koff:koff + w.B * w.H * nkb * w.D * 4].view(np.float32).reshape(w.B, w.H, nkb, w.D)

    # properties on every head
    adm = O.admissible_blocks(w.N, 128, 64, w.causal)
    n_adm = adm.sum(axis=1)
    F = O.forced_blocks(w.N, 128, 64, w.causal, w.keep_prefix_kblocks, adm)
    n_f = F.sum(axis=1)
    assert np.all(cnt_h >= np.maximum(1, n_f)[None, None, :])
    assert np.all(cnt_h <= n_adm[None, None, :])
    for b in range(w.B):
        for h in range(w.H):
            for i in range(nqb):
                c = cnt_h[b, h, i]
                lst = idx_h[b, h, i, :c]
                assert len(np.unique(lst)) == c and lst.min() >= 0 and lst.max() < nkb
                assert adm[i, lst].all()
                assert F[i, lst[:n_f[i]]].all()
                full = bits_h[b, h, i, :, c // 32 + (1 if c % 32 else 0):]
                assert not full.any()
    if w.lam == -math.inf and w.skip_rule == "lambda":
        # lambda = -inf never skips, except groups past the last row of a
        # partial block, which hold no rows and read as skipped
        real = -(-(w.N - (nqb - 1) * 128) // w.group_rows)
        assert not bits_h[:, :, :-1].any() and not bits_h[:, :, -1, :real].any()

    tau32 = float(np.float32(w.tau))
    lam32 = float(np.float32(w.lam))
    op = O.Params(causal=w.causal, tau=tau32, lam=lam32, rule=w.rule,
                  keep_prefix_kblocks=w.keep_prefix_kblocks,
                  sm_scale=float(np.float32(1.0 / math.sqrt(w.D))),
                  skip_rule=w.skip_rule, recall=float(np.float32(w.recall)),
                  topk_blocks=w.topk_blocks, G=w.group_rows)
    mode = w.prec if w.prec in ("i8fp8", "i8mxfp8") else w.dtype
    if heads is None:
        heads = list(range(w.H))
    rng = np.random.default_rng(7)
    worst = 0.0
    for h in heads:
        qh, kh, vh = Q[0, h], K[0, h], V[0, h]
        pred = O.predict_head(qh, kh, op)
        np.testing.assert_allclose(qbar[0, h], pred["qbar"], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(kbar[0, h], pred["kbar"], rtol=1e-5, atol=1e-6)
        gk = [idx_h[0, h, i, :cnt_h[0, h, i]].astype(np.int64) for i in range(nqb)]
        mpred = O.predict_from_means(qbar[0, h], kbar[0, h], w.N, op)
        n, ex, fails = compare.compare_masks([gk], [pred], 2.0 if w.rule == "topk" else tau32,
                                             [mpred])
        assert not fails, f"{name} head {h}: {fails[:3]}"
        if nblocks is None:
            blocks = list(range(nqb))
        else:
            blocks = sorted({0, nqb - 1, *rng.choice(nqb, size=nblocks - 2, replace=False).tolist()})
        sub_kept = [gk[i] if i in blocks else np.zeros(0, dtype=np.int64) for i in range(nqb)]
        gs = [decode_skips(bits_h[0, h, i], cnt_h[0, h, i]) if i in blocks
              else np.zeros((0, 128 // w.group_rows), dtype=bool) for i in range(nqb)]
        deltas = []
        if mode == "bf16" or mode == "f32":
            fn = O.sparse_attention_head
        else:
            def fn(*args, **kw):
                return O.sparse_attention_quant_head(*args, v_pow2=w.prec == "i8mxfp8", **kw)
        if w.skip_rule == "recall":
            Oref, _, _ = fn(qh, kh, vh, sub_kept, op, force_skip=gs, deltas=deltas)
            ns, mis, sf = compare.compare_recall_skips([gs[i] for i in blocks],
                                                       [deltas[i] for i in blocks], 1e-4)
        else:
            _, _, osk = fn(qh, kh, vh, sub_kept, op, deltas=deltas)
            ns, mis, sf = compare.compare_skips([gs[i] for i in blocks], [osk[i] for i in blocks],
                                                [deltas[i] for i in blocks], lam32,
                                                SKIP_TOL[mode])
            Oref, _, _ = fn(qh, kh, vh, sub_kept, op, force_skip=gs)
        assert not sf, f"{name} head {h}: skip mismatch {sf[:3]}"
        rows = np.concatenate([np.arange(i * 128, min(w.N, (i + 1) * 128)) for i in blocks])
        og = o32[0, h].cpu().numpy()
        err = float(np.abs(og[rows] - Oref[rows]).max())
        worst = max(worst, err)
        assert err <= compare.out_tol(mode, vh), f"{name} head {h}: max-abs {err}"
        if w.dtype == "bf16":
            ob = o[0, h].float().cpu().numpy()
            np.testing.assert_array_equal(ob[rows], round_to_bf16(og[rows]))
        log(f"   head {h}: masks {ex}/{n} exact, skips {mis}/{ns} near-lambda, blocks "
            f"{blocks}, max-abs {err:.3g} ({time.perf_counter() - t0:.1f}s)")
    log(f"[fullsize] {name} ok, worst max-abs {worst:.3g}")

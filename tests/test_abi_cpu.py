"""CPU checks of the C-ABI library: it loads, exports every function that
include/sparse_attn.h declares, and its host-only entry points (shapes,
workspace sizes, info, status strings) and argument validation work
without a GPU.  Validation failures return before anything is enqueued, so
the fake device pointers used here are never dereferenced."""
import ctypes
import math
import re

import numpy as np
import pytest

import block_mean_pool_amd as sa


def declared_functions():
    text = open(sa.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"sparse_attn_predict", "sparse_attn_forward"} <= set(names)
    for n in names:
        assert hasattr(sa.lib, n), n


def test_probe_library_exports():
    """The benchmark's measurement helpers build into their own library,
    outside the attention library's ABI."""
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(sa.LIB_PATH)), "probe", "libsa_probe.so")
    probe = ctypes.CDLL(path)
    for n in ("sa_probe_clock", "sa_probe_clock_max_samples", "sa_probe_mfma",
              "sa_probe_mfma_chains"):
        assert hasattr(probe, n), n
    assert probe.sa_probe_clock_max_samples() == 256
    assert not any(n.startswith("sa_probe") for n in declared_functions())
    assert not hasattr(sa.lib, "sa_probe_clock")


def test_binding_exposes_the_same_names():
    for n in declared_functions():
        assert callable(getattr(sa, n)), n


def test_struct_layout_matches_header():
    # 10 int32 + 3 float + 3 int32 = 64 bytes, + 3 int64, + int32 + float + int32,
    # padded to the 8-byte alignment of the int64 fields
    assert ctypes.sizeof(sa.SaParams) == 104
    assert sa.SaParams.stride_b.offset == 64
    assert sa.SaParams.skip_rule.offset == 88
    assert sa.SaParams.recall.offset == 92
    assert sa.SaParams.topk_blocks.offset == 96
    assert ctypes.sizeof(sa.SaMask) == 24
    # field order and names as declared in the header
    text = open(sa.HEADER).read()
    body = text[text.index("typedef struct sa_params {"):text.index("} sa_params;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    declared = re.findall(r"\b(\w+)\s*[,;]", body.split("{", 1)[1])
    ctypes_names = [f[0] for f in sa.SaParams._fields_]
    assert [n.replace("lambda", "lam") if n == "lambda" else n for n in declared] == ctypes_names


def test_shapes_and_workspace():
    p = sa.make_params(1, 40, 32760, 128)
    assert sa.sparse_attn_mask_shape(p) == (256, 512)
    pw, fw = sa.sparse_attn_workspace_size(p)
    assert pw == 40 * 256 * 128 * 4 + 40 * 512 * 128 * 4
    assert fw == 0
    q = sa.make_params(1, 16, 65536, 128, prec="i8fp8", rule="energy")
    _, fw = sa.sparse_attn_workspace_size(q)
    bh = 16
    assert fw == 2 * bh * 65536 * 128 + bh * 1024 * 128 * 64 + bh * 512 * 4 + 2 * bh * 1024 * 4
    q4 = sa.make_params(1, 16, 65536, 128, prec="i4fp8", rule="energy")
    assert sa.sparse_attn_workspace_size(q4)[1] == fw
    assert sa.sparse_attn_info() == (32, 8)
    assert sa.sparse_attn_status_str(3) == "SA_ERR_WORKSPACE"
    assert sa.sparse_attn_status_str(99) == "SA_ERR_UNKNOWN"
    p = sa.make_params(2, 3, 0, 64)
    assert sa.sparse_attn_mask_shape(p) == (0, 0)
    assert sa.sparse_attn_workspace_size(p) == (0, 0)


@pytest.mark.parametrize("prec", ["i8fp8", "i4fp8", "i8mxfp8"])
@pytest.mark.parametrize("D", [64, 128])
def test_quantised_modes_take_both_head_dimensions(prec, D):
    p = sa.make_params(1, 2, 1000, D, prec=prec)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    _, fws = sa.sparse_attn_workspace_size(p)
    # INT8 Q and K codes, the e4m3 V^T tiles, and the three scale arrays
    assert fws >= 2 * 2 * 1000 * D + 2 * nkb * D * 64 + 4 * 2 * (nqb + 2 * nkb)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), sa.SA_ERR_UNSUPPORTED),
    (dict(block_q=64), sa.SA_ERR_UNSUPPORTED),
    (dict(tau=0.0), sa.SA_ERR_INVALID_ARG),
    (dict(tau=float("nan")), sa.SA_ERR_INVALID_ARG),
    (dict(lam=float("nan")), sa.SA_ERR_INVALID_ARG),
    (dict(sm_scale=-1.0), sa.SA_ERR_INVALID_ARG),
    (dict(lambda_group_rows=48), sa.SA_ERR_UNSUPPORTED),
    (dict(lambda_group_rows=8), sa.SA_ERR_UNSUPPORTED),
    (dict(prec="i8fp8", dtype="f32"), sa.SA_ERR_UNSUPPORTED),
    (dict(prec=4), sa.SA_ERR_INVALID_ARG),
    (dict(prec="i8mxfp8", dtype="f32"), sa.SA_ERR_UNSUPPORTED),
    (dict(keep_prefix_kblocks=-1), sa.SA_ERR_INVALID_ARG),
    (dict(N=300000), sa.SA_ERR_UNSUPPORTED),
    (dict(strides=(0, 0, 100)), sa.SA_ERR_INVALID_ARG),
    (dict(strides=(0, 0, 130)), sa.SA_ERR_INVALID_ARG),
    (dict(skip_rule=2), sa.SA_ERR_INVALID_ARG),
    (dict(rule="topk", topk_blocks=0), sa.SA_ERR_INVALID_ARG),
    (dict(rule=3), sa.SA_ERR_INVALID_ARG),
    (dict(skip_rule="recall", recall=0.0), sa.SA_ERR_INVALID_ARG),
    (dict(skip_rule="recall", recall=1.5), sa.SA_ERR_INVALID_ARG),
    (dict(skip_rule="recall", recall=float("nan")), sa.SA_ERR_INVALID_ARG),
])
def test_invalid_params_rejected_before_launch(kw, code):
    base = dict(B=1, H=2, N=1000, D=128)
    shape = {k: kw.pop(k) for k in list(kw) if k in base}
    base.update(shape)
    p = sa.make_params(base["B"], base["H"], base["N"], base["D"], **kw)
    fake = 1 << 20  # never dereferenced: validation fails first
    mask = sa.make_mask(fake, fake)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict(p, fake, fake, mask, fake, ws_bytes=1 << 40, stream=0)
    assert e.value.code == code
    assert sa.sparse_attn_last_error()
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_forward(p, fake, fake, fake, mask, fake, ws=fake, ws_bytes=1 << 40,
                               stream=0)
    assert e.value.code == code
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_pool(p, fake, fake, fake, ws_bytes=1 << 40, stream=0)
    assert e.value.code == code


def test_pool_validated_before_launch():
    p = sa.make_params(1, 2, 1000, 128)
    fake = 1 << 20  # never dereferenced: validation fails first
    need = sa.sparse_attn_workspace_size(p)[0]
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_pool(p, fake, fake, fake, ws_bytes=need - 1, stream=0)
    assert e.value.code == sa.SA_ERR_WORKSPACE
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_pool(p, fake + 8, fake, fake, ws_bytes=need, stream=0)
    assert e.value.code == sa.SA_ERR_INVALID_ARG
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_pool(p, 0, fake, fake, ws_bytes=need, stream=0)
    assert e.value.code == sa.SA_ERR_INVALID_ARG
    # an empty problem is a valid no-op
    sa.sparse_attn_pool(sa.make_params(1, 2, 0, 128), 0, 0, 0, ws_bytes=0, stream=0)


def test_step_schedule_validated_before_launch():
    assert ctypes.sizeof(sa.SaSchedule) == 32
    assert sa.SaSchedule.tau_by_step.offset == 16 and sa.SaSchedule.n_tau.offset == 24
    p = sa.make_params(1, 2, 1000, 128, tau=0.9)
    fake = 1 << 20  # never dereferenced: validation fails first
    mask = sa.make_mask(fake, fake)
    bad_table = sa.make_schedule(1, 0, tau_by_step=[0.9])
    bad_table.n_tau = 0
    nan_tau = sa.make_schedule(1, 0, tau_by_step=[float("nan")])
    for sched in (sa.make_schedule(0, 0), sa.make_schedule(2, -1), sa.SaSchedule(1, 0, -3, 0),
                  bad_table, nan_tau):
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_step(p, sched, fake, fake, fake, mask, fake, predict_ws=fake,
                                forward_ws=fake, predict_ws_bytes=1 << 40,
                                forward_ws_bytes=1 << 40, stream=0)
        assert e.value.code == sa.SA_ERR_INVALID_ARG
    # a bad part of the forward half is caught before the predict half runs,
    # and the schedule does not advance
    sched = sa.make_schedule(3, 1)
    for bad in (dict(v=None), dict(forward_ws_bytes=0, forward_ws=None)):
        args = dict(q=fake, k=fake, v=fake, o=fake, predict_ws=fake, forward_ws=fake,
                    predict_ws_bytes=1 << 40, forward_ws_bytes=1 << 40)
        args.update(bad)
        q8 = sa.make_params(1, 2, 1000, 128, tau=0.9, prec="i8fp8")
        with pytest.raises(sa.SparseAttnError):
            sa.sparse_attn_step(q8, sched, args["q"], args["k"], args["v"], mask, args["o"],
                                predict_ws=args["predict_ws"], forward_ws=args["forward_ws"],
                                predict_ws_bytes=args["predict_ws_bytes"],
                                forward_ws_bytes=args["forward_ws_bytes"], stream=0)
        assert sched.step == 0


def test_null_and_workspace_errors():
    p = sa.make_params(1, 2, 1000, 128)
    fake = 1 << 20
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict(p, None, fake, sa.make_mask(fake, fake), fake, ws_bytes=1 << 30,
                               stream=0)
    assert e.value.code == sa.SA_ERR_INVALID_ARG
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict(p, fake, fake, sa.make_mask(None, fake), fake, ws_bytes=1 << 30,
                               stream=0)
    assert e.value.code == sa.SA_ERR_INVALID_ARG
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict(p, fake, fake, sa.make_mask(fake, fake), fake, ws_bytes=16,
                               stream=0)
    assert e.value.code == sa.SA_ERR_WORKSPACE
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict(p, fake + 2, fake, sa.make_mask(fake, fake), fake,
                               ws_bytes=1 << 30, stream=0)
    assert e.value.code == sa.SA_ERR_INVALID_ARG
    q = sa.make_params(1, 2, 1000, 128, prec="i8fp8")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_forward(q, fake, fake, fake, sa.make_mask(fake, fake), fake, ws=None,
                               ws_bytes=0, stream=0)
    assert e.value.code == sa.SA_ERR_WORKSPACE


def test_empty_problem_is_ok_without_pointers():
    p = sa.make_params(0, 4, 100, 128)
    sa.sparse_attn_predict(p, None, None, sa.make_mask(None, None), None, stream=0)
    sa.sparse_attn_forward(p, None, None, None, sa.make_mask(None, None), None, stream=0)
    assert sa.sparse_attn_last_error() == ""
    assert not math.isnan(0.0)


def test_cluster_structs_and_workspace():
    assert ctypes.sizeof(sa.SaClusterParams) == 16
    assert ctypes.sizeof(sa.SaReorder) == 32
    p = sa.make_params(1, 2, 1000, 128)
    cp = sa.make_cluster_params(10, 20, iters=3, metric="feature")
    z2, C, N, D, nch = 4, 20, 1000, 128, 4

    def r(x):
        return (x + 255) // 256 * 256
    want = (r(z2 * C * D * 4) + 2 * r(z2 * C * D * 2) + r(z2 * C * 4) + 2 * r(z2 * N * 4)
            + r(z2 * nch * C * 4) + 2 * r(z2 * C * 4))
    assert sa.sparse_attn_cluster_workspace_size(p, cp) == want
    ci = sa.make_cluster_params(10, 20, iters=3, metric="interaction")
    nchm = 1   # ceil(1000 / 2048)
    assert sa.sparse_attn_cluster_workspace_size(p, ci) == \
        want + r(z2 * D * D * 4) + r(z2 * nchm * D * D * 4)
    assert sa.sparse_attn_cluster_workspace_size(sa.make_params(0, 2, 1000, 128), cp) == 0


@pytest.mark.parametrize("pkw,ckw,code", [
    (dict(dtype="f32"), {}, sa.SA_ERR_UNSUPPORTED),
    (dict(causal=True), {}, sa.SA_ERR_INVALID_ARG),
    ({}, dict(clusters_q=0), sa.SA_ERR_INVALID_ARG),
    ({}, dict(clusters_k=1001), sa.SA_ERR_INVALID_ARG),
    ({}, dict(clusters_q=5000), sa.SA_ERR_INVALID_ARG),
    ({}, dict(iters=0), sa.SA_ERR_INVALID_ARG),
    ({}, dict(iters=65), sa.SA_ERR_INVALID_ARG),
    ({}, dict(metric=7), sa.SA_ERR_INVALID_ARG),
    (dict(D=96), {}, sa.SA_ERR_UNSUPPORTED),
])
def test_cluster_invalid_args_rejected_before_launch(pkw, ckw, code):
    kw = dict(B=1, H=2, N=1000, D=128)
    kw.update(pkw)
    p = sa.make_params(kw.pop("B"), kw.pop("H"), kw.pop("N"), kw.pop("D"), **kw)
    c = dict(clusters_q=8, clusters_k=16, iters=2, metric="interaction")
    c.update(ckw)
    cp = sa.make_cluster_params(**c)
    fake = 1 << 20
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_cluster(p, cp, fake, fake, sa.make_reorder(fake, fake), fake,
                               ws_bytes=1 << 40, stream=0)
    assert e.value.code == code


def test_cluster_and_permute_pointer_errors():
    p = sa.make_params(1, 2, 1000, 128)
    cp = sa.make_cluster_params(8, 16)
    fake = 1 << 20
    cases = [
        (dict(q=None), sa.SA_ERR_INVALID_ARG),
        (dict(out=sa.make_reorder(None, fake)), sa.SA_ERR_INVALID_ARG),
        (dict(ws_bytes=64), sa.SA_ERR_WORKSPACE),
        (dict(k=fake + 4), sa.SA_ERR_INVALID_ARG),
    ]
    for over, code in cases:
        a = dict(q=fake, k=fake, out=sa.make_reorder(fake, fake), ws=fake, ws_bytes=1 << 40)
        a.update(over)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_cluster(p, cp, a["q"], a["k"], a["out"], a["ws"], stream=0,
                                   ws_bytes=a["ws_bytes"])
        assert e.value.code == code
    for args, code in [((fake, fake, 0, fake, 3), sa.SA_ERR_INVALID_ARG),
                       ((fake, fake, 2, fake, 2), sa.SA_ERR_INVALID_ARG),
                       ((fake, None, 0, fake + 2048, 2), sa.SA_ERR_INVALID_ARG),
                       ((fake, fake, 0, fake, 2), sa.SA_ERR_INVALID_ARG),      # x == y
                       ((fake + 8, fake, 1, fake + 4096, 2), sa.SA_ERR_INVALID_ARG)]:
        x, perm, inv, y, eb = args
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_permute(p, x, perm, inv, y, stream=0, elem_bytes=eb)
        assert e.value.code == code
    # empty problems enqueue nothing
    sa.sparse_attn_cluster(sa.make_params(1, 0, 1000, 128), cp, None, None,
                           sa.make_reorder(None, None), None, stream=0)
    sa.sparse_attn_permute(sa.make_params(1, 2, 0, 128), None, None, 0, None, stream=0,
                           elem_bytes=2)


def _pack(lists, nkb):
    idx = np.full((len(lists), nkb), -1, dtype=np.int32)
    cnt = np.zeros(len(lists), dtype=np.int32)
    for i, lst in enumerate(lists):
        idx[i, :len(lst)] = lst
        cnt[i] = len(lst)
    return idx, cnt


@pytest.mark.parametrize("causal,keep", [(False, 0), (True, 0), (False, 2), (True, 1)])
def test_check_mask_accepts_predicted_masks_and_names_bad_rows(causal, keep):
    import oracle as O
    rng = np.random.default_rng(31)
    N, D = 1000, 64
    Q, K = (rng.standard_normal((N, D)) for _ in range(2))
    pred = O.predict_head(Q, K, O.Params(causal=causal, tau=0.9, keep_prefix_kblocks=keep))
    p = sa.make_params(1, 1, N, D, causal=causal, keep_prefix_kblocks=keep)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    idx, cnt = _pack(pred["kept"], nkb)
    assert sa.sparse_attn_check_mask(p, idx, cnt) == -1
    F = pred["forced"]
    i = nqb - 2
    lst = [int(x) for x in pred["kept"][i]]
    nf = int(F[i].sum())
    adm = pred["adm"][i]
    bad = {"count zero": (lst[:0], None), "repeat": (lst + [lst[-1]], None),
           "out of range": (lst[:-1] + [nkb], None), "negative": (lst[:-1] + [-1], None)}
    if causal:
        bad["future block"] = (lst[:-1] + [int(np.flatnonzero(~adm)[0])], None)
        bad["too many"] = (list(np.flatnonzero(adm)) + [int(np.flatnonzero(~adm)[0])], None)
    if nf >= 1 and len(lst) > nf:
        bad["forced not first"] = (lst[nf:nf + 1] + lst[:nf] + lst[nf + 1:], None)
        bad["forced missing"] = ([j for j in lst if not F[i, j]] or lst[nf:], None)
    for why, (new, _) in bad.items():
        lists = [list(x) for x in pred["kept"]]
        lists[i] = new
        bidx, bcnt = _pack(lists, nkb) if len(new) <= nkb else (None, None)
        if bidx is None:
            continue
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_check_mask(p, bidx, bcnt)
        assert e.value.code == sa.SA_ERR_INVALID_ARG, why
        assert f"row {i}" in sa.sparse_attn_last_error(), why


def test_check_mask_rows_count_batch_and_heads():
    p = sa.make_params(2, 3, 300, 128)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    idx = np.tile(np.arange(nkb, dtype=np.int32), (2, 3, nqb, 1))
    cnt = np.full((2, 3, nqb), nkb, dtype=np.int32)
    assert sa.sparse_attn_check_mask(p, idx, cnt) == -1
    cnt[1, 2, 1] = 0  # the last row of the last head of the second batch
    with pytest.raises(sa.SparseAttnError):
        sa.sparse_attn_check_mask(p, idx, cnt)
    assert f"row {1 * 3 * nqb + 2 * nqb + 1}" in sa.sparse_attn_last_error()

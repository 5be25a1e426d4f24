"""Runs the library's two stages on host arrays through the C ABI and brings
every output back as numpy.  Used by the GPU tests only."""
from __future__ import annotations

import math

import numpy as np
import torch

import block_mean_pool_amd as sa


def to_device(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def run(Q, K, V, *, dtype="bf16", causal=False, tau=0.95, lam=-5.0, rule="topcdf",
        prec="native", keep_prefix_kblocks=0, sm_scale=0.0, layout="bhnd",
        block_prob=True, want_lse=True, want_skips=True, forward=True,
        skip_rule="lambda", recall=1.0, topk_blocks=0, group_rows=32):
    """Q, K, V: float32 arrays [B, H, N, D] holding dtype-representable values.
    ``layout="bnhd"`` stores the tensors as [B, N, H, D] and passes strides."""
    B, H, N, D = Q.shape
    if layout == "bhnd":
        q, k, v = (to_device(x, dtype) for x in (Q, K, V))
        strides = (0, 0, 0)
        o = torch.empty_like(q)
        views = (q, k, v, o)
    else:
        q, k, v = (to_device(np.transpose(x, (0, 2, 1, 3)), dtype) for x in (Q, K, V))
        strides = (N * H * D, D, H * D)
        o = torch.empty_like(q)
        views = (q, k, v, o)
    kw = dict(dtype=dtype, causal=causal, tau=tau, lam=lam, rule=rule, prec=prec,
              keep_prefix_kblocks=keep_prefix_kblocks, sm_scale=sm_scale, strides=strides,
              skip_rule=skip_rule, recall=recall, topk_blocks=topk_blocks,
              lambda_group_rows=group_rows)
    p = sa.make_params(B, H, N, D, **kw)
    p32 = sa.make_params(B, H, N, D, o_fp32=True, **kw)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    pws, fws = sa.sparse_attn_workspace_size(p)
    dev = q.device
    kept_idx = torch.full((B, H, nqb, nkb), -1, dtype=torch.int32, device=dev)
    kept_cnt = torch.full((B, H, nqb), -1, dtype=torch.int32, device=dev)
    bp = torch.full((B, H, nqb, nkb), -1.0, dtype=torch.float32, device=dev) if block_prob else None
    ws_p = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    mask = sa.make_mask(kept_idx, kept_cnt, bp)
    sa.sparse_attn_predict(p, views[0], views[1], mask, ws_p)
    out = {"params": p, "nqb": nqb, "nkb": nkb}
    if forward:
        ws_f = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev) if want_lse else None
        nw = (nkb + 31) // 32
        slots = 128 // group_rows
        skips = (torch.zeros((B, H, nqb, slots, nw), dtype=torch.int32, device=dev)
                 if want_skips else None)
        # fp32 O: the computed result, compared with the oracle
        o32 = torch.empty(views[3].shape, dtype=torch.float32, device=dev)
        sa.sparse_attn_forward(p32, views[0], views[1], views[2], mask, o32, lse, skips, ws_f)
        # O in the storage dtype: must equal the fp32 result rounded
        sa.sparse_attn_forward(p, views[0], views[1], views[2], mask, views[3], None, None, ws_f)
    torch.cuda.synchronize()
    cnt = kept_cnt.cpu().numpy()
    idx = kept_idx.cpu().numpy()
    out["kept_cnt"] = cnt
    out["kept"] = [[idx[b, h, i, :cnt[b, h, i]].astype(np.int64) for i in range(nqb)]
                   for b in range(B) for h in range(H)]
    if block_prob:
        out["block_prob"] = bp.cpu().numpy()
    ws_host = ws_p.cpu().numpy()
    nq_bytes = B * H * nqb * D * 4
    out["qbar"] = ws_host[:nq_bytes].view(np.float32).reshape(B, H, nqb, D)
    koff = (nq_bytes + 255) // 256 * 256
    out["kbar"] = ws_host[koff:koff + B * H * nkb * D * 4].view(np.float32).reshape(B, H, nkb, D)
    if forward:
        o, o32h = views[3], o32
        if layout != "bhnd":
            o, o32h = o.permute(0, 2, 1, 3), o32.permute(0, 2, 1, 3)
        out["O"] = o32h.cpu().numpy()
        out["O_store"] = o.float().cpu().numpy()
        if want_lse:
            out["lse"] = lse.cpu().numpy()
        if want_skips:
            sb = skips.cpu().numpy().view(np.uint32)
            lists = []
            for b in range(B):
                for h in range(H):
                    per = []
                    for i in range(nqb):
                        c = cnt[b, h, i]
                        t = np.arange(c)
                        bits = (sb[b, h, i][:, t // 32] >> (t % 32).astype(np.uint32)) & 1
                        per.append(bits.T.astype(bool))  # [c, 128 / G]
                    lists.append(per)
            out["skips"] = lists
        if prec in ("i8fp8", "i4fp8", "i8mxfp8"):
            wf = ws_f.cpu().numpy()
            bh = B * H
            def rup(x):
                return (x + 255) // 256 * 256
            o_qc = 0
            o_kc = o_qc + rup(bh * N * D)
            o_vt = o_kc + rup(bh * N * D)
            o_sq = o_vt + rup(bh * nkb * D * 64)
            o_sk = o_sq + rup(bh * nqb * 4)
            o_sv = o_sk + rup(bh * nkb * 4)
            out["qc"] = wf[o_qc:o_qc + bh * N * D].view(np.int8).reshape(B, H, N, D)
            out["kc"] = wf[o_kc:o_kc + bh * N * D].view(np.int8).reshape(B, H, N, D)
            out["vt"] = wf[o_vt:o_vt + bh * nkb * D * 64].reshape(B, H, nkb, D, 64)
            out["sq"] = wf[o_sq:o_sq + bh * nqb * 4].view(np.float32).reshape(B, H, nqb)
            out["sk"] = wf[o_sk:o_sk + bh * nkb * 4].view(np.float32).reshape(B, H, nkb)
            out["sv"] = wf[o_sv:o_sv + bh * nkb * 4].view(np.float32).reshape(B, H, nkb)
    return out


def lam_value(lam):
    return -math.inf if lam is None else lam

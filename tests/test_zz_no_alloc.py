"""GPU check of sparse_attn_predict_noalloc (stage one with the library's
static scratch instead of a caller workspace) through the C ABI: two calls
in a row, the second on a smaller problem, each against
sparse_attn_predict with a caller workspace on the same inputs -- kept
lists, counts and the predicted map bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_mean_pool_amd as sa  # noqa: E402
from synth import Workload  # noqa: E402


def _inputs(w):
    Q, K, _ = w.tensors()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return tuple(torch.from_numpy(x).to(dt).cuda() for x in (Q, K))


def _mask(p, dev):
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    idx = torch.full((p.B, p.H, nqb, nkb), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((p.B, p.H, nqb), -7, dtype=torch.int32, device=dev)
    bp = torch.full((p.B, p.H, nqb, nkb), -1.0, dtype=torch.float32, device=dev)
    return idx, cnt, bp, sa.make_mask(idx, cnt, bp)


def _host(idx, cnt, bp):
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    i = idx.cpu().numpy()
    kept = [i[b, h, q, :c[b, h, q]] for b in range(c.shape[0]) for h in range(c.shape[1])
            for q in range(c.shape[2])]
    return c, kept, bp.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("first,second", [
    (Workload("noalloc_big", 601, 1, 8, 8000, 128, "bf16", grid=(10, 20, 40), tau=0.9),
     Workload("noalloc_small", 602, 2, 2, 1000, 64, "bf16", structure="lm", causal=True,
              tau=0.95, keep_prefix_kblocks=1)),
])
def test_noalloc_predict_matches_predict_twice(first, second):
    for w in (first, second):
        print(f"[case] no-alloc predict {w.name} B={w.B} H={w.H} N={w.N} D={w.D}", flush=True)
        q, k = _inputs(w)
        p = sa.make_params(w.B, w.H, w.N, w.D, dtype=w.dtype, causal=w.causal, tau=w.tau,
                           keep_prefix_kblocks=w.keep_prefix_kblocks)
        pws, _ = sa.sparse_attn_workspace_size(p)
        assert pws <= 64 << 20
        ws = torch.empty(pws, dtype=torch.uint8, device=q.device)
        ref = _mask(p, q.device)
        sa.sparse_attn_predict(p, q, k, ref[3], ws)
        got = _mask(p, q.device)
        sa.sparse_attn_predict_noalloc(p, q, k, got[3])
        rc, rk, rb = _host(*ref[:3])
        gc, gk, gb = _host(*got[:3])
        np.testing.assert_array_equal(gc, rc)
        assert all(np.array_equal(a, b) for a, b in zip(gk, rk))
        np.testing.assert_array_equal(gb, rb)


def test_noalloc_rejects_problems_beyond_its_scratch():
    # 24 heads x (2048 + 4096) blocks x 128 x 4 bytes of block means, about
    # 75.5 MB > 64 MiB
    p = sa.make_params(1, 24, 262144, 128)
    assert sa.sparse_attn_workspace_size(p)[0] > 64 << 20
    fake = 1 << 20  # never dereferenced: the size check comes first
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_predict_noalloc(p, fake, fake, sa.make_mask(fake, fake), stream=0)
    assert e.value.code == sa.SA_ERR_WORKSPACE
    assert "64" in sa.sparse_attn_last_error() or "67108864" in sa.sparse_attn_last_error()

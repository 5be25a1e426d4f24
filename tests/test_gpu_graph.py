"""GPU check that the two stages can be captured in a HIP graph and replayed:
stage one through sparse_attn_predict_noalloc (no workspace to allocate) and
stage two through sparse_attn_forward, captured once with torch's graph
capture on the stream the binding passes, then replayed several times with
the program's own eager work and synchronisations between the replays.
Every replay must reproduce the eager call's mask, lse and output bit for bit
(the kernels are deterministic and the library enqueues no memset or copy),
and a replay after the inputs are overwritten in place must follow the new
inputs (the graph reads its buffers at replay time)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_mean_pool_amd as sa  # noqa: E402
from synth import Workload  # noqa: E402


def _tensors(w, dev):
    Q, K, V = w.tensors()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return [torch.from_numpy(x).to(dt).to(dev) for x in (Q, K, V)]


class _Run:
    def __init__(self, w, prec, dev):
        self.p = sa.make_params(w.B, w.H, w.N, w.D, dtype=w.dtype, causal=w.causal, tau=w.tau,
                                lam=w.lam, prec=prec)
        nqb, nkb = sa.sparse_attn_mask_shape(self.p)
        _, fws = sa.sparse_attn_workspace_size(self.p)
        self.idx = torch.full((w.B, w.H, nqb, nkb), -1, dtype=torch.int32, device=dev)
        self.cnt = torch.full((w.B, w.H, nqb), -1, dtype=torch.int32, device=dev)
        self.mask = sa.make_mask(self.idx, self.cnt)
        self.ws = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
        self.o = torch.empty((w.B, w.H, w.N, w.D),
                             dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                             device=dev)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def call(self, q, k, v):
        sa.sparse_attn_predict_noalloc(self.p, q, k, self.mask)
        sa.sparse_attn_forward(self.p, q, k, v, self.mask, self.o, self.lse, None, self.ws)

    def clear(self):
        for t in (self.idx, self.cnt):
            t.fill_(-1)
        self.o.fill_(0)
        self.lse.fill_(0)

    def host(self):
        torch.cuda.synchronize()
        return (self.cnt.cpu().numpy(), self.idx.cpu().numpy(),
                self.o.float().cpu().numpy(), self.lse.cpu().numpy())


def _same(a, b):
    cnt_a, idx_a, o_a, l_a = a
    cnt_b, idx_b, o_b, l_b = b
    np.testing.assert_array_equal(cnt_a, cnt_b)
    for (bb, h, i), c in np.ndenumerate(cnt_a):
        np.testing.assert_array_equal(idx_a[bb, h, i, :c], idx_b[bb, h, i, :c])
    np.testing.assert_array_equal(o_a.view(np.uint32), o_b.view(np.uint32))
    np.testing.assert_array_equal(l_a.view(np.uint32), l_b.view(np.uint32))


@pytest.mark.parametrize("prec", ["native", "i8mxfp8"])
def test_captured_stages_replay_bit_exact(prec):
    dev = torch.device("cuda:0")
    w = Workload("graph_field", 701, 1, 2, 1000, 128, "bf16", grid=(10, 10, 10), tau=0.9,
                 lam=-5.0)
    w2 = Workload("graph_field_2", 702, 1, 2, 1000, 128, "bf16", grid=(10, 10, 10), tau=0.9,
                  lam=-5.0)
    print(f"[case] graph replay prec={prec} N={w.N}", flush=True)
    q, k, v = _tensors(w, dev)
    q2, k2, v2 = _tensors(w2, dev)
    r = _Run(w, prec, dev)

    # eager references on both inputs (this also looks up the scratch address)
    r.call(q2, k2, v2)
    ref2 = r.host()
    r.clear()
    r.call(q, k, v)
    ref = r.host()

    # capture on a side stream, as torch's graph capture requires
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.call(q, k, v)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    r.clear()
    with torch.cuda.graph(g):
        r.call(q, k, v)
    torch.cuda.synchronize()

    for rep in range(3):
        r.clear()                            # eager work between replays
        eager_mask = _Run(w, prec, dev)      # and an eager call of the same stages
        eager_mask.call(q2, k2, v2)
        torch.cuda.synchronize()
        g.replay()
        _same(r.host(), ref)
        print(f"   replay {rep} equals the eager call", flush=True)

    # the graph reads its input buffers at replay time
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    r.clear()
    g.replay()
    _same(r.host(), ref2)
    print("   replay on overwritten inputs equals the eager call on them", flush=True)

"""Benchmark: dense-equivalent attention TFLOPS and sparsity of block-sparse
attention (predict + forward through the C ABI) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over the batch: sparse_attn_predict
(block means, block scores, mask) then sparse_attn_forward (block-sparse
flash attention with the lambda skip), inputs resident in HBM.  The default
workload is the Wan-like video DiT self-attention (B=1, H=40, N=32760 from a
21x30x52 latent grid, d=128, bf16, tau=0.9, lambda=-5, non-causal) on
seeded synthetic smoothed-field Q/K and Gaussian V.

Printed: ONE JSON line with the headline metric, the roofline of the forward
kernel (executed MFMA FLOPs / its average launch time, measured with HIP
events on the launch stream) and of the predictor's pooling kernel (bytes /
its launch time), a tau sweep and the other mask and skip rules, and the
CPU-baseline leg.

The CPU-baseline leg is the only part that runs the fp64 oracle (oracle/):
worker processes, forked before anything touches the GPU, time the oracle
on a bounded sample of the workload (sampled heads: stage one for the whole
head, stage two for evenly spaced query blocks under the GPU's mask and skip
decisions) and compute the dense fp64 rows of that sample.  The same leg
reports what the oracle says about the GPU's results: max-abs against the
oracle, rel-L1 against dense attention, true recall, predicted kept mass,
block sparsity and P.V skip fraction (oracle/metrics.py).  Without it
(--no-cpu-baseline) those fields are null.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import multiprocessing
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dense-equiv attention TFLOPS + sparsity at fixed rel-L1, N=32760 H=40 d=128"
# HBM traffic per launch, from two rocprofv3 --pmc passes (FETCH_SIZE x 2.000,
# WRITE_SIZE x 1.000, the factors a 1 GiB copy reads on the same counters),
# keyed by the hash of the kernel sources it was measured on: a changed
# kernel reports null until it is measured again.
MEASURED_TRAFFIC = {
    # (kernel kind, workload, Q.K^T mode) -> (source hash, bytes read, bytes written)
    ("bf16", "wan_video", "native"): ("aba23ef178feac18", 111_721_873_280, 335_469_792),
    ("bf16", "hunyuan_video", "native"): ("aba23ef178feac18", 983_999_294_976, 731_502_560),
    ("i8fp8", "quant_long", "i8fp8"): ("18544d539b55e1cd", 96_777_516_928, 268_435_456),
    ("i8fp8", "quant_long", "i8mxfp8"): ("18544d539b55e1cd", 96_733_693_056, 268_435_456),
    ("pool", "wan_video", "native"): ("4c1ce0d8f8ed753a", 671_001_856, 15_728_640),
    ("pool", "hunyuan_video", "native"): ("4c1ce0d8f8ed753a", 1_463_053_440, 34_308_096),
    ("pool", "quant_long", "i8fp8"): ("4c1ce0d8f8ed753a", 536_935_808, 12_582_912),
    ("pool", "quant_long", "i8mxfp8"): ("4c1ce0d8f8ed753a", 536_936_576, 12_582_912),
}
# the forward kernel that dominates each kind of workload, and its sources;
# "pool" is the predictor's HBM-bound first step
FORWARD_KERNELS = {
    "bf16": ("attn_pipe_kernel (sparse_attn_forward)", ("attn_pipe.hip", "attn_common.h")),
    "f32": ("attn_kernel (sparse_attn_forward)", ("attn.hip", "attn_common.h")),
    "i8fp8": ("attn_q_kernel (sparse_attn_forward)", ("attn_q.hip", "attn_common.h")),
}
POOL_KERNEL = ("pool_kernel (sparse_attn_pool, first step of sparse_attn_predict)",
               ("pool.hip", "sa_device.h"))
PEAK_BF16_TFLOPS = 2500.0
PEAK_I8FP8_TOPS = 5000.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
PEAK_CLOCK_GHZ = 2.4  # the engine clock the published peaks assume
MAX_WORKERS = 16      # the host CPU share of one GPU on the measurement boxes
SAMPLE_HEADS = 16     # heads the CPU-baseline leg runs the oracle on
SAMPLE_BLOCKS = 16    # evenly spaced query blocks of each sampled head


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan_video")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--skip-rule", default="lambda", choices=("lambda", "recall"),
                    help="stage-two skip rule of the timed configuration")
    ap.add_argument("--prec", default=None, choices=QUANT_PRECS,
                    help="quantised Q.K^T mode of a quantised workload (default: the "
                         "workload's own)")
    ap.add_argument("--recall", type=float, default=0.95,
                    help="target recall of the recall skip rule")
    ap.add_argument("--lam", type=float, default=None,
                    help="lambda of the timed configuration (default: the workload's; "
                         "--lam=-inf switches the skip off), for per-kernel profiles")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the GEMM / copy reference measurements")
    ap.add_argument("--stage", default="all", choices=("all", "cluster"),
                    help="cluster: time only sparse_attn_cluster (interaction metric, "
                         "NQB / NKB clusters, 4 passes) on the workload and print its "
                         "timing line (for per-kernel profiles)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, launch a plain copy kernel (torch.neg on "
                         "fp32) of this many MiB, 3 times: a known-size reference "
                         "for the HBM byte counters")
    return ap.parse_args()


# quantised Q.K^T modes that run attn_q_kernel: INT8 codes with absmax/448
# FP8 V scales, and INT8 codes with power-of-two V scales applied by the
# scaled FP8 MFMA
QUANT_PRECS = ("i8fp8", "i8mxfp8")


def forward_kind(w):
    return "i8fp8" if w.prec in QUANT_PRECS else w.dtype


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "sa_build", os.path.join(ROOT, "block_mean_pool_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def kernel_source_hash(kind):
    """Hash of a kernel's sources and of the compiler flags the build gives
    them (which shape the compiled kernel); ``kind`` is a FORWARD_KERNELS key
    or "pool"."""
    import hashlib
    b = _build_module()
    h = hashlib.sha256()
    files = POOL_KERNEL[1] if kind == "pool" else FORWARD_KERNELS[kind][1]
    for name in files:
        h.update(open(os.path.join(ROOT, "block_mean_pool_amd", "csrc", name), "rb").read())
        if name.endswith(".hip"):
            h.update(repr((b.FLAGS, b.PER_FILE_FLAGS.get(name, []))).encode())
    return h.hexdigest()[:16]


PROBE_LIB = os.path.join(ROOT, "probe", "libsa_probe.so")


def load_probe():
    """The benchmark's measurement helpers (clock sampler, MFMA loop), built
    beside bench.py; None when absent."""
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.sa_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_void_p]
    lib.sa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


class ClockSampler:
    """Reads the engine clock while other work runs: one wavefront on a side
    stream (default priority) samples the engine-clock counter against the
    constant-rate real-time counter over a bounded window."""

    def __init__(self, torch, probe, dev):
        self.torch, self.probe = torch, probe
        self.S = probe.sa_probe_clock_max_samples()
        self.buf = torch.zeros(2 * self.S + 1, dtype=torch.int64, device=dev)
        self.side = torch.cuda.Stream(device=dev)
        self.rt_hz = self._calibrate()

    def _launch(self, ticks):
        rc = self.probe.sa_probe_clock(self.buf.data_ptr(), int(ticks), max(1, int(ticks) // 64),
                                       self.side.cuda_stream)
        if rc:
            raise RuntimeError(f"clock sampler launch failed (hipError {rc})")

    def _samples(self):
        b = self.buf.cpu().numpy().view(np.uint64)
        n = int(b[2 * self.S])
        return b[0:2 * n:2].astype(np.float64), b[1:2 * n:2].astype(np.float64)

    def _calibrate(self):
        """Real-time counter rate: the sampler alone over 5e6 ticks, timed
        with events on its stream."""
        torch = self.torch
        self._launch(1000)  # first launch loads the code object: keep it out of the timing
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.side)
        self._launch(5_000_000)
        e1.record(self.side)
        torch.cuda.synchronize()
        _, r = self._samples()
        return (r[-1] - r[0]) / (e0.elapsed_time(e1) * 1e-3)

    def around(self, work, window_s):
        """Engine clock (GHz) over window_s seconds of real time, sampled
        while work() (launched right after the sampler) runs."""
        torch = self.torch
        torch.cuda.synchronize()
        self._launch(window_s * self.rt_hz)
        work()
        torch.cuda.synchronize()
        m, r = self._samples()
        if len(m) < 2 or r[-1] <= r[0]:
            return None
        return float((m[-1] - m[0]) / (r[-1] - r[0]) * self.rt_hz / 1e9)


def mfma_loop_peak(torch, probe, sampler, dev):
    """Dense MFMA loop on every SIMD (four wavefronts each, eight independent
    32x32x16 bf16 chains per wavefront): TFLOP/s and the clock it ran at."""
    blocks, iters = 1024, 40000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    for it in (2000, iters):  # warm-up, then the timed size
        rc = probe.sa_probe_mfma(out.data_ptr(), blocks, it, stream)
        if rc:
            raise RuntimeError(f"MFMA loop launch failed (hipError {rc})")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run():
        e0.record()
        for _ in range(3):
            probe.sa_probe_mfma(out.data_ptr(), blocks, iters, stream)
        e1.record()

    clock = sampler.around(run, 0.03)
    flops = 3.0 * blocks * 4 * iters * probe.sa_probe_mfma_chains() * 2 * 32 * 32 * 16
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, clock


def measured_peaks(torch, dev, sampler=None, probe=None):
    """What this GPU reaches on a plain bf16 GEMM (torch.matmul, 8192^3), a
    plain 1 GiB fp32 copy and a dense MFMA loop, with the engine clock of the
    GEMM and the loop: context for the roofline fractions, which are taken
    against the published peaks."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def gemms():
        e0.record()
        for _ in range(10):
            torch.matmul(a, b)
        e1.record()

    gemm_clock = sampler.around(gemms, 0.005) if sampler else None
    if sampler is None:
        gemms()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    x = torch.ones(1 << 28, device=dev, dtype=torch.float32)
    y = torch.empty_like(x)
    y.copy_(x)
    e0.record()
    for _ in range(10):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * x.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    out = {"bf16_gemm_8192_tflops": round(gemm, 1), "copy_1gib_gbps": round(copy, 1),
           "published": {"bf16_dense_tflops": PEAK_BF16_TFLOPS, "hbm_gbps": PEAK_HBM_GBPS}}
    if sampler is not None:
        loop, loop_clock = mfma_loop_peak(torch, probe, sampler, dev)
        out.update({"bf16_gemm_clock_ghz": _r3(gemm_clock),
                    "bf16_mfma_loop_tflops": round(loop, 1),
                    "bf16_mfma_loop_clock_ghz": _r3(loop_clock),
                    "realtime_counter_mhz": round(sampler.rt_hz / 1e6, 3)})
    return out


def json_number(x):
    """A float for the JSON line: non-finite values (lambda = -inf) as their
    string, so the line stays strict JSON."""
    return x if math.isfinite(x) else str(x)


def _r3(x):
    return None if x is None else round(x, 3)


def _rd(x, n=6):
    return None if x is None else round(float(x), n)


def data_description(w):
    what = {
        "field": "smoothed-field Q/K on a %s latent grid%s, Gaussian V; stands in for the "
                 "pages' video DiT self-attention" % (
                     "x".join(map(str, w.grid)) if w.grid else "1-D",
                     f" plus {w.n_text} Gaussian text tokens" if w.n_text else ""),
        "lm": "AR(1) rho=0.95 Q/K with an attention sink on tokens 0-3, Gaussian V; stands "
              "in for LM prefill",
        "centroid": "Q/K around 8 centroids in runs of 64, Gaussian V",
        "gauss": "Gaussian Q/K/V",
    }[w.structure]
    from synth.workloads import BASE_SEED
    return (f"synthetic, seeded ({what}; numpy PCG64(SeedSequence({BASE_SEED} + {w.index})), "
            f"one child per (b, h))")


def gen_inputs(w, threads=16):
    with ThreadPoolExecutor(threads) as ex:
        heads = list(ex.map(lambda bh: w.head(bh // w.H, bh % w.H), range(w.B * w.H)))
    shape = (w.B, w.H, w.N, w.D)
    return tuple(np.stack([x[t] for x in heads]).reshape(shape) for t in range(3))


def sample_blocks(nqb, n=SAMPLE_BLOCKS):
    """n query blocks evenly spaced over the sequence (first and last
    included)."""
    return sorted({int(round(x)) for x in np.linspace(0, nqb - 1, min(n, nqb))})


def sample_heads(H, n=SAMPLE_HEADS):
    """n heads evenly spaced over 0 .. H - 1 (first and last included)."""
    return sorted({int(round(x)) for x in np.linspace(0, H - 1, min(n, H))})


def block_rows(blocks, N):
    return np.concatenate([np.arange(i * 128, min(N, (i + 1) * 128)) for i in blocks])


class Sample:
    """The rows the CPU-baseline leg evaluates: evenly spaced query blocks of
    evenly spaced heads (batch 0)."""

    def __init__(self, w, n_heads=SAMPLE_HEADS, n_blocks=SAMPLE_BLOCKS):
        self.nqb = (w.N + 127) // 128
        self.heads = sample_heads(w.H, n_heads)
        self.blocks = sample_blocks(self.nqb, n_blocks)
        self.rows = block_rows(self.blocks, w.N)

    def describe(self, w):
        return (f"heads {self.heads} of {w.H} (batch 0), query blocks {self.blocks} of "
                f"{self.nqb} ({len(self.rows)} rows per head)")

    def take(self, torch, o):
        """The sampled rows of an O tensor [B, H, N, D] as float64 numpy
        [len(heads), len(rows), D]."""
        hi = torch.as_tensor(self.heads, device=o.device)
        ri = torch.as_tensor(self.rows, device=o.device)
        return o[0].index_select(0, hi).index_select(1, ri).float().cpu().numpy()


class Runner:
    """Owns the device buffers of one configuration and runs the two calls."""

    def __init__(self, sa, torch, w, q, k, v, tau, skip_rule="lambda", recall=1.0, rule=None,
                 topk_blocks=0, prec=None, lam=None):
        self.sa, self.torch, self.w = sa, torch, w
        self.q, self.k, self.v = q, k, v
        self.o = torch.empty_like(q)
        kw = dict(dtype=w.dtype, causal=w.causal, tau=tau, lam=w.lam if lam is None else lam,
                  rule=rule or w.rule,
                  prec=prec or w.prec, topk_blocks=topk_blocks,
                  keep_prefix_kblocks=w.keep_prefix_kblocks, skip_rule=skip_rule,
                  recall=recall)
        self.p = sa.make_params(w.B, w.H, w.N, w.D, **kw)
        self.p32 = sa.make_params(w.B, w.H, w.N, w.D, o_fp32=True, **kw)
        self.nqb, self.nkb = sa.sparse_attn_mask_shape(self.p)
        pws, fws = sa.sparse_attn_workspace_size(self.p)
        dev = q.device
        self.idx = torch.empty((w.B, w.H, self.nqb, self.nkb), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((w.B, w.H, self.nqb), dtype=torch.int32, device=dev)
        self.ws_p = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
        self.mask = sa.make_mask(self.idx, self.cnt)

    def predict(self):
        self.sa.sparse_attn_predict(self.p, self.q, self.k, self.mask, self.ws_p)

    def forward(self, skips=None):
        self.sa.sparse_attn_forward(self.p, self.q, self.k, self.v, self.mask, self.o, None,
                                    skips, self.ws_f)

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.predict()
            self.forward()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for a, b, c in ev:
            a.record()
            self.predict()
            b.record()
            self.forward()
            c.record()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total = start.elapsed_time(end)
        pred = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
        fwd = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
        return total / steps, pred, fwd, wall

    def time_graph(self, steps):
        """A step (stage one through the allocation-free predict, then stage
        two) captured once in a HIP graph and replayed: mean time per replay,
        HIP events on the replay stream; None where the allocation-free
        predict's scratch cannot hold the problem."""
        torch, sa = self.torch, self.sa
        if sa.sparse_attn_workspace_size(self.p)[0] > (64 << 20):
            return None

        def step():
            sa.sparse_attn_predict_noalloc(self.p, self.q, self.k, self.mask)
            self.forward()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_pool(self, steps):
        """Mean time of the predictor's pooling kernel alone
        (sparse_attn_pool), HIP events on the launch stream."""
        torch = self.torch
        for _ in range(2):
            self.sa.sparse_attn_pool(self.p, self.q, self.k, self.ws_p)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            self.sa.sparse_attn_pool(self.p, self.q, self.k, self.ws_p)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def decisions(self, sample=None):
        """One untimed predict + forward writing skip bits and an fp32 O (the
        same arithmetic as the timed calls; only the store differs): kept
        counts and skip words of every query block, and for the sampled heads
        their kept lists, skip bits and fp32 O rows."""
        torch = self.torch
        nw = (self.nkb + 31) // 32
        skips = torch.zeros((self.w.B, self.w.H, self.nqb, 4, nw), dtype=torch.int32,
                            device=self.q.device)
        o32 = torch.empty(self.q.shape, dtype=torch.float32, device=self.q.device)
        self.predict()
        self.sa.sparse_attn_forward(self.p32, self.q, self.k, self.v, self.mask, o32, None,
                                    skips, self.ws_f)
        torch.cuda.synchronize()
        out = dict(cnt=self.cnt.cpu().numpy().astype(np.int64),
                   bits=skips.cpu().numpy().view(np.uint32))
        if sample is not None:
            idx = self.idx[0].index_select(0, torch.as_tensor(sample.heads, device=self.q.device))
            idx = idx.cpu().numpy()
            out["kept"] = {h: [idx[n, i, :out["cnt"][0, h, i]].astype(np.int64)
                               for i in range(self.nqb)] for n, h in enumerate(sample.heads)}
            out["o32_rows"] = sample.take(torch, o32)
        del o32, skips
        return out


def executed_tiles(cnt, bits, N):
    """Kept tiles, and (tile, group) pairs whose P.V ran, over every query
    block: groups past the last row of a partial query block hold no rows
    and count as neither."""
    tiles = int(cnt.sum())
    nqb = cnt.shape[-1]
    real = np.array([min(4, (min(N, (i + 1) * 128) - i * 128 + 31) // 32) for i in range(nqb)])
    skipped = 0
    for t in range(int(cnt.max()) if cnt.size else 0):
        live = cnt > t  # [B, H, nqb]
        bit = ((bits[..., t // 32] >> np.uint32(t % 32)) & 1).astype(bool)  # [B, H, nqb, 4]
        bit &= np.arange(4)[None, None, None, :] < real[None, None, :, None]
        skipped += int((bit & live[..., None]).sum())
    groups = int((cnt * real[None, None, :]).sum())
    return tiles, groups, skipped


def admissible_count(w, nqb, nkb):
    if not w.causal:
        return w.B * w.H * nqb * nkb
    tot = 0
    for i in range(nqb):
        last = min(w.N, (i + 1) * 128) - 1
        tot += last // 64 + 1
    return w.B * w.H * tot


# --------------------------------------------------------------------------
# The CPU-baseline leg: the only code here that runs the fp64 oracle.  Its
# worker processes are forked before the parent initialises the GPU and
# never touch it; each regenerates its head from the seeded generator.
# --------------------------------------------------------------------------
def cpu_cores():
    """Host cores this process may use, capped at the CPU share of one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _worker_init():
    from threadpoolctl import threadpool_limits
    global _LIMIT
    _LIMIT = threadpool_limits(1)  # one BLAS thread per worker process


def _oracle_params(w, tau, skip_rule, recall, rule, topk_blocks):
    import oracle as O
    return O.Params(causal=w.causal, tau=float(np.float32(tau)), lam=float(np.float32(w.lam)),
                    rule=rule, keep_prefix_kblocks=w.keep_prefix_kblocks,
                    sm_scale=float(np.float32(1.0 / math.sqrt(w.D))), skip_rule=skip_rule,
                    recall=float(np.float32(recall)), topk_blocks=topk_blocks)


def _oracle_sparse_task(task):
    """Timed part, one head: stage one for the whole head, then stage two
    for the sampled query blocks under the GPU's kept lists and skip bits."""
    import oracle as O
    w, h, blocks, kept, skips, pkw = task
    q, k, v = w.head(0, h)
    p = _oracle_params(w, **pkw)
    nqb = len(kept)
    t0 = time.perf_counter()
    pred = O.predict_head(q, k, p)
    t1 = time.perf_counter()
    sub_kept = [kept[i] if i in blocks else np.zeros(0, dtype=np.int64) for i in range(nqb)]
    sub_skip = [skips[i] if i in blocks else np.zeros((0, 4), dtype=bool) for i in range(nqb)]
    if w.prec in QUANT_PRECS:
        Ob, _, _ = O.sparse_attention_quant_head(q, k, v, sub_kept, p, force_skip=sub_skip,
                                                 v_pow2=w.prec == "i8mxfp8")
    else:
        Ob, _, _ = O.sparse_attention_head(q, k, v, sub_kept, p, force_skip=sub_skip)
    t2 = time.perf_counter()
    return dict(h=h, t_stage1=t1 - t0, t_stage2=t2 - t1, O=Ob[block_rows(blocks, w.N)],
                mask_exact=int(sum(np.array_equal(a, b) for a, b in zip(kept, pred["kept"]))),
                pred_mass=O.predicted_kept_mass(pred["P"], kept))


def _oracle_dense_task(task):
    """Dense fp64 rows of the sampled query blocks of one head, and the true
    recall of the GPU's mask on them."""
    import oracle as O
    w, h, blocks, kept = task
    q, k, v = w.head(0, h)
    sm = 1.0 / math.sqrt(w.D)
    t0 = time.perf_counter()
    od, _ = O.dense_attention_head(q, k, v, sm, w.causal, rows=block_rows(blocks, w.N))
    t1 = time.perf_counter()
    rec = O.true_recall(q, k, kept, 128, 64, sm, w.causal, blocks=blocks)
    return dict(h=h, dense=od, t_dense=t1 - t0, recall=rec)


def _oracle_drift_task(task):
    """Dense fp64 rows of the sampled query blocks of one head for every
    call of a drifting sequence."""
    import oracle as O
    w, h, blocks, n_steps, dtheta = task
    seq = w.drift_head(0, h, n_steps, dtheta)
    rows = block_rows(blocks, w.N)
    sm = 1.0 / math.sqrt(w.D)
    return h, [O.dense_attention_head(*seq[s], sm, w.causal, rows=rows)[0]
               for s in range(n_steps)]


def decode_skips(bits, cnt):
    """Skip bits of one query block as bool [cnt, 4] (list entry, group)."""
    t = np.arange(cnt)
    return ((bits[:, t // 32] >> (t % 32).astype(np.uint32)) & 1).T.astype(bool)


class CpuBaselineLeg:
    """Forked before the GPU is touched; afterwards runs the oracle on the
    sample and reports the baseline and the oracle's view of the results."""

    def __init__(self, cores):
        self.cores = cores
        self.pool = multiprocessing.get_context("fork").Pool(cores, initializer=_worker_init)

    def close(self):
        self.pool.close()
        self.pool.join()

    def run(self, w, sample, head, others, reuse, pkw):
        import oracle as O
        # timed: the sparse path of the oracle on the sample, all workers
        tasks = []
        for h in sample.heads:
            skips = [decode_skips(head["bits"][0, h, i], head["cnt"][0, h, i])
                     if i in sample.blocks else None for i in range(sample.nqb)]
            tasks.append((w, h, sample.blocks, head["kept"][h], skips, pkw))
        workers = min(self.cores, len(tasks))
        t0 = time.perf_counter()
        sparse = self.pool.map(_oracle_sparse_task, tasks, chunksize=1)
        wall_map = time.perf_counter() - t0
        # the dense fp64 leg (the rel-L1 reference) and the true recall
        t0 = time.perf_counter()
        dense = self.pool.map(_oracle_dense_task,
                              [(w, h, sample.blocks, head["kept"][h]) for h in sample.heads],
                              chunksize=1)
        wall_dense = time.perf_counter() - t0
        drift = {}
        if reuse:
            drift = dict(self.pool.map(
                _oracle_drift_task,
                [(w, h, reuse["sample"].blocks, reuse["n_steps"], reuse["dtheta"])
                 for h in reuse["sample"].heads], chunksize=1))
        Od = np.stack([d["dense"] for d in dense])          # [heads, rows, D]
        Oo = np.stack([r["O"] for r in sparse])
        # the oracle's view of the GPU's results
        rows_per_block = [min(w.N, (i + 1) * 128) - i * 128 for i in range(sample.nqb)]
        adm = np.tile(O.admissible_counts(w.N, 128, 64, w.causal), (w.B, w.H, 1))

        def quality(res):
            out = {"sparsity": O.block_sparsity(res["cnt"], adm)}
            skl, rows = [], []
            for b in range(w.B):
                for h in range(w.H):
                    for i in range(sample.nqb):
                        skl.append(decode_skips(res["bits"][b, h, i], res["cnt"][b, h, i]))
                        rows.append(rows_per_block[i])
            out["pv_skip_fraction"] = O.skip_fraction(skl, rows, 32)
            out["rel_l1"] = O.rel_l1(res["o_rows"], Od)
            return out

        q_head = quality(head)
        rows_all = sample.rows
        n_rows = len(rows_all) * len(sample.heads)
        t_stage1 = float(np.mean([r["t_stage1"] for r in sparse]))
        t_stage2 = float(np.sum([r["t_stage2"] for r in sparse]))
        t_all = float(np.sum([r["t_stage1"] + r["t_stage2"] for r in sparse]))
        per_block = t_stage2 / (len(sample.heads) * len(sample.blocks))
        flops = 4.0 * n_rows * w.N * w.D / (2.0 if w.causal else 1.0)
        one_thread = flops / t_all
        # the workers run one head each at a time: the sample's oracle time
        # on `workers` cores is its single-thread time shared among them
        seconds = t_all / workers
        head_s = t_stage1 + per_block * sample.nqb
        baseline = {
            "value": round(flops / seconds / 1e12, 6),
            "unit": "TFLOPS (dense-equivalent)",
            "cores": workers,
            "kind": "oracle",
            "sample": (f"{sample.describe(w)}: fp64 numpy oracle, stage one for each sampled "
                       f"head plus stage two for the sampled query blocks under the GPU's mask "
                       f"and skip decisions; one head per task on {workers} worker processes "
                       f"with one BLAS thread each; value = dense-equivalent FLOPs of the "
                       f"sampled rows / (summed oracle seconds of the tasks / {workers}); "
                       f"input generation not timed"),
            "seconds": round(seconds, 3),
            "wall_seconds_with_generation": round(wall_map, 3),
            "one_thread_tflops": round(one_thread / 1e12, 6),
            "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "blas_threads_per_worker": 1,
            "seconds_per_head_one_thread": round(head_s, 3),
            "extrapolated_full_workload_s": {
                "value": round(head_s * w.B * w.H / workers, 1),
                "note": "extrapolation, not measured: seconds per head on one thread (stage one "
                        "+ every query block at the sampled per-block time) x B*H heads / "
                        "worker processes (heads are independent)"},
            "dense_fp64_leg": {"seconds": round(wall_dense, 3),
                               "seconds_per_block_one_thread": round(
                                   float(np.sum([d["t_dense"] for d in dense])) /
                                   (len(sample.heads) * len(sample.blocks)), 4),
                               "rows": n_rows},
        }
        vs = {
            "max_abs_vs_oracle": O.max_abs(head["o32_rows"], Oo),
            "rel_l1_vs_dense": q_head["rel_l1"],
            "true_recall": float(np.mean([d["recall"] for d in dense])),
            "predicted_kept_mass": {
                "mean": float(np.mean(np.concatenate([r["pred_mass"] for r in sparse]))),
                "min": float(np.min(np.concatenate([r["pred_mass"] for r in sparse])))},
            "mask_rows_exact": f"{sum(r['mask_exact'] for r in sparse)} of "
                               f"{len(sample.heads) * sample.nqb}",
            "sparsity": q_head["sparsity"],
            "pv_skip_fraction": q_head["pv_skip_fraction"],
            "sample": sample.describe(w),
        }
        other_q = {name: quality(res) for name, res in others.items()}
        reuse_q = {}
        if reuse:
            rs = reuse["sample"]
            for kk, calls in reuse["o_rows"].items():
                rels = []
                for s, o_rows in enumerate(calls):
                    dd = np.stack([drift[h][s] for h in rs.heads])
                    rels.append(O.rel_l1(o_rows, dd))
                reuse_q[kk] = rels
        return baseline, vs, other_q, reuse_q


# --------------------------------------------------------------------------
# GPU legs (no oracle)
# --------------------------------------------------------------------------
def reuse_sweep(sa, torch, w, sample, n_steps=6, ks=(1, 3, 6), dtheta=0.05, threads=16):
    """Mask reuse across calls (sparse_attn_step): a seeded drifting
    sequence of n_steps inputs (synth Workload.drift_head, a stand-in for
    successive denoising steps), run with refresh_every = k for each k; per
    k: mean time per call (stage one amortised), the number of refreshes,
    and each call's O on the sampled rows (rel-L1 against dense fp64
    attention comes from the CPU-baseline leg)."""
    dev = torch.device("cuda:0")
    shape = (n_steps, 3, 1, w.H, w.N, w.D)
    xs = torch.empty(shape, dtype=torch.bfloat16, device=dev)

    def gen(h):
        return h, w.drift_head(0, h, n_steps, dtheta)

    with ThreadPoolExecutor(threads) as ex:
        for h, seq in ex.map(gen, range(w.H)):
            for s in range(n_steps):
                for t in range(3):
                    xs[s, t, 0, h].copy_(torch.from_numpy(seq[s][t]))
    p = sa.make_params(w.B, w.H, w.N, w.D, dtype=w.dtype, causal=w.causal, tau=w.tau,
                       lam=w.lam, rule=w.rule, prec=w.prec,
                       keep_prefix_kblocks=w.keep_prefix_kblocks)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    pws, fws = sa.sparse_attn_workspace_size(p)
    idx = torch.empty((1, w.H, nqb, nkb), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, w.H, nqb), dtype=torch.int32, device=dev)
    mask = sa.make_mask(idx, cnt)
    ws_p = torch.empty(max(pws, 1), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
    o = torch.empty((1, w.H, w.N, w.D), dtype=torch.bfloat16, device=dev)
    out, o_rows = [], {}
    for k in ks:
        sched = sa.make_schedule(k, 0)
        times, refreshes, rows = [], 0, []
        for s in range(n_steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sa.sparse_attn_step(p, sched, xs[s, 0], xs[s, 1], xs[s, 2], mask, o,
                                predict_ws=ws_p, forward_ws=ws_f)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
            refreshes += sched.refreshed
            rows.append(sample.take(torch, o))
        o_rows[k] = rows
        out.append(dict(refresh_every=k, steps=n_steps, refreshes=refreshes,
                        ms_per_call=round(float(np.mean(times)), 4)))
    del xs
    return out, dict(sample=sample, n_steps=n_steps, dtheta=dtheta, o_rows=o_rows)


def reorder_sweep(sa, torch, w, q, k, v, measure_on, taus=(0.9, 0.95, 0.98), iters=4, reps=3,
                  quant=None):
    """Token reordering (sparse_attn_cluster + sparse_attn_permute) ahead of
    the two stages: per metric, the time of the clustering (NQB query and NKB
    key clusters per head, ``iters`` passes) and of the four row
    permutations, then per tau the sparsity, P.V skip share and predict +
    forward time of the pipeline run on the reordered tokens, with O
    scattered back to the original rows for the CPU-baseline leg's rel-L1."""
    p = sa.make_params(w.B, w.H, w.N, w.D, dtype=w.dtype)
    nqb, nkb = sa.sparse_attn_mask_shape(p)
    dev = q.device
    out = []
    for metric in ("interaction", "feature"):
        cp = sa.make_cluster_params(nqb, nkb, iters, metric)
        ws = torch.empty(sa.sparse_attn_cluster_workspace_size(p, cp), dtype=torch.uint8,
                         device=dev)
        pq, pk = (torch.empty((w.B, w.H, w.N), dtype=torch.int32, device=dev) for _ in range(2))
        ro = sa.make_reorder(pq, pk)
        sa.sparse_attn_cluster(p, cp, q, k, ro, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sa.sparse_attn_cluster(p, cp, q, k, ro, ws)
        e1.record()
        torch.cuda.synchronize()
        cluster_ms = e0.elapsed_time(e1) / reps
        del ws
        qp, kp, vp = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        o_back = torch.empty_like(q)
        e0.record()
        sa.sparse_attn_permute(p, q, pq, 0, qp)
        sa.sparse_attn_permute(p, k, pk, 0, kp)
        sa.sparse_attn_permute(p, v, pk, 0, vp)
        sa.sparse_attn_permute(p, q, pq, 1, o_back)   # the size of the O scatter
        e1.record()
        torch.cuda.synchronize()
        permute_ms = e0.elapsed_time(e1)
        rows = []
        for tau in taus:
            r, m = measure_on(qp, kp, vp, tau, None, lambda rr: sa.sparse_attn_permute(
                p, rr.o, pq, 1, o_back) or o_back, f"reorder_{metric}_tau{tau}")
            rows.append(dict(tau=tau, key=f"reorder_{metric}_tau{tau}",
                             sparsity=round(m["sparsity"], 5),
                             pv_skip_fraction=round(m["skip"], 5),
                             predict_forward_ms=round(m["ms"], 4)))
            del r
        if quant is not None and metric == "interaction":
            for prec in ("i8fp8", "i8mxfp8", "i4fp8"):
                r, m = measure_on(qp, kp, vp, w.tau, prec, lambda rr: sa.sparse_attn_permute(
                    p, rr.o, pq, 1, o_back) or o_back, f"reorder_{metric}_{prec}")
                quant.append(dict(order="interaction clusters", prec=prec, tau=w.tau,
                                  key=f"reorder_{metric}_{prec}",
                                  sparsity=round(m["sparsity"], 5),
                                  pv_skip_fraction=round(m["skip"], 5),
                                  forward_ms=round(m["forward_ms"], 4)))
                del r
        out.append(dict(metric=metric, clusters_q=nqb, clusters_k=nkb, iters=iters,
                        cluster_ms=round(cluster_ms, 4), permute_ms=round(permute_ms, 4),
                        by_tau=rows))
        del qp, kp, vp, o_back
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by head with no communication, so multi-GPU figures are not "
              "measured here", file=sys.stderr)
        sys.exit(2)
    from synth import make_workload
    w = make_workload(args.workload)
    if args.prec is not None:
        if w.prec not in QUANT_PRECS:
            print(f"--prec applies to quantised workloads; {w.name} computes in {w.dtype}",
                  file=sys.stderr)
            sys.exit(2)
        w = make_workload(args.workload, prec=args.prec)
    if args.lam is not None:
        w = make_workload(args.workload, prec=w.prec, lam=args.lam)
    leg = None
    if not args.no_cpu_baseline and args.stage == "all":
        # forked now, while nothing in this process has touched the GPU
        leg = CpuBaselineLeg(cpu_cores())
    try:
        run(args, w, leg)
    finally:
        if leg is not None:
            leg.close()


def run(args, w, leg):
    import torch
    import block_mean_pool_amd as sa

    print(f"[bench] generating {w.name} B={w.B} H={w.H} N={w.N} D={w.D}", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    Q, K, V = gen_inputs(w)
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(tdt).to(dev) for x in (Q, K, V))
    del Q, K, V
    dense = w.dense_flops()

    if args.stage == "cluster":
        p = sa.make_params(w.B, w.H, w.N, w.D, dtype=w.dtype)
        nqb, nkb = sa.sparse_attn_mask_shape(p)
        cp = sa.make_cluster_params(nqb, nkb, 4, "interaction")
        ws = torch.empty(sa.sparse_attn_cluster_workspace_size(p, cp), dtype=torch.uint8,
                         device=dev)
        pq, pk = (torch.empty((w.B, w.H, w.N), dtype=torch.int32, device=dev) for _ in range(2))
        ro = sa.make_reorder(pq, pk)
        for _ in range(args.warmup):
            sa.sparse_attn_cluster(p, cp, q, k, ro, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            sa.sparse_attn_cluster(p, cp, q, k, ro, ws)
        e1.record()
        torch.cuda.synchronize()
        print(json.dumps({"stage": "sparse_attn_cluster", "workload": w.name,
                          "clusters_q": nqb, "clusters_k": nkb, "iters": 4,
                          "metric": "interaction", "steps": args.steps,
                          "ms_per_call": round(e0.elapsed_time(e1) / max(args.steps, 1), 4)}),
              flush=True)
        return

    sample = Sample(w)
    captures = {}  # name -> {"cnt", "bits", "o_rows"} for the CPU-baseline leg

    def measure(tau, steps, warmup, skip_rule=None, recall=None, rule=None, topk_blocks=0,
                tensors=None, prec=None, o_view=None, key=None, lam=None):
        qq, kk, vv = tensors or (q, k, v)
        r = Runner(sa, torch, w, qq, kk, vv, tau,
                   skip_rule=skip_rule or args.skip_rule,
                   recall=args.recall if recall is None else recall, rule=rule,
                   topk_blocks=topk_blocks, prec=prec, lam=lam)
        ms, pred_ms, fwd_ms, wall = r.time_steps(steps, warmup)
        o_rows = sample.take(torch, o_view(r) if o_view else r.o)
        dec = r.decisions()
        tiles, groups, skipped = executed_tiles(dec["cnt"], dec["bits"], w.N)
        adm = admissible_count(w, r.nqb, r.nkb)
        if key is not None:
            captures[key] = dict(cnt=dec["cnt"], bits=dec["bits"], o_rows=o_rows)
        # executed MFMA work: Q.K^T on every kept tile, P.V on every group
        # that was not skipped (32 rows x 64 keys x D per group)
        flops = 2.0 * 128 * 64 * w.D * tiles + 2.0 * 32 * 64 * w.D * (groups - skipped)
        return r, dict(ms=ms, predict_ms=pred_ms, forward_ms=fwd_ms, wall=wall,
                       sparsity=1.0 - tiles / adm, skip=skipped / max(groups, 1),
                       exec_flops=flops, tiles=tiles)

    print(f"[bench] timing tau={w.tau}: {args.warmup} warmup + {args.steps} steps",
          file=sys.stderr, flush=True)
    r, m = measure(w.tau, args.steps, args.warmup)
    value = dense / (m["ms"] * 1e-3) / 1e12
    peak = PEAK_I8FP8_TOPS if w.prec in QUANT_PRECS else (
        PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS)
    achieved = m["exec_flops"] / (m["forward_ms"] * 1e-3) / 1e12
    head = r.decisions(sample)
    head["o_rows"] = sample.take(torch, r.o)
    pool_ms = r.time_pool(max(5, args.steps))
    try:
        graph_ms = r.time_graph(max(5, args.steps))
    except Exception as e:  # noqa: BLE001 -- context only
        print(f"[bench] graph replay skipped: {e}", file=sys.stderr, flush=True)
        graph_ms = None
    esz = 2 if w.dtype == "bf16" else 4
    pool_bytes = (2.0 * w.B * w.H * w.N * w.D * esz +
                  4.0 * w.B * w.H * (r.nqb + r.nkb) * w.D)
    print(f"[bench] {m['ms']:.3f} ms/step -> {value:.1f} dense-equiv TFLOPS; forward "
          f"{m['forward_ms']:.3f} ms = {achieved:.1f} TFLOP/s executed; pool {pool_ms:.4f} ms = "
          f"{pool_bytes / (pool_ms * 1e-3) / 1e9:.0f} GB/s", file=sys.stderr, flush=True)

    sweep, recall_sweep, topk_sweep = [], [], []
    few = max(3, args.steps // 4)

    # the same mask and kernel with the skip switched off (lambda = -inf):
    # every kept tile multiplies, so the forward is a dense product over the
    # kept tiles, comparable with a plain GEMM's rate on this chip
    skip_off, r_off = None, None
    if not args.no_sweep:
        r_off, ms_ = measure(w.tau, few, 1, lam=float("-inf"))
        tf = ms_["exec_flops"] / (ms_["forward_ms"] * 1e-3) / 1e12
        skip_off = {"lambda": "-inf", "forward_ms": round(ms_["forward_ms"], 4),
                    "pv_skip_fraction": round(ms_["skip"], 5),
                    "executed_flops_per_launch": ms_["exec_flops"],
                    "achieved": round(tf, 2), "frac": round(tf / peak, 4), "clock": None}
        print(f"[bench] skip off: {skip_off}", file=sys.stderr, flush=True)

    def sweep_row(key, ms_, **fields):
        return dict(**fields, key=key, sparsity=round(ms_["sparsity"], 5),
                    pv_skip_fraction=round(ms_["skip"], 5), ms_per_step=round(ms_["ms"], 4),
                    dense_equiv_tflops=round(dense / (ms_["ms"] * 1e-3) / 1e12, 2))

    if not args.no_sweep and w.name == "wan_video":
        for tau in (0.9, 0.95, 0.99):
            rs, ms_ = measure(tau, few, 1, key=f"tau{tau}")
            sweep.append(sweep_row(f"tau{tau}", ms_, tau=tau))
            del rs
            print(f"[bench] sweep tau={tau}: {sweep[-1]}", file=sys.stderr, flush=True)
        # the recall skip rule (dynamic threshold from the cumulative energy)
        # against the static lambda, at the headline tau
        for rho in (0.99, 0.95, 0.9):
            key = f"recall{rho}"
            rs, ms_ = measure(w.tau, few, 1, skip_rule="recall", recall=rho, key=key)
            recall_sweep.append(sweep_row(key, ms_, recall=rho, tau=w.tau))
            del rs
            print(f"[bench] recall rule rho={rho}: {recall_sweep[-1]}", file=sys.stderr,
                  flush=True)
        # the fixed-budget top-k mask against the cumulative-mass cut: the
        # first budget matches the mean kept count of the headline tau
        mean_kept = int(round(m["tiles"] / (w.B * w.H * r.nqb)))
        for kb in (mean_kept, r.nkb // 2, r.nkb // 4):
            key = f"topk{kb}"
            rs, ms_ = measure(w.tau, few, 1, rule="topk", topk_blocks=kb, key=key)
            topk_sweep.append(sweep_row(key, ms_, topk_blocks=kb))
            del rs
            print(f"[bench] top-k {kb}: {topk_sweep[-1]}", file=sys.stderr, flush=True)

    reuse, reuse_cap = [], None
    reorder, quant = [], []
    if not args.no_sweep and w.name == "wan_video":
        print("[bench] mask reuse across a drifting sequence", file=sys.stderr, flush=True)
        reuse, reuse_cap = reuse_sweep(sa, torch, w, Sample(w, 3, 8))
        for r_ in reuse:
            print(f"[bench] reuse {r_}", file=sys.stderr, flush=True)
        # INT8 and 4-bit Q.K^T (FP8 P.V) at the headline tau, contiguous order
        for prec in ("i8fp8", "i8mxfp8", "i4fp8"):
            key = f"contiguous_{prec}"
            rs, ms_ = measure(w.tau, few, 1, prec=prec, key=key)
            quant.append(dict(order="contiguous", prec=prec, tau=w.tau, key=key,
                              sparsity=round(ms_["sparsity"], 5),
                              pv_skip_fraction=round(ms_["skip"], 5),
                              forward_ms=round(ms_["forward_ms"], 4)))
            del rs
        print("[bench] token reordering", file=sys.stderr, flush=True)
        reorder = reorder_sweep(
            sa, torch, w, q, k, v,
            lambda qq, kk, vv, tau, prec, o_view, key: measure(
                tau, few, 1, tensors=(qq, kk, vv), prec=prec, o_view=o_view, key=key),
            quant=quant)
        for r_ in reorder:
            print(f"[bench] reorder {r_}", file=sys.stderr, flush=True)
        for r_ in quant:
            print(f"[bench] quantised Q.K^T {r_}", file=sys.stderr, flush=True)

    if not args.no_sweep and w.prec in QUANT_PRECS:
        # the other quantised mode on the same workload
        for prec in QUANT_PRECS:
            if prec == w.prec:
                continue
            key = f"workload_{prec}"
            rs, ms_ = measure(w.tau, few, 1, prec=prec, key=key)
            tops = ms_["exec_flops"] / (ms_["forward_ms"] * 1e-3) / 1e12
            quant.append(dict(order="contiguous", prec=prec, tau=w.tau, key=key,
                              sparsity=round(ms_["sparsity"], 5),
                              pv_skip_fraction=round(ms_["skip"], 5),
                              forward_ms=round(ms_["forward_ms"], 4),
                              executed_tops=round(tops, 1),
                              frac=round(tops / PEAK_I8FP8_TOPS, 4)))
            del rs
            print(f"[bench] quantised Q.K^T {quant[-1]}", file=sys.stderr, flush=True)

    peaks, clock = None, None
    if not args.no_peaks:
        # context only: a failure here leaves these fields null, not the line
        sampler = probe = None
        try:
            probe = load_probe()
            sampler = ClockSampler(torch, probe, dev) if probe is not None else None
            if sampler is not None:
                # the engine clock while the timed configuration's forward
                # runs (ten untimed launches; 0.1 s of them sampled)
                ghz = sampler.around(lambda: [r.forward() for _ in range(10)], 0.1)
                if ghz:
                    clock = {"forward_ghz": round(ghz, 3),
                             "frac_at_clock": round(achieved / (peak * ghz / PEAK_CLOCK_GHZ),
                                                    4),
                             "source": "s_memtime against s_memrealtime, one wavefront on a "
                                       "side stream during ten forward launches"}
                if r_off is not None:
                    ghz = sampler.around(lambda: [r_off.forward() for _ in range(10)], 0.1)
                    if ghz:
                        skip_off["clock"] = {
                            "forward_ghz": round(ghz, 3),
                            "frac_at_clock": round(skip_off["achieved"] /
                                                   (peak * ghz / PEAK_CLOCK_GHZ), 4)}
        except Exception as e:  # noqa: BLE001
            print(f"[bench] clock reading skipped: {e}", file=sys.stderr, flush=True)
            sampler = None
        try:
            peaks = measured_peaks(torch, dev, sampler, probe)
        except Exception as e:  # noqa: BLE001
            print(f"[bench] reference peaks skipped: {e}", file=sys.stderr, flush=True)
        if skip_off is not None and peaks and peaks.get("bf16_gemm_8192_tflops") \
                and w.dtype == "bf16" and w.prec not in QUANT_PRECS:
            skip_off["vs_bf16_gemm"] = round(skip_off["achieved"] /
                                             peaks["bf16_gemm_8192_tflops"], 4)
    r_off = None  # the skip-off leg's buffers

    cpu, vs_oracle = None, None
    if leg is not None:
        print(f"[bench] CPU-baseline leg: the oracle on {sample.describe(w)} with "
              f"{leg.cores} worker processes", file=sys.stderr, flush=True)
        pkw = dict(tau=w.tau, skip_rule=args.skip_rule,
                   recall=args.recall if args.skip_rule == "recall" else 1.0, rule=w.rule,
                   topk_blocks=0)
        cpu, vs_oracle, other_q, reuse_q = leg.run(w, sample, head, captures, reuse_cap, pkw)
        for row in sweep + recall_sweep + topk_sweep + quant:
            row["rel_l1"] = _rd(other_q[row["key"]]["rel_l1"])
            row["sparsity_oracle_metric"] = _rd(other_q[row["key"]]["sparsity"], 5)
        for r_ in reorder:
            for row in r_["by_tau"]:
                row["rel_l1"] = _rd(other_q[row["key"]]["rel_l1"])
        for r_ in reuse:
            rels = reuse_q[r_["refresh_every"]]
            r_["rel_l1_mean"] = _rd(np.mean(rels))
            r_["rel_l1_max"] = _rd(np.max(rels))
        print(f"[bench] CPU baseline {cpu['value']:.4g} TFLOPS on {cpu['cores']} cores; "
              f"max-abs vs oracle {vs_oracle['max_abs_vs_oracle']:.3g}, true recall "
              f"{vs_oracle['true_recall']:.4f}", file=sys.stderr, flush=True)
    for rows in (sweep, recall_sweep, topk_sweep, quant):
        for row in rows:
            row.pop("key", None)
    for r_ in reorder:
        for row in r_["by_tau"]:
            row.pop("key", None)

    kind = forward_kind(w)
    traffic = None
    mt = MEASURED_TRAFFIC.get((kind, w.name, w.prec))
    if mt and mt[0] == kernel_source_hash(kind):
        traffic = {"read_bytes": mt[1], "written_bytes": mt[2], "total_bytes": mt[1] + mt[2],
                   "source": "rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated"}
    pool_traffic = None
    mt = MEASURED_TRAFFIC.get(("pool", w.name, w.prec))
    if mt and mt[0] == kernel_source_hash("pool"):
        pool_traffic = {"read_bytes": mt[1], "written_bytes": mt[2],
                        "total_bytes": mt[1] + mt[2],
                        "source": "rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated"}
    pool_gbps = pool_bytes / (pool_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8/fp8" if w.prec in QUANT_PRECS else w.dtype,
        "data": data_description(w),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "causal": w.causal, "tau": w.tau,
                   "lambda": json_number(w.lam), "rule": w.rule,
                   "block_q": 128, "block_k": 64, "lambda_group_rows": 32,
                   "skip_rule": args.skip_rule,
                   **({"recall": args.recall} if args.skip_rule == "recall" else {}),
                   **({"qk_precision": w.prec} if w.prec in QUANT_PRECS else {})},
        "sparsity": _rd(vs_oracle["sparsity"], 5) if vs_oracle else None,
        "pv_skip_fraction": _rd(vs_oracle["pv_skip_fraction"], 5) if vs_oracle else None,
        "rel_l1_vs_dense": _rd(vs_oracle["rel_l1_vs_dense"]) if vs_oracle else None,
        "true_recall": _rd(vs_oracle["true_recall"]) if vs_oracle else None,
        "predicted_kept_mass": ({k_: _rd(v_) for k_, v_ in
                                 vs_oracle["predicted_kept_mass"].items()}
                                if vs_oracle else None),
        "max_abs_vs_oracle": _rd(vs_oracle["max_abs_vs_oracle"], 7) if vs_oracle else None,
        "oracle_sample": vs_oracle["sample"] if vs_oracle else None,
        "mask_rows_equal_to_oracle": vs_oracle["mask_rows_exact"] if vs_oracle else None,
        "predict_ms": round(m["predict_ms"], 4),
        "graph_replay": ({"ms_per_step": round(graph_ms, 4),
                          "what": "sparse_attn_predict_noalloc + sparse_attn_forward captured "
                                  "once in a HIP graph and replayed (context: value is the "
                                  "eager path)"} if graph_ms is not None else None),
        "forward_ms": round(m["forward_ms"], 4),
        "skip_off": skip_off,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": FORWARD_KERNELS[kind][0],
                     "kernel_source_hash": kernel_source_hash(kind),
                     "executed_flops_per_launch": m["exec_flops"],
                     "clock": clock,
                     "measured_peaks": peaks},
        "roofline_predictor": {"bound": "hbm", "achieved": round(pool_gbps, 1),
                               "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                               "frac": round(pool_gbps / PEAK_HBM_GBPS, 4),
                               "traffic": pool_traffic, "kernel": POOL_KERNEL[0],
                               "kernel_source_hash": kernel_source_hash("pool"),
                               "bytes_per_launch": pool_bytes, "ms_per_launch": round(pool_ms, 5),
                               "mask_kernel_ms": round(m["predict_ms"] - pool_ms, 4)},
        "tau_sweep": sweep,
        "recall_rule_sweep": recall_sweep,
        "topk_rule_sweep": topk_sweep,
        "mask_reuse": {"sequence": "6 calls, inputs cos(0.05 s) A + sin(0.05 s) B (seeded)",
                       "rel_l1_sample": reuse_cap["sample"].describe(w) if reuse_cap else None,
                       "by_refresh_every": reuse},
        "token_reorder": reorder,
        "qk_precision": quant,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x torch.neg over {args.copy_calibration_mib} MiB "
              f"(reads and writes {n * 4} bytes each)", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()

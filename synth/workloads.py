"""Seeded generators for the five synthetic attention workloads.

Every array is drawn from ``numpy.random.Generator(PCG64(SeedSequence(s)))``
with ``s = 20261203 + workload_index``; one child sequence is spawned per
(batch, head) so that any head can be regenerated on its own.  Values are
drawn in float64, cast to float32, and (for bf16 workloads) rounded to
bfloat16 with round-to-nearest-even.  The rounded values are what both the
GPU kernels and the CPU oracle consume.

Structures (the shapes of the pages' video-DiT and LM workloads):

* ``centroid``: tokens come in runs of 64; a run takes one of 8 Gaussian
  centroids (each centroid used by two runs, run order shuffled), Q and K
  are ``2*centroid + N(0, 0.3^2)`` with independent noise.
* ``field``: a 3-D Gaussian-smoothed random field on a (t, h, w) latent
  grid (sigma = 2 cells, kernel truncated at 4 sigma, reflecting edges,
  standardised per channel), flattened row-major; Q and K are the field plus
  independent ``N(0, 0.5^2)`` noise.  Optionally ``n_text`` tokens with
  N(0, 1) Q and K are prepended.
* ``lm``: a shared AR(1) process (rho = 0.95, unit stationary variance) per
  channel plus independent N(0, 1) noise for Q and K; tokens 0..3 get an
  extra ``4*c`` with ``c ~ N(0, I)`` per head (an attention sink).

V is i.i.d. N(0, 1) everywhere.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Tuple

import numpy as np
from scipy import ndimage as _ndimage

BASE_SEED = 20261203


def _rng_children(index: int, count: int):
    ss = np.random.SeedSequence(BASE_SEED + index)
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(count)]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns float32 arrays whose values are exactly representable in bf16.
    NaN stays NaN; infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    r = (r << np.uint64(16)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.nan
    return out


def _gauss_kernel(sigma: float, truncate: float = 4.0) -> np.ndarray:
    radius = int(truncate * sigma + 0.5)
    t = np.arange(-radius, radius + 1, dtype=np.float64)
    w = np.exp(-0.5 * (t / sigma) ** 2)
    return w / w.sum()


def _smooth_axis(x: np.ndarray, axis: int, kernel: np.ndarray) -> np.ndarray:
    """Separable 1-D convolution along ``axis`` with reflecting edges
    (edge sample repeated: d c b a | a b c d | d c b a)."""
    r = (len(kernel) - 1) // 2
    n = x.shape[axis]
    pad = [(0, 0)] * x.ndim
    pad[axis] = (r, r)
    if n >= r:
        xp = np.pad(x, pad, mode="symmetric")
    else:  # very short axis: repeat reflection until wide enough
        xp = x
        while xp.shape[axis] < n + 2 * r:
            xp = np.concatenate([np.flip(xp, axis), xp, np.flip(xp, axis)], axis=axis)
        start = (xp.shape[axis] - n) // 2 - r
        xp = np.take(xp, np.arange(start, start + n + 2 * r), axis=axis)
    out = np.zeros_like(x)
    for t, w in enumerate(kernel):
        out += w * np.take(xp, np.arange(t, t + n), axis=axis)
    return out


def smoothed_field(rng: np.random.Generator, grid: Tuple[int, int, int], d: int,
                   sigma: float = 2.0) -> np.ndarray:
    """[prod(grid), d] standardised Gaussian-smoothed field, row-major (t,h,w)."""
    T, Hh, W = grid
    x = rng.standard_normal((T, Hh, W, d))
    for ax in range(3):
        # scipy's 'reflect' mode is the edge-repeating reflection used above
        x = _ndimage.gaussian_filter1d(x, sigma, axis=ax, mode="reflect",
                                       truncate=4.0)
    x = x.reshape(T * Hh * W, d)
    x -= x.mean(axis=0, keepdims=True)
    sd = x.std(axis=0, keepdims=True)
    sd[sd == 0] = 1.0
    x /= sd
    return x


def field_qk(rng: np.random.Generator, grid, d: int, noise: float = 0.5,
             n_text: int = 0):
    f = smoothed_field(rng, grid, d)
    q = f + noise * rng.standard_normal(f.shape)
    k = f + noise * rng.standard_normal(f.shape)
    if n_text:
        tq = rng.standard_normal((n_text, d))
        tk = rng.standard_normal((n_text, d))
        q = np.concatenate([tq, q], axis=0)
        k = np.concatenate([tk, k], axis=0)
    return q, k


def lm_qk(rng: np.random.Generator, n: int, d: int, rho: float = 0.95,
          sink_tokens: int = 4, sink_sigma: float = 4.0):
    e = rng.standard_normal((n, d))
    a = np.empty((n, d))
    a[0] = e[0]
    c = np.sqrt(1.0 - rho * rho)
    # AR(1) with unit stationary variance, in chunks of rows for speed
    for t in range(1, n):
        a[t] = rho * a[t - 1] + c * e[t]
    q = a + rng.standard_normal((n, d))
    k = a + rng.standard_normal((n, d))
    sink = rng.standard_normal(d)
    q[:sink_tokens] += sink_sigma * sink
    k[:sink_tokens] += sink_sigma * sink
    return q, k


def centroid_qk(rng: np.random.Generator, n: int, d: int, n_centroids: int = 8,
                run: int = 64, scale: float = 2.0, noise: float = 0.3):
    n_runs = (n + run - 1) // run
    cent = rng.standard_normal((n_centroids, d))
    ids = np.arange(n_runs) % n_centroids
    rng.shuffle(ids)
    tok = np.repeat(ids, run)[:n]
    q = scale * cent[tok] + noise * rng.standard_normal((n, d))
    k = scale * cent[tok] + noise * rng.standard_normal((n, d))
    return q, k


@dataclasses.dataclass
class Workload:
    """One attention problem: shapes, parameters and a per-head generator."""
    name: str
    index: int
    B: int
    H: int
    N: int
    D: int
    dtype: str                 # "bf16" or "f32" (storage dtype of Q/K/V/O)
    causal: bool = False
    tau: float = 0.95
    lam: float = -5.0
    rule: str = "topcdf"       # "topcdf" or "energy"
    prec: str = "native"       # "native" or "i8fp8"
    keep_prefix_kblocks: int = 0
    block_q: int = 128
    block_k: int = 64
    structure: str = "field"
    grid: Optional[Tuple[int, int, int]] = None
    n_text: int = 0
    skip_rule: str = "lambda"  # "lambda" or "recall" (stage-two skip rule)
    recall: float = 1.0        # target recall of the "recall" rule
    topk_blocks: int = 0       # budget of the "topk" mask rule
    group_rows: int = 32       # rows G per skip group of stage two

    def head(self, b: int, h: int, n: Optional[int] = None):
        """(Q, K, V) float32 arrays [N, D] for one (b, h), rounded to the
        storage dtype.  ``n`` truncates the sequence (LM / centroid only)."""
        rng = _rng_children(self.index, self.B * self.H)[b * self.H + h]
        N = self.N if n is None else n
        if self.structure == "centroid":
            q, k = centroid_qk(rng, N, self.D)
        elif self.structure == "lm":
            q, k = lm_qk(rng, N, self.D)
        elif self.structure == "field":
            q, k = field_qk(rng, self.grid, self.D, n_text=self.n_text)
            if n is not None:
                q, k = q[:n], k[:n]
        elif self.structure == "gauss":
            q = rng.standard_normal((N, self.D))
            k = rng.standard_normal((N, self.D))
        else:
            raise ValueError(self.structure)
        v = rng.standard_normal((N, self.D))
        out = []
        for x in (q, k, v):
            x = x.astype(np.float32)
            if self.dtype == "bf16":
                x = round_to_bf16(x)
            out.append(x)
        return tuple(out)

    def tensors(self, heads=None):
        """Stacked float32 arrays [B, H, N, D] (or only ``heads``, a list of
        (b, h)), as (Q, K, V)."""
        if heads is None:
            heads = [(b, h) for b in range(self.B) for h in range(self.H)]
        qs, ks, vs = [], [], []
        for (b, h) in heads:
            q, k, v = self.head(b, h)
            qs.append(q)
            ks.append(k)
            vs.append(v)
        shape = (self.B, self.H, self.N, self.D) if len(heads) == self.B * self.H \
            else (len(heads), 1, self.N, self.D)
        return (np.stack(qs).reshape(shape), np.stack(ks).reshape(shape),
                np.stack(vs).reshape(shape))

    def drift_head(self, b: int, h: int, n_steps: int, dtheta: float = 0.05):
        """A sequence of n_steps inputs for one (b, h) that drift slowly, a
        stand-in for successive denoising steps: step s mixes this head's
        draw A with an independent draw B of the same structure (seed index
        + 1000) as cos(s dtheta) A + sin(s dtheta) B, which keeps the
        per-element variance, then rounds to the storage dtype."""
        a = self.head(b, h)
        partner = dataclasses.replace(self, index=self.index + 1000, dtype="f32")
        bb = partner.head(b, h)
        out = []
        for s in range(n_steps):
            c, sn = np.cos(s * dtheta), np.sin(s * dtheta)
            step = []
            for x, y in zip(a, bb):
                z = (c * x.astype(np.float64) + sn * y.astype(np.float64)).astype(np.float32)
                step.append(round_to_bf16(z) if self.dtype == "bf16" else z)
            out.append(tuple(step))
        return out

    def dense_flops(self) -> float:
        f = 4.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2.0 if self.causal else f


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 0, 1, 2, 1024, 64, "f32", causal=False,
                          tau=0.9, lam=-5.0, structure="centroid"),
    "wan_video": Workload("wan_video", 1, 1, 40, 32760, 128, "bf16", causal=False,
                          tau=0.9, lam=-5.0, structure="field", grid=(21, 30, 52)),
    "hunyuan_video": Workload("hunyuan_video", 2, 1, 24, 119056, 128, "bf16",
                              causal=False, tau=0.95, lam=-5.0, structure="field",
                              grid=(33, 45, 80), n_text=256,
                              keep_prefix_kblocks=4),
    "lm_causal": Workload("lm_causal", 3, 1, 32, 32768, 128, "bf16", causal=True,
                          tau=0.95, lam=-5.0, structure="lm"),
    "quant_long": Workload("quant_long", 4, 1, 16, 65536, 128, "bf16",
                           causal=False, tau=0.95, lam=-5.0, rule="energy",
                           prec="i8fp8", structure="field", grid=(16, 64, 64)),
}


def make_workload(name: str, **overrides) -> Workload:
    w = dataclasses.replace(WORKLOADS[name])
    for k, v in overrides.items():
        setattr(w, k, v)
    return w

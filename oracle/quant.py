"""Quantised variant of the oracle: INT8 Q.K^T and FP8 (e4m3) P.V.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Passages: the SpargeAttn abstract calls the attention "sparse and quantized";
the DynSparse story says the filter combines with quantization.  The pages
fix no format, so the readings are:

* Q and K: one scale per (batch, head, block) -- query blocks of BQ rows,
  key blocks of BK rows -- equal to the block's absolute maximum / 127
  (1 when the block is all zero); code = round-half-even(x / scale) clamped
  to [-127, 127].  The scale and the quotient are float32 operations, the
  same precision the kernel decides the codes in.
* V: one scale per key block = absmax / 448 (1 when zero); code = e4m3 of
  the float32 quotient.
* P: multiplied by exactly 2^8 before the e4m3 conversion and by 2^-8 after
  (a plain cast would flush P below about 2^-10 to zero).  The running sum l
  uses the unquantised P.
* e4m3 is the OCP 8-bit floating point E4M3 format: 1 sign, 4 exponent bits
  with bias 7, 3 mantissa bits, no infinities, largest finite 448, smallest
  normal 2^-6, subnormals k * 2^-9.  Conversion rounds to nearest, ties to
  even, and saturates finite overflow to +-448.
* V with a power-of-two scale (``v_pow2``, the SA_PREC_I8_MXFP8 mode): the
  per-key-block scale is 2^e with e the smallest integer such that
  absmax <= 448 * 2^e (1 when the block is all zero), the E8M0 block scale
  of the OCP microscaling formats; code = e4m3(x / 2^e), an exact division.
  The pages fix no V scale, so this is an equally plain reading of "V in FP8
  e4m3" that the gfx950 scaled MFMA can apply in hardware.  In this mode the
  output is normalised by the sum of the quantised weights, O = sum of
  2^-8 e4m3(2^8 P) s_v V~ over sum of 2^-8 e4m3(2^8 P) (kept tiles, skipped
  P.V included), so O is exactly a weighted average of the quantised V rows
  with the weights the product uses; the recall rule's energies stay the
  unquantised P.
* Stage one (pooling, scores, mask) uses the unquantised inputs.
* 4-bit Q.K^T (``qmax = 7``): the PARO abstract on the search page reports
  INT4 attention once tokens are reordered.  Reading: the same per-block
  symmetric codes with absmax / 7 as the scale and codes clamped to
  [-7, 7]; the dot products stay exact integers.  gfx950 has no INT4 MFMA,
  so the kernel runs these codes on the INT8 one: the mode measures the
  accuracy of 4-bit Q.K^T, not its speed.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from .sparse_attn_oracle import Params, group_skip, n_blocks


def e4m3_round(x) -> np.ndarray:
    """Round float64 values to the nearest e4m3 value (ties to even),
    saturating at +-448.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                  # a = f * 2^E, f in [0.5, 1)
    e = np.maximum(E - 1, -6)           # binade exponent; subnormals use 2^-6's
    quantum = np.ldexp(1.0, e - 3)      # 3 mantissa bits
    r = np.rint(a / quantum) * quantum  # exact scaling by a power of two
    r = np.minimum(r, 448.0)
    out = np.copysign(r, x)
    out[np.isnan(x)] = np.nan
    return out


def e4m3_flip_slack(x, eps) -> np.ndarray:
    """How far e4m3_round can move when its argument moves by a relative
    error of at most ``eps`` (elementwise, eps >= 0): e4m3_round(x (1 + eps))
    - e4m3_round(x (1 - eps)) for x >= 0.  Rounding is monotone, so any value
    in that interval rounds within this distance of e4m3_round(x); the
    result is 0 where no rounding boundary lies in the interval.  Used to
    bound the effect of a code computed in lower precision than here."""
    x = np.asarray(x, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    return e4m3_round(x * (1.0 + eps)) - e4m3_round(x * (1.0 - eps))


def e4m3_encode(x) -> np.ndarray:
    """Bit patterns (uint8) of e4m3_round(x)."""
    r = e4m3_round(x)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.uint8) << 7
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = (a > 0) & (a < 2.0 ** -6)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.uint8)
    nrm = a >= 2.0 ** -6
    _, E = np.frexp(a[nrm])
    e = E - 1
    mant = np.rint(a[nrm] / np.ldexp(1.0, e) * 8.0 - 8.0).astype(np.int64)
    code[nrm] = ((e + 7) << 3 | mant).astype(np.uint8)
    code = code | sign
    code[np.isnan(r)] = 0x7F
    return code


def int_quantize_blocks(X, bs: int, qmax: int):
    """Per-block symmetric integer codes in [-qmax, qmax] with scale
    absmax / qmax.  Returns (codes int8 [N, d], scales float32 [NB])."""
    X = np.asarray(X, dtype=np.float32)
    N, d = X.shape
    nb = n_blocks(N, bs)
    codes = np.zeros((N, d), dtype=np.int8)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        blk = X[b * bs:min(N, (b + 1) * bs)]
        amax = np.float32(np.abs(blk).max())
        s = np.float32(amax / np.float32(qmax)) if amax > 0 else np.float32(1.0)
        q = np.rint(blk / s)                      # float32 division, half-even
        codes[b * bs:min(N, (b + 1) * bs)] = np.clip(q, -qmax, qmax).astype(np.int8)
        scales[b] = s
    return codes, scales


def int8_quantize_blocks(X, bs: int):
    """Per-block symmetric INT8 codes.  Returns (codes int8 [N, d],
    scales float32 [NB])."""
    return int_quantize_blocks(X, bs, 127)


def fp8_quantize_v_blocks(V, bk: int):
    """Per-key-block e4m3 values of V.  Returns (values float64 on the e4m3
    grid [N, d], scales float32 [NKB])."""
    V = np.asarray(V, dtype=np.float32)
    N, d = V.shape
    nb = n_blocks(N, bk)
    vals = np.zeros((N, d), dtype=np.float64)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        blk = V[b * bk:min(N, (b + 1) * bk)]
        amax = np.float32(np.abs(blk).max())
        s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        vals[b * bk:min(N, (b + 1) * bk)] = e4m3_round((blk / s).astype(np.float64))
        scales[b] = s
    return vals, scales


def pow2_scale(amax: float, top: float = 448.0) -> float:
    """The smallest power of two s = 2^e with amax <= top * s (1 for amax = 0),
    found by exact comparisons against top * 2^e."""
    if amax == 0.0:
        return 1.0
    _, E = math.frexp(amax / top)
    e = E
    while amax <= top * math.ldexp(1.0, e - 1):
        e -= 1
    while amax > top * math.ldexp(1.0, e):
        e += 1
    return math.ldexp(1.0, e)


def fp8_quantize_v_blocks_pow2(V, bk: int):
    """Per-key-block e4m3 values of V with power-of-two scales (pow2_scale of
    the block's absmax).  Returns (values float64 on the e4m3 grid [N, d],
    scales float32 [NKB])."""
    V = np.asarray(V, dtype=np.float32)
    N, d = V.shape
    nb = n_blocks(N, bk)
    vals = np.zeros((N, d), dtype=np.float64)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        blk = V[b * bk:min(N, (b + 1) * bk)].astype(np.float64)
        s = pow2_scale(float(np.abs(blk).max()))
        vals[b * bk:min(N, (b + 1) * bk)] = e4m3_round(blk / s)   # exact division
        scales[b] = s
    return vals, scales


def sparse_attention_quant_head(Q, K, V, kept: List[np.ndarray], p: Params,
                                force_skip: Optional[List[np.ndarray]] = None,
                                deltas: Optional[list] = None, qmax: int = 127,
                                v_pow2: bool = False, code_slack: Optional[list] = None):
    """Quantised stage two: the same online softmax, processing order and
    skip rule as the unquantised oracle, with
    S = sm * s_q(i) * s_k(j) * (Qcode . Kcode)  (exact integer dot product) and
    the P.V term  s_v(j) * 2^-8 * sum_c e4m3(2^8 * P) * Vcode.
    ``deltas`` collects the group statistics and the skip rule (lambda or
    recall) is applied as in the unquantised oracle.  ``qmax`` = 127 for
    INT8 Q/K codes, 7 for 4-bit ones; ``v_pow2`` takes V's scales from
    fp8_quantize_v_blocks_pow2 and normalises O (and lse) by the running sum
    of the quantised weights.
    ``code_slack`` (a list, filled per query block) receives, for v_pow2, a
    per-row bound on how far that sum can move, relative to the sum, when
    each weight's code e4m3(2^8 P) is taken from P computed in fp32 instead
    of fp64 (0 for the other modes and for rows with no weight).  With
    u = 2^-24: the exponent argument (S - m) in log2 units, formed from fp32
    values (a scale carrying four roundings: log2(e), sm, s_q, s_k; the
    running max; 8 - max; one fused multiply-add), moves P by at most
    u (5 |S| + 7 |m| + 11) relative, and the exp2 by a few u more;
    eps = 2^-21 (|S| + |m|) + 2^-19 covers both, and each code can then
    move by e4m3_flip_slack of eps.
    Returns (O, lse, skips)."""
    N, d = np.asarray(Q).shape
    sm = p.sm(d)
    qc, qs = int_quantize_blocks(Q, p.BQ, qmax)
    kc, ks = int_quantize_blocks(K, p.BK, qmax)
    vq, vs = (fp8_quantize_v_blocks_pow2 if v_pow2 else fp8_quantize_v_blocks)(V, p.BK)
    qc = qc.astype(np.int64)
    kc = kc.astype(np.int64)
    n_groups = (p.BQ + p.G - 1) // p.G
    O = np.zeros((N, d))
    lse = np.full(N, -np.inf)
    skips = []
    for i, lst in enumerate(kept):
        rows = np.arange(i * p.BQ, min(N, (i + 1) * p.BQ))
        nr = len(rows)
        m = np.full(nr, -np.inf)
        l = np.zeros(nr)
        lq = np.zeros(nr)     # v_pow2: running sum of the quantised weights
        lslack = np.zeros(nr)  # code_slack: bound on the change of lq
        acc = np.zeros((nr, d))
        drop = np.zeros(nr)
        sk = np.zeros((len(lst), n_groups), dtype=bool)
        dl = np.full((len(lst), n_groups), -np.inf)
        for t, j in enumerate(lst):
            cols = np.arange(j * p.BK, min(N, (j + 1) * p.BK))
            idot = qc[rows] @ kc[cols].T               # exact in int64
            S = sm * float(qs[i]) * float(ks[j]) * idot.astype(np.float64)
            if p.causal:
                S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
            mloc = S.max(axis=1)
            mnew = np.maximum(m, mloc)
            alpha = np.ones(nr)
            moved = np.isfinite(mnew) & (m != mnew)
            alpha[moved] = np.exp(m[moved] - mnew[moved])   # exp(-inf) = 0
            safe = np.where(np.isfinite(mnew), mnew, 0.0)
            P = np.where(np.isfinite(S), np.exp(S - safe[:, None]), 0.0)
            E = P.sum(axis=1)
            l = alpha * l + E
            drop = alpha * drop
            acc = alpha[:, None] * acc
            Pq = e4m3_round(P * 256.0) / 256.0
            lq = alpha * lq + Pq.sum(axis=1)
            if code_slack is not None:
                smax = np.where(np.isfinite(S), np.abs(S), 0.0).max(axis=1)
                eps = 2.0 ** -21 * (smax + np.abs(safe)) + 2.0 ** -19
                lslack = alpha * lslack + e4m3_flip_slack(P * 256.0, eps[:, None]).sum(axis=1) / 256.0
            delta_r = np.where(np.isfinite(mloc), mloc - safe, -np.inf)
            for g in range(n_groups):
                gr = slice(g * p.G, min(nr, (g + 1) * p.G))
                skip, dl[t, g] = group_skip(p, gr, nr, delta_r, E, l, drop)
                if force_skip is not None:
                    skip = bool(force_skip[i][t, g])
                sk[t, g] = skip
                if gr.start < nr:
                    if skip:
                        drop[gr] += E[gr]
                    else:
                        acc[gr] += float(vs[j]) * (Pq[gr] @ vq[cols])
            m = mnew
        skips.append(sk)
        if deltas is not None:
            deltas.append(dl)
        if code_slack is not None:
            rel = np.divide(lslack, lq, out=np.zeros(nr), where=lq > 0)
            code_slack.append(rel if v_pow2 else np.zeros(nr))
        ln = lq if v_pow2 else l
        ok = ln > 0
        O[rows[ok]] = acc[ok] / ln[ok, None]
        lse[rows[ok]] = m[ok] + np.log(ln[ok])
    return O, lse, skips


__all__ = ["e4m3_round", "e4m3_flip_slack", "e4m3_encode", "int8_quantize_blocks", "int_quantize_blocks",
           "fp8_quantize_v_blocks", "pow2_scale", "fp8_quantize_v_blocks_pow2",
           "sparse_attention_quant_head", "math"]

"""Why the quantised forward converts its integer scores before the FMA.

The INT8 Q.K^T MFMA returns exact integer dot products d.  The kernels form
the exponent argument of 2^8 P = exp2(csc * d + cb) (csc = sm log2(e) s_q s_k,
cb = 8 - m) as fma(float(d), csc, cb): one conversion, one FMA, one rounding
of the exact value.  A conversion-free form starts the integer accumulator at
the bits of M = 1.5 * 2^23, so that the accumulator read as a float is
y = M + d exactly (|d| < 2^22), and folds M into the constant:
fma(y, csc, cb - csc * M).  That constant is rounded in fp32 at the magnitude
of csc * M, far above the argument's own, so the argument moves by up to about
ulp(csc * M), and the FP8 codes of P (and decisions taken from P) change.  This emulates both forms in numpy on scores of the quantised
workload's size and checks that the kernel's form stays within one fp32
rounding of the exact argument while the folded form does not, and how many
P codes each changes.  CPU only.
"""
import math

import numpy as np

from oracle.quant import e4m3_round

M = 1.5 * 2.0 ** 23
f32 = np.float32


def _fma32(a, b, c):
    # a * b is exact in float64 (two 24-bit significands); the float64 sum's
    # own rounding (2^-53 relative) is far below the effects measured here
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) +
            np.asarray(c, np.float64)).astype(f32)


def _scores(seed, amax_q, amax_k, rows=128, keys=512, d=128):
    rng = np.random.default_rng(seed)
    q = np.clip(np.rint(rng.normal(0, 0.3, (rows, d)) * 127), -127, 127).astype(np.int64)
    k = np.clip(np.rint(rng.normal(0, 0.3, (keys, d)) * 127), -127, 127).astype(np.int64)
    dot = q @ k.T                                   # exact integer scores
    assert np.abs(dot).max() < 2 ** 22
    csc = f32(1.0 / math.sqrt(d) * math.log2(math.e) * (amax_q / 127) * (amax_k / 127))
    xmax = dot.max(axis=1).astype(f32)
    m = (xmax * csc).astype(f32)                    # the running max of this tile
    cb = (f32(8.0) - m).astype(f32)
    return dot, csc, cb


def _arguments(dot, csc, cb):
    ref = dot.astype(np.float64) * float(csc) + cb.astype(np.float64)[:, None]
    kernel = _fma32(dot.astype(f32), csc, cb[:, None])           # convert, then FMA
    y = (dot + int(M)).astype(f32)                               # exact: M + d
    folded_c = (cb - f32(np.float64(csc) * M).astype(f32)).astype(f32)
    folded = _fma32(y, csc, folded_c[:, None])
    return ref, kernel, folded


def test_converted_scores_keep_the_exact_argument():
    dot, csc, cb = _scores(1, 5.0, 5.0)
    ref, kernel, _ = _arguments(dot, csc, cb)
    half_ulp = np.spacing(np.abs(kernel).astype(f32)).astype(np.float64) / 2
    assert np.all(np.abs(kernel - ref) <= half_ulp * (1 + 1e-9))


def test_folded_offset_moves_the_argument_and_the_p_codes():
    for amax, min_flips in ((2.0, 4), (5.0, 30)):
        dot, csc, cb = _scores(2, amax, amax)
        ref, kernel, folded = _arguments(dot, csc, cb)
        err_k = np.abs(kernel - ref).max()
        err_f = np.abs(folded - ref).max()
        # the folded constant's rounding is of the order of ulp(csc * M)
        bound = float(np.spacing(f32(np.float64(csc) * M)))
        assert err_f > 50 * err_k
        assert err_f <= 2 * bound
        live = ref > -20.0                      # weights above 2^-20 (FP8 codes > 0)
        p_ref = e4m3_round(np.exp2(ref[live]))
        flips_k = int((e4m3_round(np.exp2(kernel[live].astype(np.float64))) != p_ref).sum())
        flips_f = int((e4m3_round(np.exp2(folded[live].astype(np.float64))) != p_ref).sum())
        assert flips_k == 0 and flips_f >= min_flips, (amax, flips_k, flips_f)


def test_folded_offset_reaches_past_the_lambda_band_at_large_scales():
    # block absmax 20 (large activations): the folded argument moves by more
    # than the 1e-3 (natural-log units) band within which a skip decision
    # may differ from the oracle's, so a decision taken from it (the recall
    # rule sums the tile's P) can change away from its threshold; the
    # converted form stays within fp32 rounding
    dot, csc, cb = _scores(3, 20.0, 20.0)
    ref, kernel, folded = _arguments(dot, csc, cb)
    band = 1e-3 * math.log2(math.e)
    assert np.abs(folded - ref).max() > band
    assert np.abs(kernel - ref).max() < band / 50

"""CPU pins of the oracle's quantised path (INT8 Q.K^T, e4m3 P.V).

* e4m3 rounding against torch's float8_e4m3fn cast (an independent library
  routine) over every finite bfloat16 bit pattern below the overflow
  boundary, plus hand-worked points of the OCP E4M3 definition
  (tests/golden/e4m3_ocp_points.txt) covering saturation, the smallest
  subnormal and ties to even;
* INT8: inputs that are integer multiples of the block scale quantise
  exactly, so the integer Q.K^T times the scales equals the float64 product;
* the quantised attention against the scalar brute force run with the same
  quantised scores and P.V terms.
"""
import math
import os

import numpy as np
import torch

import brute
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def test_e4m3_golden_points():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    x = np.array([float(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    codes = np.array([int(r[2], 16) for r in rows], dtype=np.uint8)
    np.testing.assert_array_equal(O.e4m3_round(x), want)
    np.testing.assert_array_equal(O.e4m3_encode(x), codes)


def test_e4m3_matches_torch_on_all_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        x = bits.view(np.float32).astype(np.float64)
    finite = np.isfinite(x) & (np.abs(x) < 464.0)
    ref = torch.from_numpy(x[finite].astype(np.float32)).to(torch.float8_e4m3fn)
    ref_vals = ref.to(torch.float64).numpy()
    got = O.e4m3_round(x[finite])
    np.testing.assert_array_equal(got, ref_vals)
    # bit patterns too (torch keeps the sign of zero, as does the encoder)
    np.testing.assert_array_equal(O.e4m3_encode(x[finite]), ref.view(torch.uint8).numpy())
    # saturation above the largest finite value
    big = x[np.isfinite(x) & (np.abs(x) >= 464.0)]
    np.testing.assert_array_equal(np.abs(O.e4m3_round(big)), 448.0)


def test_int8_exact_on_scale_multiples():
    rng = np.random.default_rng(0)
    N, d, bs = 96, 16, 32
    scales = np.float32(2.0) ** rng.integers(-6, 3, size=3).astype(np.float32)
    codes = rng.integers(-127, 128, size=(N, d)).astype(np.float32)
    for b in range(3):
        codes[b * bs, 0] = 127.0       # make the block absmax exactly 127 * s
    X = codes * np.repeat(scales, bs)[:, None]
    c, s = O.int8_quantize_blocks(X, bs)
    np.testing.assert_array_equal(s, scales)
    np.testing.assert_array_equal(c.astype(np.float32), codes)
    Y = X[::-1].copy()
    cy, sy = O.int8_quantize_blocks(Y, bs)
    prod = (c.astype(np.int64) @ cy.astype(np.int64).T).astype(np.float64)
    deq = prod * np.repeat(s, bs)[:, None].astype(np.float64) \
        * np.repeat(sy, bs)[None, :].astype(np.float64)
    np.testing.assert_array_equal(deq, X.astype(np.float64) @ Y.astype(np.float64).T)


def test_int8_rounding_and_zero_block():
    X = np.zeros((4, 2), dtype=np.float32)
    c, s = O.int8_quantize_blocks(X, 4)
    assert s[0] == 1.0 and not c.any()
    # absmax 127 -> scale 1; halves round to even
    X = np.array([[127.0, 0.5], [1.5, -2.5], [-127.0, 2.5], [0.0, -0.5]], np.float32)
    c, s = O.int8_quantize_blocks(X, 4)
    assert s[0] == 1.0
    np.testing.assert_array_equal(c, [[127, 0], [2, -2], [-127, 2], [0, 0]])


def test_fp8_v_scale_maps_absmax_to_448():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((130, 8)).astype(np.float32)
    vals, s = O.fp8_quantize_v_blocks(V, 64)
    assert vals.shape == V.shape and s.shape == (3,)
    for b in range(3):
        blk = vals[b * 64:(b + 1) * 64]
        assert np.abs(blk).max() == 448.0
        assert np.all(O.e4m3_round(blk) == blk)


def test_quant_attention_matches_brute():
    rng = np.random.default_rng(2)
    N, d, BQ, BK, G = 36, 4, 8, 4, 4
    q = rng.standard_normal((N, d)).astype(np.float32) * 2
    k = rng.standard_normal((N, d)).astype(np.float32) * 2
    v = rng.standard_normal((N, d)).astype(np.float32)
    for causal in (False, True):
        for lam in (-math.inf, -1.0):
            p = O.Params(BQ=BQ, BK=BK, causal=causal, tau=0.8, lam=lam, G=G,
                         rule="energy")
            pr = O.predict_head(q, k, p)
            got, _, sk = O.sparse_attention_quant_head(q, k, v, pr["kept"], p)
            qc, qs = O.int8_quantize_blocks(q, BQ)
            kc, ks = O.int8_quantize_blocks(k, BK)
            vq, vs = O.fp8_quantize_v_blocks(v, BK)
            sm = 1 / math.sqrt(d)

            def score(r, c):
                dot = sum(int(qc[r, e]) * int(kc[c, e]) for e in range(d))
                return sm * float(qs[r // BQ]) * float(ks[c // BK]) * dot

            def pv(r, c, pval):
                pq = float(O.e4m3_round(np.array([pval * 256.0]))[0]) / 256.0
                return [float(vs[c // BK]) * pq * vq[c, e] for e in range(d)]

            exp, esk = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                                       [list(x) for x in pr["kept"]], BQ, BK, causal,
                                       lam, G, score=score, pv=pv)
            np.testing.assert_allclose(got, np.array(exp), atol=1e-12)
            assert [s.tolist() for s in sk] == esk


def test_int4_codes_exact_on_scale_multiples_and_rounding():
    """qmax = 7: codes in [-7, 7]; blocks built as code * scale with a
    power-of-two scale round-trip exactly; halves round to even."""
    rng = np.random.default_rng(3)
    N, d, bs = 64, 8, 16
    scales = np.float32(2.0) ** rng.integers(-4, 3, size=4).astype(np.float32)
    codes = rng.integers(-7, 8, size=(N, d)).astype(np.float32)
    for b in range(4):
        codes[b * bs, 0] = -7.0            # block absmax exactly 7 * s
    X = codes * np.repeat(scales, bs)[:, None]
    c, s = O.int_quantize_blocks(X, bs, 7)
    np.testing.assert_array_equal(s, scales)
    np.testing.assert_array_equal(c.astype(np.float32), codes)
    assert np.abs(c).max() == 7
    X = np.array([[7.0, 0.5], [1.5, -2.5], [-7.0, 3.5], [0.0, -0.5]], np.float32)
    c, s = O.int_quantize_blocks(X, 4, 7)
    assert s[0] == 1.0
    np.testing.assert_array_equal(c, [[7, 0], [2, -2], [-7, 4], [0, 0]])
    # the INT8 helper is the qmax = 127 case
    c8, s8 = O.int8_quantize_blocks(X, 4)
    c127, s127 = O.int_quantize_blocks(X, 4, 127)
    np.testing.assert_array_equal(c8, c127)
    np.testing.assert_array_equal(s8, s127)


def test_int4_quant_attention_matches_brute():
    rng = np.random.default_rng(4)
    N, d, BQ, BK, G = 36, 4, 8, 4, 4
    q = rng.standard_normal((N, d)).astype(np.float32) * 2
    k = rng.standard_normal((N, d)).astype(np.float32) * 2
    v = rng.standard_normal((N, d)).astype(np.float32)
    p = O.Params(BQ=BQ, BK=BK, tau=0.8, lam=-1.0, G=G)
    pr = O.predict_head(q, k, p)
    got, _, sk = O.sparse_attention_quant_head(q, k, v, pr["kept"], p, qmax=7)
    qc, qs = O.int_quantize_blocks(q, BQ, 7)
    kc, ks = O.int_quantize_blocks(k, BK, 7)
    vq, vs = O.fp8_quantize_v_blocks(v, BK)
    assert np.abs(qc).max() <= 7 and np.abs(kc).max() <= 7
    sm = 1 / math.sqrt(d)

    def score(r, c):
        dot = sum(int(qc[r, e]) * int(kc[c, e]) for e in range(d))
        return sm * float(qs[r // BQ]) * float(ks[c // BK]) * dot

    def pv(r, c, pval):
        pq = float(O.e4m3_round(np.array([pval * 256.0]))[0]) / 256.0
        return [float(vs[c // BK]) * pq * vq[c, e] for e in range(d)]

    exp, esk = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                               [list(x) for x in pr["kept"]], BQ, BK, False,
                               -1.0, G, score=score, pv=pv)
    np.testing.assert_allclose(got, np.array(exp), atol=1e-12)
    assert [s.tolist() for s in sk] == esk
    # coarser codes: farther from the unquantised result than INT8 codes
    o8, _, _ = O.sparse_attention_quant_head(q, k, v, pr["kept"], p)
    ref, _, _ = O.sparse_attention_head(q, k, v, pr["kept"], p)
    assert np.abs(got - ref).mean() > np.abs(o8 - ref).mean()


def _pow2_brute(amax):
    """Smallest 2^e (integer e) with amax <= 448 * 2^e, by enumeration."""
    if amax == 0:
        return 1.0
    for e in range(-200, 200):
        if amax <= 448.0 * 2.0 ** e:
            return 2.0 ** e
    raise AssertionError(amax)


def test_pow2_scale_hand_values_and_enumeration():
    assert O.pow2_scale(448.0) == 1.0
    assert O.pow2_scale(np.nextafter(np.float32(448.0), np.float32(1e9))) == 2.0
    assert O.pow2_scale(224.0) == 0.5
    assert O.pow2_scale(np.nextafter(np.float32(224.0), np.float32(1e9))) == 1.0
    assert O.pow2_scale(3.5) == 2.0 ** -7       # 448 * 2^-7 = 3.5 exactly
    assert O.pow2_scale(3.6) == 2.0 ** -6
    assert O.pow2_scale(0.0) == 1.0
    rng = np.random.default_rng(21)
    for a in np.concatenate([rng.lognormal(0, 6, 400), 448.0 * 2.0 ** rng.integers(-60, 60, 50)]):
        a = float(np.float32(a))
        assert O.pow2_scale(a) == _pow2_brute(a), a


def test_pow2_v_blocks_range_grid_and_round_trip():
    rng = np.random.default_rng(22)
    V = (rng.standard_normal((200, 16)) * rng.lognormal(0, 2, (200, 1))).astype(np.float32)
    vals, s = O.fp8_quantize_v_blocks_pow2(V, 64)
    for b in range(4):
        blk = V[b * 64:(b + 1) * 64]
        e = math.log2(float(s[b]))
        assert e == int(e)                                     # a power of two
        r = float(np.abs(blk).max()) / float(s[b])
        assert 224.0 < r <= 448.0
        q = vals[b * 64:(b + 1) * 64]
        assert np.all(O.e4m3_round(q) == q) and np.abs(q).max() <= 448.0
        np.testing.assert_array_equal(q, O.e4m3_round(blk.astype(np.float64) / float(s[b])))
    # values on the e4m3 grid times a power of two come back exactly
    grid = O.e4m3_round(rng.uniform(-448, 448, (64, 8)))
    grid[0, 0] = 448.0
    X = (grid * 2.0 ** -5).astype(np.float32)
    vals, s = O.fp8_quantize_v_blocks_pow2(X, 64)
    assert s[0] == 2.0 ** -5
    np.testing.assert_array_equal(vals, grid)


def test_pow2_quant_attention_matches_brute():
    rng = np.random.default_rng(23)
    N, d, BQ, BK, G = 36, 4, 8, 4, 4
    q = rng.standard_normal((N, d)).astype(np.float32) * 2
    k = rng.standard_normal((N, d)).astype(np.float32) * 2
    v = rng.standard_normal((N, d)).astype(np.float32)
    for causal in (False, True):
        p = O.Params(BQ=BQ, BK=BK, causal=causal, tau=0.8, lam=-1.0, G=G)
        pr = O.predict_head(q, k, p)
        got, _, sk = O.sparse_attention_quant_head(q, k, v, pr["kept"], p, v_pow2=True)
        qc, qs = O.int8_quantize_blocks(q, BQ)
        kc, ks = O.int8_quantize_blocks(k, BK)
        sv = [_pow2_brute(float(np.abs(v[j * BK:(j + 1) * BK]).max())) for j in range(N // BK)]
        sm = 1 / math.sqrt(d)

        def score(r, c):
            dot = sum(int(qc[r, e]) * int(kc[c, e]) for e in range(d))
            return sm * float(qs[r // BQ]) * float(ks[c // BK]) * dot

        def pv(r, c, pval):
            pq = float(O.e4m3_round(np.array([pval * 256.0]))[0]) / 256.0
            s = sv[c // BK]
            return [s * pq * float(O.e4m3_round(np.array([float(v[c, e]) / s]))[0])
                    for e in range(d)]

        def weight(pval):  # the quantised weight normalises O
            return float(O.e4m3_round(np.array([pval * 256.0]))[0]) / 256.0

        exp, esk = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                                   [list(x) for x in pr["kept"]], BQ, BK, causal, -1.0, G,
                                   score=score, pv=pv, weight=weight)
        np.testing.assert_allclose(got, np.array(exp), atol=1e-12)
        assert [s.tolist() for s in sk] == esk
        # the V codes differ from the absmax / 448 reading; both stay within
        # e4m3's resolution (1/16 relative) of the unquantised result
        o8, _, _ = O.sparse_attention_quant_head(q, k, v, pr["kept"], p)
        ref, _, _ = O.sparse_attention_head(q, k, v, pr["kept"], p)
        assert not np.array_equal(got, o8)
        for o in (got, o8):
            assert np.abs(o - ref).max() <= np.abs(v).max() / 8


def test_pow2_output_is_a_weighted_average_of_quantised_values():
    """With lambda = -inf nothing is skipped, and in the power-of-two mode O
    is a convex combination of the quantised V rows s_v V~: each output lies
    within their range; the absmax / 448 mode normalises by the unquantised
    sum instead, which the quantised weights need not match."""
    rng = np.random.default_rng(24)
    N, d = 256, 8
    q, k = (rng.standard_normal((N, d)).astype(np.float32) * 2 for _ in range(2))
    v = rng.standard_normal((N, d)).astype(np.float32)
    p = O.Params(BQ=32, BK=16, tau=1.0, lam=-math.inf, G=8)
    kept = O.predict_head(q, k, p)["kept"]
    got, _, _ = O.sparse_attention_quant_head(q, k, v, kept, p, v_pow2=True)
    vq, vs = O.fp8_quantize_v_blocks_pow2(v, 16)
    deq = vq * np.repeat(vs.astype(np.float64), 16)[:, None]
    assert np.all(got <= deq.max(axis=0) + 1e-12) and np.all(got >= deq.min(axis=0) - 1e-12)
    # all-equal V rows: the weighted average returns them exactly
    vc = np.tile(np.float32([0.5, -1.25, 3.0, 0.0, 2.0, -4.0, 1.0, 0.125]), (N, 1))
    got, _, _ = O.sparse_attention_quant_head(q, k, vc, kept, p, v_pow2=True)
    np.testing.assert_allclose(got, np.tile(vc[0], (N, 1)), rtol=0, atol=1e-12)


def test_flip_slack_bounds_every_perturbed_rounding():
    # e4m3_round is monotone, so every value within a relative eps of x
    # rounds within e4m3_flip_slack(x, eps) of e4m3_round(x); the slack is 0
    # on the e4m3 grid (far from a rounding boundary) and one step at a
    # midpoint
    rng = np.random.default_rng(41)
    x = rng.uniform(0.0, 300.0, 20000)
    eps = 10.0 ** rng.uniform(-7, -2, x.size)
    slack = O.e4m3_flip_slack(x, eps)
    base = O.e4m3_round(x)
    for _ in range(8):
        r = rng.uniform(-1.0, 1.0, x.size) * eps
        assert np.all(np.abs(O.e4m3_round(x * (1.0 + r)) - base) <= slack)
    grid = O.e4m3_round(rng.uniform(1.0, 256.0, 1000))
    assert np.all(O.e4m3_flip_slack(grid, 1e-4) == 0.0)
    np.testing.assert_array_equal(O.e4m3_flip_slack(np.array([1.0625, 17.0, 136.0]), 1e-6),
                                  [0.125, 2.0, 16.0])


def test_code_slack_bounds_codes_computed_in_fp32():
    # One kept tile per query block (128 of them).  The quantised
    # weights' sum of the power-of-two mode, recomputed with the exponent
    # argument and exp2 in fp32 (scale = fl(fl(fl(sm log2e) sq) sk), max,
    # 8 - max, one fused multiply-add), changes some rows' codes; every
    # row's lse stays within the bound code_slack gives.
    rng = np.random.default_rng(43)
    N, d = 16384, 128
    q = (rng.standard_normal((N, d)) * 2).astype(np.float32)
    k = (rng.standard_normal((N, d)) * 2).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    sm = float(np.float32(1 / math.sqrt(d)))
    p = O.Params(BQ=128, BK=64, causal=False, tau=0.9, lam=-math.inf, G=32, sm_scale=sm)
    nqb = N // 128
    kept = [np.array([(3 * i + 1) % (N // 64)]) for i in range(nqb)]
    slack = []
    _, lse, _ = O.sparse_attention_quant_head(q, k, v, kept, p, v_pow2=True, code_slack=slack)
    qc, qs = O.int8_quantize_blocks(q, 128)
    kc, ks = O.int8_quantize_blocks(k, 64)
    f32 = np.float32
    c2 = f32(f32(sm) * f32(1.4426950408889634))
    flips = 0
    for i in range(nqb):
        j = int(kept[i][0])
        rows, cols = slice(i * 128, (i + 1) * 128), slice(j * 64, (j + 1) * 64)
        dot = qc[rows].astype(np.int64) @ kc[cols].astype(np.int64).T
        csc = f32(f32(c2 * f32(qs[i])) * f32(ks[j]))
        x = dot.astype(f32)
        m2 = (x.max(axis=1) * csc).astype(f32)                    # log2 units
        cb = (f32(8.0) - m2).astype(f32)
        arg = (x.astype(np.float64) * float(csc) + cb.astype(np.float64)[:, None]).astype(f32)
        codes = O.e4m3_round(np.exp2(arg).astype(np.float64))     # 2^8 P
        lse32 = (m2.astype(np.float64) + np.log2(codes.sum(axis=1) / 256.0)) * math.log(2.0)
        S = sm * float(qs[i]) * float(ks[j]) * dot.astype(np.float64)
        rel = slack[i]
        assert np.all(rel < 1.0)
        tol = 1e-5 + np.maximum(np.log1p(rel), -np.log1p(-rel))
        assert np.all(np.abs(lse32 - lse[rows]) <= tol), i
        # codes taken from the fp64 scores, to show that fp32 moves some
        flips += int(np.sum(codes != O.e4m3_round(256.0 * np.exp(S - S.max(axis=1)[:, None]))))
    assert flips > 0


def test_flip_slack_at_the_ends_of_the_e4m3_range():
    # subnormals (a fixed quantum of 2^-9): the midpoint 3 * 2^-10 between
    # 2^-9 and 2^-8 can round either way, 2^-9 itself cannot; zero stays
    # zero; at the top, values round to 448 and saturate there, so the
    # midpoint 432 between 416 and 448 has one step of slack and 448 none
    x = np.array([0.0, 3 * 2.0 ** -10, 2.0 ** -9, 432.0, 448.0, 500.0])
    np.testing.assert_array_equal(O.e4m3_flip_slack(x, 1e-6),
                                  [0.0, 2.0 ** -9, 0.0, 32.0, 0.0, 0.0])

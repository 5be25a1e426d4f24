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

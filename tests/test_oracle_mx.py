"""Pins for the oracle's MXFP8 quantisation and GEMM (CPU only)."""

import math

import numpy as np
import pytest

from oracle import codec, mx


@pytest.mark.parametrize("fmt,mx_,cases", [
    ("e4m3", 448.0, [(448.0, 0), (448.5, 1), (896.0, 1), (896.5, 2), (224.0, -1), (224.5, 0), (1.0, -8),
                     (1.75, -8), (1.76, -7), (2.0 ** -20, -28)]),
    ("e5m2", 57344.0, [(57344.0, 0), (57345.0, 1), (1.0, -15), (1.75, -15), (1.8, -14), (65536.0, 1)]),
])
def test_scale_exponent_hand_values(fmt, mx_, cases):
    # the smallest e with amax <= MAX * 2^e: 448 = 1.75 * 2^8, so amax in (1.75 * 2^(k-1), 1.75 * 2^k] -> e = k - 8
    for amax, e in cases:
        assert mx.scale_exponent(np.float32(amax), fmt) == e, (amax, e)


def test_scale_exponent_special_and_clamped():
    assert mx.scale_exponent(0.0, "e4m3") == 0
    assert mx.scale_exponent(np.inf, "e4m3") == 0 and mx.scale_exponent(np.nan, "e5m2") == 0
    # smallest fp32 subnormal 2^-149: e = ceil(-149 - log2(448)) = -157, clamped to -127
    assert mx.scale_exponent(np.float32(2.0 ** -149), "e4m3") == -127
    # largest fp32: 2^128 (1 - 2^-24) <= 448 * 2^e  ->  e = 120
    assert mx.scale_exponent(np.finfo(np.float32).max, "e4m3") == 120


def test_quantize_properties_and_hand_block():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 128)) * 10.0 ** rng.uniform(-20, 20, size=(5, 1))).astype(np.float32)
    x[2, 32:64] = 0.0
    for fmt in ("e4m3", "e5m2"):
        f = codec.FORMATS[fmt]
        q, s = mx.quantize_mx(x, fmt)
        assert q.shape == x.shape and s.shape == (5, 4) and s[2, 1] == 127
        for r in range(5):
            for b in range(4):
                blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
                amax = np.max(np.abs(blk))
                if amax == 0:
                    continue
                e = int(s[r, b]) - 127
                # nothing saturates, and the block max lands in (MAX / 2, MAX]
                assert amax <= f.max_value * 2.0 ** e and amax > f.max_value * 2.0 ** (e - 1)
        d = mx.dequant_mx(q, s, fmt)
        # values in the element format's normal range at their block's scale round with relative error <= 2^-(m+1)
        e_el = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
        normal = np.abs(x.astype(np.float64)) >= np.ldexp(2.0 ** (1 - f.bias), e_el)
        rel = 2.0 ** -(f.mbits + 1)
        assert normal.sum() > 300
        assert np.all(np.abs(d - x)[normal] <= rel * np.abs(x[normal]))
    # a block of exactly representable values comes back exactly: 2^-10 * {1, 1.125, ..., 1.75} x signs
    v = np.float32([1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, -1.75] * 4) * np.float32(2.0 ** -10)
    q, s = mx.quantize_mx(v.reshape(1, 32), "e4m3")
    assert s[0, 0] == 127 + (-10 - 8) and np.array_equal(mx.dequant_mx(q, s, "e4m3")[0], v.astype(np.float64))


def test_mx_gemm_against_block_loop():
    rng = np.random.default_rng(4)
    qa = rng.integers(0, 0x7F, size=(3, 64)).astype(np.uint8)
    qb = (rng.integers(0, 0x7C, size=(2, 64)) | 0x80 * rng.integers(0, 2, size=(2, 64))).astype(np.uint8)
    sa = rng.integers(100, 150, size=(3, 2)).astype(np.uint8)
    sb = rng.integers(100, 150, size=(2, 2)).astype(np.uint8)
    c = mx.mx_gemm(qa, sa, "e4m3", qb, sb, "e5m2")
    da, db = codec.decode(qa, "e4m3"), codec.decode(qb, "e5m2")
    for m in range(3):
        for n in range(2):
            want = 0.0
            for k in range(64):
                want += da[m, k] * math.ldexp(1.0, int(sa[m, k // 32]) - 127) * db[n, k] * \
                    math.ldexp(1.0, int(sb[n, k // 32]) - 127)
            assert c[m, n] == pytest.approx(want, rel=1e-12, abs=0)

"""Pins for the oracle's FP8 codec (CPU only).

The three encoders were written independently (integer rounding on fp32 bits;
fp64 frexp/rint; brute-force nearest code).  Agreement between them over every
rounding class, plus the format facts the pages state, pins the codec.
"""

import numpy as np
import pytest

from oracle import codec
from synth import adversarial_f32

FMTS = [codec.E4M3, codec.E5M2]


def test_format_facts_match_pages(golden):
    g = golden("format_facts.txt")
    assert (codec.E4M3.ebits, codec.E4M3.mbits) == (g["e4m3_exponent_bits"], g["e4m3_mantissa_bits"])
    assert (codec.E5M2.ebits, codec.E5M2.mbits) == (g["e5m2_exponent_bits"], g["e5m2_mantissa_bits"])
    assert codec.decode(codec.E4M3.max_code, "e4m3") == g["e4m3_max"]
    # more precision vs more range, as the formats page says
    assert codec.E4M3.max_value < codec.E5M2.max_value
    t4, t5 = codec.finite_table("e4m3"), codec.finite_table("e5m2")
    rel4 = np.min(np.diff(t4[8:]) / t4[9:])   # relative step in the normal range
    rel5 = np.min(np.diff(t5[4:]) / t5[5:])
    assert rel4 < rel5


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x58, 16.0), (0x5A, 20.0), (0x7E, 448.0), (0x80, -0.0),
    (0xF9, -288.0), (0xFE, -448.0)])
def test_e4m3_decode_fields(code, value):
    v = codec.decode(code, "e4m3")
    assert v == value and np.signbit(v) == np.signbit(value)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -16), (0x03, 3 * 2.0 ** -16), (0x04, 2.0 ** -14), (0x3C, 1.0),
    (0x3D, 1.25), (0x4D, 20.0), (0x7B, 57344.0), (0x7C, np.inf), (0xFC, -np.inf), (0xBC, -1.0)])
def test_e5m2_decode_fields(code, value):
    assert codec.decode(code, "e5m2") == value


def test_nan_codes():
    c = np.arange(256)
    n4 = np.flatnonzero(np.isnan(codec.decode(c, "e4m3")))
    n5 = np.flatnonzero(np.isnan(codec.decode(c, "e5m2")))
    assert n4.tolist() == [0x7F, 0xFF]
    assert n5.tolist() == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_finite_table_strictly_increasing(f):
    t = codec.finite_table(f)
    assert t[0] == 0 and np.all(np.diff(t) > 0)
    assert t[-1] == f.max_value
    # the step doubles exactly at each binade boundary above the subnormals
    steps = np.diff(t)
    assert np.all(steps[: 1 << f.mbits] == steps[0])


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_round_trip_all_256_codes(f):
    c = np.arange(256, dtype=np.uint8)
    v = codec.decode(c, f)
    enc = codec.encode(v.astype(np.float32), f)
    finite = np.isfinite(v)
    assert np.array_equal(enc[finite], c[finite])
    # NaN codes come back as sign|0x7F; E5M2 infinities saturate to +-max
    nan = np.isnan(v)
    assert np.all(enc[nan] == ((c[nan] & 0x80) | 0x7F))
    inf = np.isinf(v)
    assert np.all(enc[inf] == ((c[inf] & 0x80) | f.max_code))


@pytest.mark.parametrize("x,code", [
    (448.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (1e9, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE),
    (17.0, 0x58), (19.0, 0x5A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (-1e-30, 0x80), (-0.0, 0x80),
    (432.0, 0x7E), (416.0, 0x7D), (2.0 ** -9, 0x01), (1.0625, 0x38), (1.1875, 0x3A), (-298.66669, 0xF9)])
def test_e4m3_specials(x, code):
    for enc in (codec.encode, codec.encode_rint, codec.encode_nearest):
        assert int(enc(np.float32(x), "e4m3").reshape(-1)[0]) == code, enc.__name__


@pytest.mark.parametrize("x,code", [
    (57344.0, 0x7B), (61440.0, 0x7B), (1e30, 0x7B), (np.inf, 0x7B), (-np.inf, 0xFB), (19.0, 0x4D),
    (1.0, 0x3C), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02), (-0.0, 0x80)])
def test_e5m2_specials(x, code):
    for enc in (codec.encode, codec.encode_rint, codec.encode_nearest):
        assert int(enc(np.float32(x), "e5m2").reshape(-1)[0]) == code, enc.__name__


def test_nan_encodes_to_sign_7f():
    bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32)
    for f in FMTS:
        for enc in (codec.encode, codec.encode_rint, codec.encode_nearest):
            out = enc(bits.view(np.float32), f)
            assert out.tolist() == [0x7F, 0xFF, 0x7F, 0xFF]


def _structured_patterns() -> np.ndarray:
    """Every (sign, exponent, top-11 mantissa bits) combination with the low 12
    mantissa bits in each rounding class (zero, tiny, just below/at/just above
    half, all ones).  For every format and exponent the dropped bits split at or
    above bit 12, so this reaches each of {exact, below half, tie, above half}
    for every kept value, odd and even."""
    top = np.arange(1 << 11, dtype=np.uint32) << np.uint32(12)
    low = np.array([0x000, 0x001, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    mant = (top[:, None] | low[None, :]).reshape(-1)
    exps = np.arange(256, dtype=np.uint32) << np.uint32(23)
    pos = (exps[:, None] | mant[None, :]).reshape(-1)
    return np.concatenate([pos, pos | np.uint32(0x80000000)])


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_encoders_agree_structured(f):
    x = _structured_patterns().view(np.float32)
    a = codec.encode(x, f)
    b = codec.encode_rint(x, f)
    bad = np.flatnonzero(a != b)
    assert bad.size == 0, [hex(int(v)) for v in x.view(np.uint32)[bad[:8]]]


@pytest.mark.parametrize("f,exps", [
    (codec.E4M3, [127 - 10, 127 - 7, 127 + 8]),
    (codec.E5M2, [127 - 17, 127 - 15, 127 + 15])], ids=["e4m3", "e5m2"])
def test_encoders_agree_on_whole_binades(f, exps):
    """Every fp32 pattern of the subnormal-boundary, unit and top binades."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    for E in exps:
        x = ((np.uint32(E) << np.uint32(23)) | mant).view(np.float32)
        assert np.array_equal(codec.encode(x, f), codec.encode_rint(x, f)), E


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_encoders_agree_random_bits(f):
    rng = np.random.default_rng(1234)
    x = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    assert np.array_equal(codec.encode(x, f), codec.encode_rint(x, f))


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_brute_force_nearest_on_samples(f):
    x = adversarial_f32(seed=5, random_count=3000)
    rng = np.random.default_rng(99)
    near = (rng.standard_normal(3000) * f.max_value / 4).astype(np.float32)
    x = np.concatenate([x, near])
    assert np.array_equal(codec.encode(x, f), codec.encode_nearest(x, f))


@pytest.mark.parametrize("f", FMTS, ids=lambda f: f.name)
def test_midpoints_round_to_even_code(f):
    t = codec.finite_table(f)
    mid = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (t[:-1] + t[1:]) / 2)   # midpoints are exact in fp32
    lo_code = np.arange(t.size - 1)
    want = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    assert np.array_equal(codec.encode(mid, f), want.astype(np.uint8))
    above = np.nextafter(mid, np.float32(np.inf))
    below = np.nextafter(mid, np.float32(0))
    assert np.array_equal(codec.encode(above, f), (lo_code + 1).astype(np.uint8))
    assert np.array_equal(codec.encode(below, f), lo_code.astype(np.uint8))

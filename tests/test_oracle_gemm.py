"""Pins for the oracle's dequantised GEMM, error bound and grouped GEMM (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, gemm, scaling
from synth import bf16_bits_from_f32, moe_token_counts


def _rand_codes(rng, shape, fmt):
    """Random finite codes of the format (NaN / Inf codes excluded)."""
    f = codec.FORMATS[fmt]
    mag = rng.integers(0, f.max_code + 1, size=shape)
    sign = rng.integers(0, 2, size=shape) << 7
    return (mag | sign).astype(np.uint8)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
def test_exact_dot_against_fractions(fa, fb):
    rng = np.random.default_rng(1)
    a = _rand_codes(rng, 300, fa)
    b = _rand_codes(rng, 300, fb)
    num, sh = gemm.exact_dot(a, fa, b, fb)
    want = sum((Fraction(float(x)) * Fraction(float(y))
                for x, y in zip(codec.decode(a, fa), codec.decode(b, fb))), Fraction(0))
    assert Fraction(num, 2 ** sh) == want


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
def test_dequant_gemm_matches_exact_loops(fa, fb):
    rng = np.random.default_rng(2)
    qa = _rand_codes(rng, (6, 40), fa)
    qb = _rand_codes(rng, (40, 5), fb)
    sa, sb = np.float32(0.25), np.float32(3.0)
    c = gemm.dequant_gemm(qa, fa, qb, fb, sa, sb)
    ex = gemm.exact_gemm_small(qa, fa, qb, fb) * 0.75
    assert np.array_equal(c, ex)


def test_one_hot_and_permutation_select_columns():
    rng = np.random.default_rng(3)
    qa = _rand_codes(rng, (16, 32), "e4m3")
    perm = rng.permutation(32)
    qb = np.zeros((32, 32), dtype=np.uint8)
    qb[perm, np.arange(32)] = 0x38                 # 1.0 in E4M3
    c = gemm.dequant_gemm(qa, "e4m3", qb, "e4m3", np.float32(0.5), np.float32(1.0))
    assert np.array_equal(c, codec.decode(qa, "e4m3")[:, perm] * 0.5)


@pytest.mark.parametrize("K", [128, 4096, 16384])
def test_all_max_operands_closed_form(K):
    qa = np.full((2, K), 0x7E, dtype=np.uint8)
    qb = np.full((K, 3), 0x7E, dtype=np.uint8)
    c = gemm.dequant_gemm(qa, "e4m3", qb, "e4m3", np.float32(1), np.float32(1))
    assert np.all(c == K * 448.0 ** 2)
    qg = np.full((2, K), 0x7B, dtype=np.uint8)
    c2 = gemm.dequant_gemm(qg, "e5m2", qb, "e4m3", np.float32(1), np.float32(1))
    assert np.all(c2 == K * 448.0 * 57344.0)


def test_zero_operand_gives_zero_and_zero_bound():
    qa = np.zeros((4, 64), dtype=np.uint8)
    qb = _rand_codes(np.random.default_rng(4), (64, 4), "e4m3")
    assert not gemm.dequant_gemm(qa, "e4m3", qb, "e4m3", 1.0, 1.0).any()
    assert not gemm.abs_bound(qa, "e4m3", qb, "e4m3", 1.0, 1.0).any()


def test_abs_bound_is_relative_sum_of_magnitudes():
    rng = np.random.default_rng(5)
    qa = _rand_codes(rng, (3, 50), "e4m3")
    qb = _rand_codes(rng, (50, 2), "e4m3")
    b = gemm.abs_bound(qa, "e4m3", qb, "e4m3", np.float32(2), np.float32(0.5))
    A, B = np.abs(codec.decode(qa, "e4m3")), np.abs(codec.decode(qb, "e4m3"))
    for m in range(3):
        for n in range(2):
            assert np.isclose(b[m, n], 1e-5 * sum(A[m, k] * B[k, n] for k in range(50)), rtol=1e-12)


def test_bf16_round_matches_synth_rounding_and_bracket():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(10000) * 100).astype(np.float32)
    want = (bf16_bits_from_f32(x).astype(np.uint32) << np.uint32(16)).view(np.float32)
    assert np.array_equal(gemm.bf16_round(x.astype(np.float64)), want)
    lo, hi = gemm.bf16_bracket(x.astype(np.float64), np.zeros_like(x, dtype=np.float64))
    assert np.array_equal(lo, want) and np.array_equal(hi, want)
    lo, hi = gemm.bf16_bracket(np.float64([1.0]), np.float64([2.0 ** -9]))
    assert lo[0] == 1.0 == hi[0]                   # 1 - 2^-9 is a tie that rounds to even (1.0)
    lo, hi = gemm.bf16_bracket(np.float64([1.0]), np.float64([2.0 ** -7]))
    assert lo[0] == 1.0 - 2.0 ** -7 and hi[0] == 1.0 + 2.0 ** -7


def test_grouped_reduces_to_per_group_gemm_with_uniform_scales():
    rng = np.random.default_rng(7)
    offs = np.array([0, 5, 5, 17])                 # includes an empty expert
    K, N = 300, 260
    qa = _rand_codes(rng, (17, K), "e4m3")
    qb = _rand_codes(rng, (3, N, K), "e4m3")
    sa = np.full((17, 3), np.float32(0.5), dtype=np.float32)
    sb = np.full((3, 3, 3), np.float32(0.25), dtype=np.float32)
    c = gemm.grouped_gemm(qa, sa, qb, sb, offs)
    for g in range(3):
        r0, r1 = offs[g], offs[g + 1]
        want = gemm.dequant_gemm(qa[r0:r1], "e4m3", qb[g].T, "e4m3", 0.5, 0.25)
        assert np.allclose(c[r0:r1], want, rtol=1e-13, atol=0)


def test_grouped_matches_explicit_block_loops():
    rng = np.random.default_rng(8)
    offs = np.array([0, 3, 7])
    K, N = 140, 129
    qa = _rand_codes(rng, (7, K), "e4m3")
    qb = _rand_codes(rng, (2, N, K), "e4m3")
    sa = (2.0 ** rng.integers(-8, 8, size=(7, 2))).astype(np.float32)
    sb = (2.0 ** rng.integers(-8, 8, size=(2, 2, 2))).astype(np.float32)
    c = gemm.grouped_gemm(qa, sa, qb, sb, offs)
    A = codec.decode(qa, "e4m3")
    for m in range(7):
        g = 0 if m < 3 else 1
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                tot += Fraction(float(A[m, k])) * Fraction(float(codec.decode(qb[g, n, k], "e4m3"))) \
                    * Fraction(float(sa[m, k // 128])) * Fraction(float(sb[g, n // 128, k // 128]))
            assert c[m, n] == float(tot) or abs(c[m, n] - float(tot)) <= 1e-12 * abs(float(tot))


def test_grouped_row_subset_matches_full():
    rng = np.random.default_rng(9)
    offs = np.array([0, 4, 9])
    qa = _rand_codes(rng, (9, 256), "e4m3")
    qb = _rand_codes(rng, (2, 128, 256), "e4m3")
    sa = rng.uniform(0.1, 2, size=(9, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 2, size=(2, 1, 2)).astype(np.float32)
    full = gemm.grouped_gemm(qa, sa, qb, sb, offs)
    rows = np.array([8, 0, 4])
    assert np.array_equal(gemm.grouped_gemm(qa, sa, qb, sb, offs, rows=rows), full[rows])


def test_blockwise_quantize_then_grouped_approximates_float_product():
    """End-to-end sanity: per-block FP8 GEMM is close to the fp64 product of the inputs."""
    rng = np.random.default_rng(10)
    A = rng.standard_normal((64, 256)).astype(np.float32)
    W = (rng.standard_normal((128, 256)) * 0.02).astype(np.float32)
    qa, sa = scaling.quantize_blockwise(A, 1, 128)
    qw, sw = scaling.quantize_blockwise(W, 128, 128)
    c = gemm.grouped_gemm(qa, sa, qw[None], sw[None], np.array([0, 64]))
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(c - ref)) < 0.05 * np.max(np.abs(ref))


def test_moe_counts_recipe():
    c = moe_token_counts()
    assert c.sum() == 16384 and c.size == 8
    assert np.all(c % 128 == 0) and c.min() >= 128 and c.max() <= 4096


def test_requant_bracket_hand_values():
    """Codes of re-quantised outputs, derived by hand from the formats."""
    # zero bound: one code each; 3*2 = 6 and -0.5*2 = -1 exact, 1000*2 saturates to 448
    r = gemm.requant_bracket(np.array([3.0, -0.5, 1000.0, 0.0]), np.zeros(4), np.float32(2.0), "e4m3")
    assert list(r["lo"]) == [6.0, -1.0, 448.0, 0.0] and list(r["hi"]) == [6.0, -1.0, 448.0, 0.0]
    assert r["amax"] == (1000.0, 1000.0) and r["sat"] == (1, 1)
    # 1.0625 is the midpoint of E4M3 1.0 and 1.125: ties to even give 1.0; any positive bound admits 1.125
    r = gemm.requant_bracket(np.array([1.0625]), np.array([0.0]), np.float32(1.0), "e4m3")
    assert r["lo"][0] == 1.0 and r["hi"][0] == 1.0
    r = gemm.requant_bracket(np.array([1.0625]), np.array([1e-6]), np.float32(1.0), "e4m3")
    assert r["lo"][0] == 1.0 and r["hi"][0] == 1.125
    # E5M2 around its max: c in [53248, 69632]; 53248 is the midpoint of 49152 (mantissa 10b) and
    # 57344 (11b), so it rounds to the even 49152; 69632 saturates to 57344
    r = gemm.requant_bracket(np.array([61440.0]), np.array([8192.0]), np.float32(1.0), "e5m2")
    assert r["lo"][0] == 49152.0 and r["hi"][0] == 57344.0
    assert r["sat"] == (0, 1) and r["amax"] == (53248.0, 69632.0)
    # a bracket across zero: the amax bracket starts at 0, negative and positive codes both admitted
    r = gemm.requant_bracket(np.array([0.25]), np.array([0.5]), np.float32(1.0), "e4m3")
    assert r["lo"][0] == -0.25 and r["hi"][0] == 0.75 and r["amax"] == (0.0, 0.75)


def _fraction_grouped_bound(qa, sa, qb, sb, offs, fa="e4m3", fb="e4m3", block=128):
    """1e-5 * sum_kb |sa[m,kb]| |sb[g,n/128,kb]| sum_{k in kb} |a_k| |b_k|, exactly, by loops."""
    G, N, K = qb.shape
    A = np.abs(codec.decode(qa, fa))
    out = np.zeros((int(offs[-1]), N))
    for g in range(G):
        B = np.abs(codec.decode(qb[g], fb))
        for m in range(int(offs[g]), int(offs[g + 1])):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    tot += Fraction(float(A[m, k])) * Fraction(float(B[n, k])) \
                        * abs(Fraction(float(sa[m, k // block]))) * abs(Fraction(float(sb[g, n // block, k // block])))
                out[m, n] = float(Fraction(1, 100000) * tot)
    return out


def test_grouped_abs_bound_against_fraction_brute_force():
    """The grouped tolerance, element by element, against an exact evaluation of
    its definition: an empty expert, N and K not multiples of 128 (partial
    weight and K blocks), block scales that differ per row, per 128-column
    block and per K block, some of them negative (the bound takes magnitudes).
    A wrong block index, a missing |.| or a dropped K block changes elements."""
    rng = np.random.default_rng(11)
    offs = np.array([0, 3, 3, 7])                  # expert 1 is empty
    K, N, G = 300, 150, 3                          # 3 K blocks (last 44 deep), 2 N blocks (last 22 wide)
    qa = _rand_codes(rng, (7, K), "e4m3")
    qb = _rand_codes(rng, (G, N, K), "e4m3")
    sa = (rng.uniform(0.5, 2, size=(7, 3)) * 2.0 ** rng.integers(-6, 6, size=(7, 3))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, size=(G, 2, 3)) * 2.0 ** rng.integers(-6, 6, size=(G, 2, 3))).astype(np.float32)
    sa[1, 2] *= -1
    sb[2, 1, 0] *= -1
    got = gemm.grouped_abs_bound(qa, sa, qb, sb, offs)
    want = _fraction_grouped_bound(qa, sa, qb, sb, offs)
    assert np.allclose(got, want, rtol=1e-12, atol=0)
    # a row subset gives the same rows
    rows = np.array([6, 0, 3])
    assert np.array_equal(gemm.grouped_abs_bound(qa, sa, qb, sb, offs, rows=rows), got[rows])
    # and the bound really is the tolerance of the grouped sum: the exact grouped
    # sum with every term's sign dropped is 1e5 times the bound
    mag = gemm.grouped_gemm(np.where(qa == 0x80, 0, qa & 0x7F).astype(np.uint8), np.abs(sa),
                            (qb & 0x7F).astype(np.uint8), np.abs(sb), offs)
    assert np.allclose(mag * 1e-5, got, rtol=1e-12, atol=0)


def test_grouped_abs_bound_mixed_formats_and_single_block():
    """E5M2 weights against E4M3 activations; K = 16 (one partial block) and
    N = 1: the bound reduces to 1e-5 |sa| |sb| sum_k |a_k b_k|."""
    rng = np.random.default_rng(12)
    qa = _rand_codes(rng, (2, 16), "e4m3")
    qb = _rand_codes(rng, (1, 1, 16), "e5m2")
    sa = np.array([[0.5], [-3.0]], dtype=np.float32)
    sb = np.array([[[0.125]]], dtype=np.float32)
    got = gemm.grouped_abs_bound(qa, sa, qb, sb, np.array([0, 2]), fa="e4m3", fb="e5m2")
    A, B = np.abs(codec.decode(qa, "e4m3")), np.abs(codec.decode(qb[0, 0], "e5m2"))
    for m, s in ((0, 0.5), (1, 3.0)):
        want = Fraction(1, 100000) * Fraction(s) * Fraction(0.125) * sum(
            (Fraction(float(x)) * Fraction(float(y)) for x, y in zip(A[m], B)), Fraction(0))
        assert abs(got[m, 0] - float(want)) <= 1e-12 * float(want)

"""Pins for the oracle's FP8 gradient all-reduce parts (CPU only)."""

import numpy as np

from oracle import allreduce, codec


def test_shared_scale_hand_values():
    # the largest amax over the ranks sets the scale: 57344 / 2 = 28672, 1 / 28672 rounded to fp32
    s, si = allreduce.shared_scale([0.5, 2.0, 1.0], "e5m2")
    assert s == np.float32(28672.0) and si == np.float32(1.0 / 28672.0)
    s, si = allreduce.shared_scale([0.03, 0.0], "e4m3")
    assert s == np.float32(np.float64(448.0) / np.float64(np.float32(0.03)))
    # nothing usable (all zero, or a NaN amax): scale 1
    assert allreduce.shared_scale([0.0, 0.0], "e5m2") == (1.0, 1.0)
    assert allreduce.shared_scale([1.0, np.nan], "e5m2") == (1.0, 1.0)


def test_exact_gradients_sum_exactly():
    """Gradients with amax 1.75 get the power-of-two shared scale 57344 / 1.75 =
    2^15, and values of at most three significant bits are exact E5M2 codes at
    that scale: every payload decodes back to its gradient and the restored sum
    equals the exact sum."""
    vals = np.array([0.25, -0.5, 1.0, 1.75, -1.75, 0.0, 2.0 ** -10, 1.5, -0.375], dtype=np.float32)
    rng = np.random.default_rng(1)
    grads = [vals[rng.integers(0, vals.size, size=64)] for _ in range(4)]
    for g in grads:
        g[0] = 1.75
    r = allreduce.fp8_allreduce(grads, "e5m2")
    assert r["scale"] == np.float32(32768.0) and r["scale_inv"] == np.float32(2.0 ** -15)
    for g, q in zip(grads, r["payloads"]):
        assert np.array_equal(codec.decode(q, "e5m2") * 2.0 ** -15, g.astype(np.float64))
    assert np.array_equal(r["sum"].astype(np.float64), np.sum(np.stack(grads).astype(np.float64), axis=0))


def test_identical_ranks_give_r_times_one_rank():
    rng = np.random.default_rng(2)
    g = (rng.standard_normal(1000) * 1e-3).astype(np.float32)
    one = allreduce.fp8_allreduce([g], "e5m2")["sum"]
    eight = allreduce.fp8_allreduce([g] * 8, "e5m2")["sum"]
    # 8 equal E5M2 values sum exactly in fp32 (3 significant bits, times 8); the restore then scales by 8
    assert np.array_equal(eight, (one * np.float32(8.0)).astype(np.float32))


def test_rank_order_of_the_fp32_sum():
    """E5M2 payloads 2^15, then 1, then 1 (scale_inv 1): rank order gives
    fp32(fp32(32768 + 1) + 1) = 32770 exactly; with 2^24 in place of 2^15 the ones
    are lost one at a time: the sum stays 2^24 (a pairwise (1 + 1) first would
    give 2^24 + 2)."""
    enc = lambda x: codec.encode(np.float32([x]), "e5m2")
    assert allreduce.dequant_sum([enc(32768.0), enc(1.0), enc(1.0)], "e5m2", np.float32(1.0))[0] == 32770.0
    big = np.float32(2.0 ** 24)
    # 2^24 is not an E5M2 value (max 57344), so build the fp32 accumulation with scale_inv = 2^9 instead
    s = allreduce.dequant_sum([enc(32768.0), enc(2.0 ** -9), enc(2.0 ** -9)], "e5m2", np.float32(2.0 ** 9))
    assert s[0] == np.float32((np.float32(32768.0) + np.float32(2.0 ** -9) + np.float32(2.0 ** -9)) * 512.0)
    assert s[0] == big

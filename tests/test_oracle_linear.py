"""Pins for the oracle's FP8 linear-layer step (forward, dgrad, wgrad) (CPU only)."""

import numpy as np

from oracle import codec, linear, scaling

# Values each format holds exactly.  The E4M3 set needs three mantissa bits
# (E5M2 cannot hold 1.125, 1.375, ...); the E5M2 set lies outside E4M3's range
# or below its smallest subnormal, so giving an operand the wrong format
# changes the result.
E4M3_ONLY = np.array([1.125, -1.375, 0.5625, 1.875, -2.25, 3.5, -0.8125, 0.0])
E5M2_ONLY = np.array([1024.0, -1536.0, 2.0 ** -12, -(2.0 ** -11), 3072.0, 0.75, -512.0, 0.0])


def _pick(rng, table, shape):
    return table[rng.integers(0, table.size, size=shape)].astype(np.float32)


def _states():
    return (scaling.DelayedScaling("e4m3", 16), scaling.DelayedScaling("e4m3", 16),
            scaling.DelayedScaling("e5m2", 16))


def test_formats_hold_the_chosen_values():
    assert np.array_equal(codec.decode(codec.encode(E4M3_ONLY.astype(np.float32), "e4m3"), "e4m3"), E4M3_ONLY)
    assert np.array_equal(codec.decode(codec.encode(E5M2_ONLY.astype(np.float32), "e5m2"), "e5m2"), E5M2_ONLY)
    # and not the other format's (so a swapped format would show)
    assert not np.array_equal(codec.decode(codec.encode(E4M3_ONLY.astype(np.float32), "e5m2"), "e5m2"), E4M3_ONLY)
    assert not np.array_equal(codec.decode(codec.encode(E5M2_ONLY.astype(np.float32), "e4m3"), "e4m3"), E5M2_ONLY)


def test_unit_scales_reduce_to_the_plain_products():
    """Fresh states cast with scale 1; with exactly representable inputs the three
    products are the fp64 matrix products of the inputs (all partial sums exact)."""
    rng = np.random.default_rng(11)
    T, I, O = 5, 7, 3
    x, w, dy = _pick(rng, E4M3_ONLY, (T, I)), _pick(rng, E4M3_ONLY, (O, I)), _pick(rng, E5M2_ONLY, (T, O))
    r = linear.hybrid_linear_step(x, w, dy, *_states())
    X, W, G = (a.astype(np.float64) for a in (x, w, dy))
    assert r["y"].shape == (T, O) and r["dx"].shape == (T, I) and r["dw"].shape == (O, I)
    assert np.array_equal(r["y"], X @ W.T)
    assert np.array_equal(r["dx"], G @ W)
    assert np.array_equal(r["dw"], G.T @ X)


def test_gradients_match_finite_differences_of_the_forward():
    """dX and dW are the derivatives of L = sum(Y * dY) with Y the oracle's own
    forward product: perturbing one input element by an exactly representable
    step changes L by exactly step * gradient (L is bilinear, sums are exact)."""
    rng = np.random.default_rng(12)
    T, I, O = 4, 6, 5
    x, w, dy = _pick(rng, E4M3_ONLY, (T, I)), _pick(rng, E4M3_ONLY, (O, I)), _pick(rng, E5M2_ONLY, (T, O))
    base = linear.hybrid_linear_step(x, w, dy, *_states())

    def loss(xx, ww):
        r = linear.hybrid_linear_step(xx, ww, dy, *_states())
        return float(np.sum(r["y"] * dy.astype(np.float64)))

    l0 = loss(x, w)

    def other(v):  # another value of the E4M3 table, so the perturbed input stays exact
        return np.float32(E4M3_ONLY[(int(np.flatnonzero(E4M3_ONLY == v)[0]) + 3) % E4M3_ONLY.size])

    for t, i in [(0, 0), (3, 5), (2, 1)]:
        xp = x.copy()
        xp[t, i] = other(x[t, i])
        step = float(xp[t, i]) - float(x[t, i])
        assert step != 0 and loss(xp, w) - l0 == step * base["dx"][t, i]
    for o, i in [(0, 0), (4, 2), (1, 5)]:
        wp = w.copy()
        wp[o, i] = other(w[o, i])
        step = float(wp[o, i]) - float(w[o, i])
        assert step != 0 and loss(x, wp) - l0 == step * base["dw"][o, i]


def test_second_step_uses_the_amax_derived_scales():
    """Step 1 casts with scale 1 and records each tensor's amax; step 2 casts
    with 448 / amax (E4M3) and 57344 / amax (E5M2).  Magnitudes span less than
    the formats' normal range, so at step 2 every code is normal and each
    product term is within the formats' relative rounding of the exact one."""
    rng = np.random.default_rng(13)
    T, I, O = 32, 48, 40

    def mags(lo, hi, shape):
        return (rng.uniform(lo, hi, shape) * rng.choice([-1.0, 1.0], shape)).astype(np.float32)

    x, w, dy = mags(0.01, 0.03, (T, I)), mags(0.005, 0.02, (O, I)), mags(2e-5, 1e-4, (T, O))
    sx, sw, sg = _states()
    r1 = linear.hybrid_linear_step(x, w, dy, sx, sw, sg)
    assert r1["scale_inv"] == (1.0, 1.0, 1.0)
    ax, aw, ag = (float(np.max(np.abs(a))) for a in (x, w, dy))
    assert (sx.scale, sw.scale, sg.scale) == (np.float32(448.0 / ax), np.float32(448.0 / aw),
                                              np.float32(57344.0 / ag))
    after_step1 = (sx.scale_inv, sw.scale_inv, sg.scale_inv)
    r2 = linear.hybrid_linear_step(x, w, dy, sx, sw, sg)
    assert r2["scale_inv"] == after_step1
    # E5M2 exponent field 0 = subnormal or zero: dY ~ 1e-4 at scale 1 has such codes, not at step 2
    assert np.any(((r1["qg"] >> 2) & 0x1F) == 0) and np.all(((r2["qg"] >> 2) & 0x1F) != 0)
    assert np.all(((r2["qx"] >> 3) & 0xF) != 0) and np.all(((r2["qw"] >> 3) & 0xF) != 0)
    X, W, G = (a.astype(np.float64) for a in (x, w, dy))
    # per term: (1 + 2^-4)^2 - 1 < 0.13 for E4M3 x E4M3, (1 + 2^-3)(1 + 2^-4) - 1 < 0.2 with E5M2
    for got, want, absprod, rel in ((r2["y"], X @ W.T, np.abs(X) @ np.abs(W).T, 0.13),
                                    (r2["dx"], G @ W, np.abs(G) @ np.abs(W), 0.2),
                                    (r2["dw"], G.T @ X, np.abs(G).T @ np.abs(X), 0.2)):
        assert np.all(np.abs(got - want) <= rel * absprod)

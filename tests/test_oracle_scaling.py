"""Pins for the oracle's amax, scale rule, delayed-scaling ring and scaled cast (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, scaling
from synth import adversarial_f32, stream_sigma


# --------------------------------------------------------------------------- worked numbers
def test_worked_example_a(golden):
    """Worked example A: amax 0.03 -> scale ~ 14933; range fills [-298, 448]."""
    g = golden("worked_example_a.txt")
    ok, s, si = scaling.scale_from_amax(np.float32(g["amax"]), g["fp8_max"])
    assert ok
    assert round(float(s)) == g["scale_approx"]
    assert float(s) == 14933.333984375                     # fp32 nearest to 448 / fp32(0.03)
    hi = np.float32(g["tensor_high"]) * s
    lo = np.float32(g["tensor_low"]) * s
    assert float(hi) == g["scaled_range_high"]
    assert int(float(lo)) == g["scaled_range_low_printed"]  # page prints the truncation of -298.67
    x = np.array([g["tensor_low"], g["tensor_high"]], dtype=np.float32)
    q, am, sat = scaling.quantize(x, s, "e4m3")
    assert float(am) == float(np.float32(g["amax"]))
    assert q.tolist() == [0xF9, 0x7E] and sat == 0
    assert codec.decode(q, "e4m3").tolist() == [-288.0, 448.0]
    ok, s2, _ = scaling.scale_from_amax(np.float32(g["large_amax"]), g["fp8_max"])
    assert ok and float(s2) == float(np.float32(g["large_scale"])) and s2 < 1


def test_exercise_2_closed_form(golden):
    g = golden("exercise_2.txt")
    ok, sa, _ = scaling.scale_from_amax(np.float32(g["amax_a"]), g["fp8_max"])
    assert ok and float(sa) == g["scale_a_exact"]
    ok, sb, _ = scaling.scale_from_amax(np.float32(g["amax_b"]), g["fp8_max"])
    exact = Fraction(int(g["scale_b_num"]), int(g["scale_b_den"]))
    # fp32 nearest to 28/75: no fp32 value is closer
    s = Fraction(float(sb))
    up = Fraction(float(np.nextafter(sb, np.float32(1))))
    dn = Fraction(float(np.nextafter(sb, np.float32(0))))
    assert abs(s - exact) <= abs(up - exact) and abs(s - exact) <= abs(dn - exact)


# --------------------------------------------------------------------------- scale rule
def test_scale_matches_numpy_fp32_division():
    """fp32(MAX/m) via one fp64 quotient == IEEE fp32 division done by numpy."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0x00800000, 0x7F000000, size=200000, dtype=np.uint64).astype(np.uint32)
    m = bits.view(np.float32)
    for fmax in (448.0, 57344.0):
        with np.errstate(over="ignore"):
            want = np.float32(fmax) / m
        for i in range(0, m.size, 997):
            ok, s, si = scaling.scale_from_amax(m[i], fmax)
            if np.isfinite(want[i]):
                assert ok and s == want[i]
                assert si == np.float32(1.0) / want[i]
            else:
                assert not ok


@pytest.mark.parametrize("m", [0.0, np.inf, np.nan, 1e-45, 3e-41])
def test_scale_held_for_zero_nonfinite_or_overflowing(m):
    ok, _, _ = scaling.scale_from_amax(np.float32(m), 448.0)
    assert not ok


# --------------------------------------------------------------------------- amax
def test_amax_is_max_abs_for_finite():
    rng = np.random.default_rng(4)
    for shape in [(1,), (7,), (33, 65), (128, 4096)]:
        x = (rng.standard_normal(shape) * 10 ** rng.uniform(-5, 5)).astype(np.float32)
        assert scaling.amax(x) == np.max(np.abs(x))


def test_amax_propagates_nan_and_inf_and_ignores_sign_of_zero():
    x = np.array([1.0, -3.0, 2.0], dtype=np.float32)
    assert scaling.amax(x) == 3.0
    assert np.isinf(scaling.amax(np.append(x, -np.inf)))
    assert np.isnan(scaling.amax(np.append(x, [np.nan, np.inf])))
    assert scaling.amax(np.array([-0.0, 0.0], dtype=np.float32)) == 0.0
    assert not np.signbit(scaling.amax(np.array([-0.0], dtype=np.float32)))


def test_widen_bf16_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    f = scaling.widen(bits.astype(np.uint16), "bf16")
    assert np.array_equal(f.view(np.uint32), bits << np.uint32(16))


# --------------------------------------------------------------------------- delayed scaling
def _drive(amaxes, length=16, fmax=448.0):
    st = scaling.DelayedScaling("e4m3" if fmax == 448.0 else "e5m2", length)
    used = []
    for a in amaxes:
        used.append(st.scale)        # the scale a cast at this step would use
        st.update(np.float32(a))
    return st, used


def test_fresh_state_and_first_step_uses_scale_one():
    st = scaling.DelayedScaling("e4m3", 16)
    assert st.scale == 1.0 and st.scale_inv == 1.0 and st.head == 0 and not st.history.any()
    _, used = _drive([2.0, 4.0])
    assert used[0] == 1.0 and float(used[1]) == 224.0


def test_scale_uses_max_of_last_n_past_amaxes_only():
    rng = np.random.default_rng(8)
    amaxes = np.float32(10.0 ** rng.uniform(-3, 3, size=60))
    for n in (1, 4, 16):
        _, used = _drive(amaxes, length=n)
        for t in range(1, 60):
            m = np.max(amaxes[max(0, t - n):t])
            assert used[t] == np.float32(448.0) / np.float32(m), (n, t)


def test_history_length_one_is_previous_step_only():
    amaxes = np.float32([5, 50, 0.5, 7])
    _, used = _drive(amaxes, length=1)
    assert [float(u) for u in used[1:]] == [float(np.float32(448) / np.float32(a)) for a in amaxes[:-1]]


def test_stream_drift_and_spike_invariants():
    """Drift x1.05 per step with a x50 spike at step 20: the amax sequence here is
    the sigma sequence itself (a stand-in with the same ordering)."""
    sig = np.float32([stream_sigma(t) for t in range(32)])
    _, used = _drive(sig, length=16)
    for t in range(1, 21):                   # monotone drift: previous step's amax rules
        assert used[t] == np.float32(448) / sig[t - 1]
    assert used[20] > np.float32(448) / sig[20]       # the spike is cast with a stale, too large scale
    for t in range(21, 32):                  # spike stays in the 16-long window and dominates
        assert used[t] == np.float32(448) / sig[20]


def test_hold_on_zero_nan_inf_and_wraparound():
    st = scaling.DelayedScaling("e4m3", 4)
    st.update(np.float32(0.0))
    assert st.scale == 1.0 and st.status & scaling.STATUS_HELD
    st = scaling.DelayedScaling("e4m3", 4)
    st.update(np.float32(2.0))
    s_before = st.scale
    st.update(np.float32(np.nan))
    assert st.scale == s_before and st.status == scaling.STATUS_HELD
    for _ in range(3):                       # NaN stays in the window for 4 updates
        st.update(np.float32(1.0))
        assert st.scale == s_before
    st.update(np.float32(1.0))               # NaN has left the ring
    assert st.scale == 448.0 and st.head == 2
    st.update(np.float32(np.inf))
    assert st.scale == 448.0


# --------------------------------------------------------------------------- cast
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_is_encode_of_fp32_product(fmt):
    rng = np.random.default_rng(11)
    x = np.concatenate([adversarial_f32(seed=2, random_count=2000),
                        (rng.standard_normal(5000) * 3).astype(np.float32)])
    for s in (np.float32(1.0), np.float32(14933.334), np.float32(0.448), np.float32(3.0e-3)):
        with np.errstate(over="ignore", invalid="ignore"):
            p = x * s                                 # IEEE fp32 multiply (numpy), independent path
        q, am, sat = scaling.quantize(x, s, fmt)
        assert np.array_equal(q, codec.encode(p, fmt))
        with np.errstate(invalid="ignore"):
            assert sat == int(np.sum(np.abs(p) > codec.FORMATS[fmt].max_value))
        assert am.view(np.uint32) == np.max(x.view(np.uint32) & np.uint32(0x7FFFFFFF))


def test_saturation_never_produces_inf_or_nan_for_finite_inputs():
    x = np.float32([1e3, -1e3, 3e38, -3e38])
    q, _, sat = scaling.quantize(x, np.float32(448.0), "e5m2")
    assert q.tolist() == [0x7B, 0xFB, 0x7B, 0xFB] and sat == 4


# --------------------------------------------------------------------------- per-block scaling
@pytest.mark.parametrize("shape,br,bc", [((5, 300), 1, 128), ((260, 300), 128, 128), ((1, 1), 1, 128)])
def test_blockwise_matches_per_block_loop(shape, br, bc):
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(shape) * 10 ** rng.uniform(-3, 3, size=shape)).astype(np.float32)
    if shape[0] > 1:
        x[0, :min(128, shape[1])] = 0.0          # an all-zero block gets scale 1
    q, si = scaling.quantize_blockwise(x, br, bc)
    R, C = shape
    for i in range(0, R, br):
        for j in range(0, C, bc):
            blk = x[i:i + br, j:j + bc]
            m = np.max(np.abs(blk))
            s = np.float32(448.0) / m if m > 0 else np.float32(1.0)
            with np.errstate(over="ignore"):
                want = codec.encode(blk * s, "e4m3")
            assert np.array_equal(q[i:i + br, j:j + bc], want)
            assert si[i // br, j // bc] == np.float32(1.0) / s

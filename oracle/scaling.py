"""amax, scale rule, delayed-scaling history, scaled cast, per-block scaling
(test infrastructure; CPU oracle).

What the pages fix ("4.2 Hopper I — Transformer Engine·FP8")
-------------------------------------------------------------
* §4.2.4: amax is the absolute maximum of the tensor; the scale is about
  FP8_MAX / amax; the FP8 tensor is round_to_fp8(tensor × scale); using a
  scale from an underestimated amax saturates large values, one from an
  overestimated amax pushes small values into underflow.
* §4.2.4 delayed scaling: the scale for this step is predicted from the amax
  history of past steps (e.g. the max over the last N steps) so the tensor is
  cast in one pass; the price is a one-step lag behind spikes.
* §4.2.5 worked example A: FP8_MAX 448, amax 0.03 -> scale about 14933, the
  scaled range fills [-298, 448]; amax 1000 -> scale 0.448.
* §4.2.6 recipe: amax_history_len = 16, amax_compute_algo = "max"; HYBRID =
  E4M3 forward, E5M2 backward; TE updates amax after the step to set the next
  step's scale.
* §4.2.10 exercise 2: amax 0.05 and 1200 with FP8_MAX 448.
* "FP8 and low-precision formats", "Deep dive": per-tensor OR per-block
  scale factors.

Readings where the pages are silent (each listed in the design notes):
* amax of the *unscaled* input, as the max of |x| over fp32 bit patterns
  (bits & 0x7FFFFFFF compared as integers): exact, order-free, and NaN > Inf >
  every finite value, so non-finite inputs reach the history.
* scale = fp32(FP8_MAX / m) correctly rounded; no margin, no power-of-two
  rounding.  scale_inv = fp32(1 / scale).  (Computed as the fp64 quotient
  rounded once to fp32, which equals the correctly rounded fp32 quotient.)
* The scale is updated only when m is finite and > 0 and the quotient is
  finite; otherwise scale and scale_inv are held and status bit 0 is set.
  Fresh state: history all 0, head 0, scale 1, scale_inv 1.
* The cast multiplies in fp32 (one rounding, RNE), then encodes (a second
  rounding).  bf16 inputs are widened exactly to fp32 first.
* Saturation count = #{ |fp32(x·s)| > FP8_MAX } (Inf counts, NaN does not).
* Per-block (current) scaling: each block gets scale fp32(448 / amax_block),
  with 1.0 when the block amax is 0 or non-finite or the quotient overflows.

Parity status: pinned (worked example A, exercise 2, closed forms, a
cross-check against numpy's own fp32 division, history invariants).
"""

from __future__ import annotations

import numpy as np

from . import codec

__all__ = ["widen", "amax", "scale_from_amax", "DelayedScaling", "quantize", "saturation_count",
           "quantize_blockwise", "STATUS_HELD"]

STATUS_HELD = 1


def widen(data: np.ndarray, dtype: str) -> np.ndarray:
    """Return the fp32 values of a host input (exact for bf16 bit patterns)."""
    if dtype == "f32":
        return np.ascontiguousarray(data, dtype=np.float32)
    if dtype == "bf16":
        return (np.ascontiguousarray(data, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def amax(x32: np.ndarray) -> np.float32:
    """max |x| as the integer max over magnitude bit patterns (NaN/Inf propagate)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)
    m = b.max() if b.size else np.uint32(0)
    return np.asarray(m, dtype=np.uint32).view(np.float32)[()]


def _fp32_div(num: float, den) -> np.float32:
    """Correctly rounded fp32 quotient of two fp32 values (via one fp64 division:
    53 >= 2*24 + 2 makes the fp64 -> fp32 double rounding exact)."""
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        return np.float32(np.float64(np.float32(num)) / np.float64(np.float32(den)))


def scale_from_amax(m, fmt_max: float):
    """(ok, scale, scale_inv): scale = fp32(fmt_max / m) when 0 < m < inf and the
    quotient is finite; ok False otherwise (caller holds the old scale)."""
    m = np.float32(m)
    if not (np.isfinite(m) and m > 0):
        return False, None, None
    s = _fp32_div(fmt_max, m)
    if not np.isfinite(s) or s == 0:
        return False, None, None
    return True, s, _fp32_div(1.0, s)


class DelayedScaling:
    """Per-tensor delayed-scaling state: an amax history ring of ``length``
    entries, a head index, the current scale and its inverse, a status word."""

    def __init__(self, fmt="e4m3", length: int = 16):
        self.fmt = codec._fmt(fmt)
        self.length = int(length)
        self.history = np.zeros(self.length, dtype=np.float32)
        self.head = 0
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.status = 0

    def copy(self) -> "DelayedScaling":
        c = DelayedScaling(self.fmt, self.length)
        c.history = self.history.copy()
        c.head, c.scale, c.scale_inv, c.status = self.head, self.scale, self.scale_inv, self.status
        return c

    def history_max(self) -> np.float32:
        """The "max" rule over the whole ring (integer max over bit patterns)."""
        return amax(self.history)

    def update(self, new_amax) -> None:
        """Record this step's amax, advance the head, recompute the scale used
        by the NEXT cast from the max of the history."""
        self.history[self.head] = np.float32(new_amax)
        self.head = (self.head + 1) % self.length
        ok, s, si = scale_from_amax(self.history_max(), self.fmt.max_value)
        if ok:
            self.scale, self.scale_inv = s, si
        else:
            self.status |= STATUS_HELD


def _scaled(x32: np.ndarray, scale) -> np.ndarray:
    """fp32(x * s): the exact product of two fp32 numbers fits in fp64, so
    rounding it once to fp32 is the correctly rounded fp32 product."""
    with np.errstate(over="ignore", invalid="ignore"):
        return (x32.astype(np.float64) * np.float64(np.float32(scale))).astype(np.float32)


def saturation_count(p32: np.ndarray, fmt) -> int:
    f = codec._fmt(fmt)
    with np.errstate(invalid="ignore"):
        return int(np.count_nonzero(np.abs(p32.astype(np.float64)) > f.max_value))


def quantize(x32: np.ndarray, scale, fmt):
    """Scaled saturating cast of one tensor with a given (delayed) scale.

    Returns (codes uint8, amax of the unscaled input, saturation count).
    """
    p = _scaled(x32, scale)
    return codec.encode(p, fmt), amax(x32), saturation_count(p, fmt)


def _block_scales(m: np.ndarray, fmt_max: float):
    """Vector form of ``scale_from_amax`` with the per-block fallback scale 1.0."""
    m = np.asarray(m, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        s = (np.float64(np.float32(fmt_max)) / m.astype(np.float64)).astype(np.float32)
        ok = np.isfinite(m) & (m > 0) & np.isfinite(s) & (s != 0)
        s = np.where(ok, s, np.float32(1.0)).astype(np.float32)
        si = (1.0 / s.astype(np.float64)).astype(np.float32)
    return s, si


def quantize_blockwise(x32: np.ndarray, block_rows: int, block_cols: int, fmt="e4m3"):
    """Current (not delayed) per-block scaling of a 2-D tensor.

    Every block of ``block_rows x block_cols`` (ragged at the edges) gets its
    own scale fp32(MAX / amax_block) (1.0 for an all-zero or non-finite block);
    returns (codes [R x C] uint8, scale_inv [ceil(R/br) x ceil(C/bc)] fp32).
    """
    f = codec._fmt(fmt)
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    R, C = x32.shape
    nbr, nbc = -(-R // block_rows), -(-C // block_cols)
    mag = x32.view(np.uint32) & np.uint32(0x7FFFFFFF)
    pad = np.zeros((nbr * block_rows, nbc * block_cols), dtype=np.uint32)   # 0 never wins a max
    pad[:R, :C] = mag
    bmax = pad.reshape(nbr, block_rows, nbc, block_cols).max(axis=(1, 3)).view(np.float32)
    s, si = _block_scales(bmax, f.max_value)
    s_el = np.repeat(np.repeat(s, block_rows, axis=0), block_cols, axis=1)[:R, :C]
    p = _scaled_elementwise(x32, s_el)
    return codec.encode(p, f), si


def _scaled_elementwise(x32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore", invalid="ignore"):
        return (x32.astype(np.float64) * s32.astype(np.float64)).astype(np.float32)

"""MXFP8: FP8 elements sharing one power-of-two scale per block of 32
consecutive values of a row, and the GEMM on such operands (test
infrastructure; CPU oracle).

What the pages fix
------------------
* "FP8 and low-precision formats", "Deep dive": scale factors per tensor or
  per block keep values inside FP8's usable range; newer formats (MXFP8,
  MXFP4, NVFP4) go further with shared micro-scaling blocks.
* "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: a block's amax sets its
  scale so that the block fits the format (scale about MAX / amax), the cast
  saturates beyond max; §4.2.8 the OCP FP8 element formats.

Readings where the pages are silent (each listed in the design notes):
* A block is 32 consecutive values along a row (the K direction of a GEMM
  operand); its scale is a power of two, 2^e, stored as an 8-bit exponent
  code e + 127 (0 .. 254).
* e is the smallest integer with amax <= MAX * 2^e: the power-of-two version
  of the pages' rule "scale = MAX / amax" (the block's amax lands in
  (MAX/2, MAX], nothing saturates); clamped to [-127, 127].  A block whose
  amax is 0, Inf or NaN gets e = 0.
* The element codes are round_to_fp8(fp32(x * 2^-e)) with the cast's rule
  (RNE, saturating, NaN -> sign|0x7F).  Multiplying by a power of two is exact
  in fp32 except where the result underflows, and there the code is +-0 either
  way.
* The GEMM's value is sum_k dec(a) 2^ea(k) * dec(b) 2^eb(k) (fp64 here).

Parity status: pinned (tests/test_oracle_mx.py): hand-computed exponents
(format maxima and their neighbours, powers of two, subnormal amax, zero and
non-finite blocks), the no-saturation and tightness properties, exact round
trips of representable blocks, and the GEMM against a per-block loop.
"""

from __future__ import annotations

import math

import numpy as np

from . import codec, scaling

__all__ = ["BLOCK", "scale_exponent", "quantize_mx", "dequant_mx", "mx_gemm"]

BLOCK = 32


def scale_exponent(amax, fmt) -> int:
    """Smallest integer e with amax <= MAX * 2^e, clamped to [-127, 127];
    0 when amax is 0 or not finite."""
    f = codec._fmt(fmt)
    a = float(np.float32(amax))
    if not math.isfinite(a) or a == 0.0:
        return 0
    e = math.ceil(math.log2(a / f.max_value))
    # exact correction of the floating-point guess: ldexp and the comparison are exact
    while a > math.ldexp(f.max_value, e):
        e += 1
    while a <= math.ldexp(f.max_value, e - 1):
        e -= 1
    return max(-127, min(127, e))


def quantize_mx(x32: np.ndarray, fmt):
    """x32 [rows x cols] fp32 (cols a multiple of 32) -> (codes uint8 [rows x cols],
    scale codes uint8 [rows x cols/32])."""
    f = codec._fmt(fmt)
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    rows, cols = x32.shape
    assert cols % BLOCK == 0
    nb = cols // BLOCK
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, nb), dtype=np.uint8)
    for r in range(rows):
        for b in range(nb):
            blk = x32[r, b * BLOCK:(b + 1) * BLOCK]
            e = scale_exponent(scaling.amax(blk), f)
            scales[r, b] = e + 127
            codes[r, b * BLOCK:(b + 1) * BLOCK], _, _ = scaling.quantize(blk, np.float32(math.ldexp(1.0, -e)), f)
    return codes, scales


def dequant_mx(codes, scales, fmt) -> np.ndarray:
    """Element values times their block's 2^e, in fp64."""
    f = codec._fmt(fmt)
    v = codec.decode(codes, f)
    e = scales.astype(np.int64) - 127
    return v * np.ldexp(1.0, np.repeat(e, BLOCK, axis=1)[:, :v.shape[1]])


def mx_gemm(qa, sa, fa, qb, sb, fb) -> np.ndarray:
    """C[m, n] = sum_k dec(a[m,k]) 2^ea[m,k/32] * dec(b[n,k]) 2^eb[n,k/32] (fp64);
    both operands [rows x K], K contiguous."""
    return dequant_mx(qa, sa, fa) @ dequant_mx(qb, sb, fb).T

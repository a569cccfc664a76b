"""OCP 8-bit floating point: E4M3 and E5M2 (test infrastructure; CPU oracle).

What the pages fix
------------------
* Two layouts: E4M3 = 1 sign, 4 exponent, 3 mantissa bits (more precision,
  less range; weights and activations); E5M2 = 1 sign, 5 exponent, 2 mantissa
  bits (more range, coarser steps; gradients).  ("FP8 and low-precision
  formats", "Deep dive"; "4.2 Hopper I — Transformer Engine·FP8", §4.2.3.)
* The layouts are the OCP FP8 standard that other vendors adopt (§4.2.8).
* The E4M3 maximum is taken as 448 (§4.2.5, worked example A).

The exact special values are left to the standard by §4.2.3.  Reading used
(OCP 8-bit floating point, the variant whose E4M3 maximum is 448):

* E4M3: bias 7; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is
  NaN; there is no infinity; max 448 (0x7E); min normal 2^-6; min subnormal
  2^-9.
* E5M2: bias 15; IEEE-like; exponent field 31 with mantissa 0 is +-Inf,
  otherwise NaN; max 57344 (0x7B); min normal 2^-14; min subnormal 2^-16.

Encoding an fp32 value (reading of "round_to_fp8" in §4.2.4, saturation in
§4.2.4 / §4.2.9):
  1. NaN -> sign | 0x7F.
  2. |v| > max (including +-Inf) -> sign | max code   (saturate, never Inf).
  3. otherwise round |v| to the nearest representable value, ties to the
     even mantissa (code LSB 0); gradual underflow through subnormals;
     |v| <= half the min subnormal -> signed zero.
  4. the sign bit is always kept (-0.0 -> 0x80).

Three encoders are given, written independently of each other so that each
can pin the others:
  ``encode``          integer rounding on the fp32 bit pattern (the one the
                      rest of the oracle uses);
  ``encode_rint``     fp64 arithmetic: frexp/ldexp to the quantum, ``rint``;
  ``encode_nearest``  brute force: nearest of all finite codes by distance.

Parity status: pinned (exhaustive round trip of all 256 codes per format,
encoder agreement over every fp32 bit pattern in each format's active band,
brute force on samples, the pages' worked numbers; ``encode`` equals the
value-based C encoder of codec_ref.c on all 2^32 fp32 bit patterns of both
formats, tests/test_oracle_codec_exhaustive.py).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Fp8Format", "E4M3", "E5M2", "FORMATS", "decode", "encode", "encode_rint",
           "encode_nearest", "finite_table"]


@dataclass(frozen=True)
class Fp8Format:
    name: str
    ebits: int
    mbits: int
    bias: int
    max_code: int       # code of the largest finite magnitude
    max_value: float    # its value
    has_inf: bool

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal number (1 - bias)."""
        return 1 - self.bias


E4M3 = Fp8Format("e4m3", 4, 3, 7, 0x7E, 448.0, False)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 0x7B, 57344.0, True)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}


def _fmt(f) -> Fp8Format:
    return FORMATS[f] if isinstance(f, str) else f


# ---------------------------------------------------------------------------
# Decoder: the value each code stands for, straight from the bit fields.
# ---------------------------------------------------------------------------
def decode(codes, fmt) -> np.ndarray:
    """Decode uint8 codes to float64 values (NaN for NaN codes, +-Inf for E5M2 Inf)."""
    f = _fmt(fmt)
    c = np.asarray(codes, dtype=np.int64)
    sign = (c >> 7) & 1
    e = (c >> f.mbits) & ((1 << f.ebits) - 1)
    m = c & ((1 << f.mbits) - 1)
    sub = np.ldexp(m.astype(np.float64), f.emin - f.mbits)
    nor = np.ldexp(((1 << f.mbits) + m).astype(np.float64), e - f.bias - f.mbits)
    mag = np.where(e == 0, sub, nor)
    emax_field = (1 << f.ebits) - 1
    if f.has_inf:
        mag = np.where((e == emax_field) & (m == 0), np.inf, mag)
        mag = np.where((e == emax_field) & (m != 0), np.nan, mag)
    else:
        mag = np.where((e == emax_field) & (m == (1 << f.mbits) - 1), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def finite_table(fmt) -> np.ndarray:
    """Values of the non-negative finite codes 0 .. max_code, ascending."""
    f = _fmt(fmt)
    return decode(np.arange(f.max_code + 1), f)


def _f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)


_MAXBITS = {"e4m3": int(np.float32(448.0).view(np.uint32)), "e5m2": int(np.float32(57344.0).view(np.uint32))}


# ---------------------------------------------------------------------------
# Encoder 1: integer round-to-nearest-even on the fp32 bit pattern.
# ---------------------------------------------------------------------------
def encode(x, fmt) -> np.ndarray:
    """Encode fp32 values to FP8 codes (uint8): RNE, saturating, NaN -> s|0x7F.

    |x| = S * 2**(E' - 150) with S the 24-bit significand (hidden bit included
    for normal fp32) and E' = max(E, 1).  The FP8 quantum is
    2**(max(e, emin) - mbits), e = floor(log2|x|); dividing S by the quantum is
    a right shift by ``sh`` with round-to-nearest-even on the dropped bits.
    The code is then n + ((max(e, emin) - emin) << mbits): a carry out of the
    mantissa moves into the exponent field by itself.
    """
    f = _fmt(fmt)
    u = _f32_bits(x)
    sign = (u >> 31) << 7
    a = u & 0x7FFFFFFF
    E = a >> 23
    F = a & 0x7FFFFF
    S = np.where(E == 0, F, F | 0x800000)
    Ee = np.maximum(E, 1)
    e = Ee - 127
    eq = np.maximum(e, f.emin)
    sh = (eq - f.mbits) - (Ee - 150)
    sh = np.clip(sh, 1, 40)                     # sh >= 23 - mbits in practice; > 25 gives n = 0
    q = S >> sh
    r = S & ((np.int64(1) << sh) - 1)
    half = np.int64(1) << (sh - 1)
    n = q + ((r > half) | ((r == half) & ((q & 1) == 1))).astype(np.int64)
    code = n + ((eq - f.emin) << f.mbits)
    code = np.where(a > _MAXBITS[f.name], f.max_code, code)   # saturate (and Inf)
    code = np.where(a > 0x7F800000, 0x7F, code)               # NaN
    return (code | sign).astype(np.uint8).reshape(np.shape(x))


# ---------------------------------------------------------------------------
# Encoder 2: fp64 arithmetic (frexp / ldexp / rint), then value -> code lookup.
# ---------------------------------------------------------------------------
def encode_rint(x, fmt) -> np.ndarray:
    f = _fmt(fmt)
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    neg = np.signbit(x32)
    with np.errstate(invalid="ignore"):
        v = np.abs(x32.astype(np.float64))
    finite = np.isfinite(v)
    vv = np.where(finite, v, 0.0)
    _, ex = np.frexp(vv)                      # vv = m * 2**ex, m in [0.5, 1)
    e = np.where(vv > 0, ex - 1, f.emin)
    qexp = np.maximum(e, f.emin) - f.mbits
    n = np.rint(np.ldexp(vv, -qexp))          # exact scaling, then round half to even
    r = np.ldexp(n, qexp)
    table = finite_table(f)
    r = np.minimum(r, f.max_value)
    idx = np.searchsorted(table, r)
    idx = np.minimum(idx, f.max_code)
    assert np.all(table[idx] == r), "rounded value is not an FP8 value"
    code = idx.astype(np.int64)
    code = np.where(~finite | (v > f.max_value), f.max_code, code)
    code = np.where(np.isnan(x32), 0x7F, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8).reshape(np.shape(x))


# ---------------------------------------------------------------------------
# Encoder 3: brute force over every finite code (for samples).
# ---------------------------------------------------------------------------
def encode_nearest(x, fmt) -> np.ndarray:
    """Nearest finite code by absolute distance; ties go to the even code;
    NaN -> s|0x7F; |x| > max -> max code."""
    f = _fmt(fmt)
    x32 = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    table = finite_table(f)
    out = np.empty(x32.size, dtype=np.uint8)
    for i, xv in enumerate(x32):
        s = 0x80 if np.signbit(xv) else 0
        if np.isnan(xv):
            out[i] = s | 0x7F
            continue
        v = abs(float(xv))
        if v > f.max_value:
            out[i] = s | f.max_code
            continue
        d = np.abs(table - v)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:
            best = best[best % 2 == 0]
        out[i] = s | int(best[0])
    return out

"""Dequantised FP8 GEMM, its error bound, and the fine-grained grouped GEMM
(test infrastructure; CPU oracle).

What the pages fix
------------------
* "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: the GEMM runs on FP8
  inputs, accumulates in FP32, and the result is restored by ×(1/scale) of
  each operand; accumulation is always high precision.  §4.2.6: HYBRID uses
  E4M3 for forward operands and E5M2 for gradients.
* "FP8 and low-precision formats", "Technical insight": scale, FP8
  multiply-accumulate, divide back, partial sums kept in FP16/FP32.
* "#fp8" tag page, DeepGEMM entry: grouped GEMM for MoE and two-level
  accumulation ("promotion") of FP8 partial sums; "Deep dive" of the formats
  page: scale factors per tensor or per block.

Definitions used here
---------------------
``dequant_gemm``   C[m,n] = (sum_k dec(a[m,k]) * dec(b[k,n])) * sinv_a * sinv_b
                   in fp64, where sinv_a, sinv_b are the fp32 inverse scales
                   handed to the GEMM.  Products of two FP8 values are exact
                   in fp64; the fp64 sum's rounding is far below the bound.
``exact_dot``      the same inner sum with no rounding at all: every E4M3 value
                   is an integer times 2^-9 and every E5M2 value an integer
                   times 2^-16, so the sum is an exact integer times a power
                   of two.
``abs_bound``      1e-5 * sum_k |dec(a) dec(b)| * sinv_a * sinv_b: the per
                   element tolerance for fp32 outputs.
``bf16_bracket``   for bf16 outputs: round-to-nearest-even is monotone, so a
                   bf16 result is acceptable iff it lies between the bf16
                   roundings of C64 - bound and C64 + bound.
``requant_bracket`` for FP8 outputs re-quantised with the next consumer's
                   scale s ("4.2 Hopper I", §4.2.4: the restore combined with
                   the next stage's scale): the code is round_to_fp8(fp32(c*s))
                   for the fp32 result c, which is only fixed up to the bound;
                   fp32 rounding, the multiply by s > 0 and the encoding are
                   all monotone, so an output code is acceptable iff its value
                   lies between those of the encodings of C64 - bound and
                   C64 + bound.  The same monotone argument brackets the amax
                   of the results and the saturation count.
``grouped_gemm``   per expert g and per 128-wide K block kb,
                   C[m,n] += sinv_a[m,kb] * sinv_b[g, n//128, kb] *
                             sum_{k in kb} dec(a[m,k]) dec(b_g[n,k]).

Parity status: requant_bracket is pinned by hand-computed codes (exact
values, a round-to-even midpoint, saturation) in tests/test_oracle_gemm.py;
grouped_abs_bound by an exact Fraction evaluation of its definition (an empty
expert, partial weight and K blocks, per-row / per-block / negative scales)
and by its identity with 1e-5 times the grouped sum of magnitudes.
The sum is pinned (exact integer dot products on small
matrices and on sampled elements; one-hot, permutation, all-zero and
all-max operands with closed-form results).  The fp32 accumulation ORDER of
the device is not pinned; the device is held to the stated bound instead.
"""

from __future__ import annotations

import numpy as np

from . import codec, scaling

__all__ = ["dequant_gemm", "exact_dot", "exact_gemm_small", "abs_bound", "bf16_round",
           "bf16_bracket", "requant_bracket", "grouped_gemm", "grouped_abs_bound", "INT_SHIFT"]

# Every finite value of the format is an integer multiple of 2**-INT_SHIFT.
INT_SHIFT = {"e4m3": 9, "e5m2": 16}


def _dec(q, fmt) -> np.ndarray:
    return codec.decode(q, fmt)


def dequant_gemm(qa, fa, qb, fb, sinv_a, sinv_b) -> np.ndarray:
    """qa [M x K] codes, qb [K x N] codes (logical orientation) -> fp64 [M x N]."""
    A = _dec(qa, fa)
    B = _dec(qb, fb)
    return (A @ B) * np.float64(np.float32(sinv_a)) * np.float64(np.float32(sinv_b))


def abs_bound(qa, fa, qb, fb, sinv_a, sinv_b, rel: float = 1e-5) -> np.ndarray:
    A = np.abs(_dec(qa, fa))
    B = np.abs(_dec(qb, fb))
    return rel * (A @ B) * np.float64(np.float32(sinv_a)) * np.float64(np.float32(sinv_b))


def _int_codes(q, fmt) -> np.ndarray:
    """Integer I with dec(q) = I * 2**-INT_SHIFT[fmt] (finite codes only)."""
    f = codec._fmt(fmt)
    v = _dec(q, f)
    if not np.all(np.isfinite(v)):
        raise ValueError("exact_dot needs finite codes")
    i = np.ldexp(v, INT_SHIFT[f.name])
    assert np.all(i == np.rint(i))
    return i.astype(np.int64)


def exact_dot(a_codes, fa, b_codes, fb):
    """Exact sum_k dec(a_k) dec(b_k) as (integer N, shift s) with value N * 2**-s."""
    ia = _int_codes(np.asarray(a_codes).reshape(-1), fa)
    ib = _int_codes(np.asarray(b_codes).reshape(-1), fb)
    total = 0
    for s in range(0, ia.size, 1024):       # each 1024-term chunk fits in int64
        total += int(np.dot(ia[s:s + 1024], ib[s:s + 1024]))
    return total, INT_SHIFT[codec._fmt(fa).name] + INT_SHIFT[codec._fmt(fb).name]


def exact_gemm_small(qa, fa, qb, fb):
    """Exact inner sums for small matrices by explicit loops; returns fp64 values
    (exactly representable when they fit in 53 bits, which holds for the sizes
    this is used with) of sum_k dec(a[m,k]) dec(b[k,n])."""
    M, K = qa.shape
    K2, N = qb.shape
    assert K == K2
    out = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            num, sh = exact_dot(qa[m, :], fa, qb[:, n], fb)
            out[m, n] = np.ldexp(float(num), -sh)
    return out


def bf16_round(x) -> np.ndarray:
    """fp64 -> fp32 (nearest even) -> bf16 (nearest even), returned as fp32 values."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def bf16_bracket(c64, bound):
    """(lo, hi) fp32 arrays such that a bf16 output y is within the bound iff lo <= y <= hi."""
    return bf16_round(c64 - bound), bf16_round(c64 + bound)


def requant_bracket(c64, bound, out_scale, fmt) -> dict:
    """Acceptance bracket of a GEMM output re-quantised to FP8 with `out_scale`.

    Returns fp64 arrays ``lo``, ``hi`` (an output code q is acceptable iff
    lo <= dec(q) <= hi), and the brackets ``amax`` = (lo, hi) of the amax of the
    unscaled results and ``sat`` = (lo, hi) of the saturation count.  The fp32
    values nearest to C64 -+ bound stand in for the extreme fp32 results (at
    most one fp32 ulp outside the bound, which only widens the bracket)."""
    c64 = np.asarray(c64, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    f = codec._fmt(fmt)
    lo32 = (c64 - bound).astype(np.float32)
    hi32 = (c64 + bound).astype(np.float32)
    q_lo, _, _ = scaling.quantize(lo32, out_scale, f)
    q_hi, _, _ = scaling.quantize(hi32, out_scale, f)
    mag_lo = np.maximum(np.abs(c64) - bound, 0.0)
    mag_hi = np.abs(c64) + bound
    sat_lo = scaling.saturation_count(scaling._scaled(mag_lo.astype(np.float32), out_scale), f)
    sat_hi = scaling.saturation_count(scaling._scaled(mag_hi.astype(np.float32), out_scale), f)
    return {"lo": codec.decode(q_lo, f), "hi": codec.decode(q_hi, f),
            "amax": (float(mag_lo.max(initial=0.0)), float(mag_hi.max(initial=0.0))), "sat": (sat_lo, sat_hi)}


def _blocks(K: int, kb: int = 128):
    return [(s, min(K, s + kb)) for s in range(0, K, kb)]


def grouped_gemm(qa, sinv_a, qb, sinv_b, m_offsets, fa="e4m3", fb="e4m3", block=128,
                 rows=None) -> np.ndarray:
    """Fine-grained grouped GEMM in fp64.

    qa [Mtot x K] codes with sinv_a [Mtot x ceil(K/128)] (one per 1x128 K tile);
    qb [G x N x K] codes with sinv_b [G x ceil(N/128) x ceil(K/128)] (one per
    128x128 block); m_offsets [G+1] row offsets of each expert's tokens.
    ``rows`` (optional) restricts the output to those global row indices.
    """
    G, N, K = qb.shape
    offs = np.asarray(m_offsets, dtype=np.int64)
    row_ids = np.arange(offs[-1]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((row_ids.size, N), dtype=np.float64)
    group_of = np.searchsorted(offs, row_ids, side="right") - 1
    nblk = np.arange(N) // block
    for g in range(G):
        sel = np.flatnonzero(group_of == g)
        if sel.size == 0:
            continue
        r = row_ids[sel]
        A = _dec(qa[r], fa)
        B = _dec(qb[g], fb)
        acc = np.zeros((sel.size, N), dtype=np.float64)
        for j, (k0, k1) in enumerate(_blocks(K, block)):
            part = A[:, k0:k1] @ B[:, k0:k1].T
            sa = sinv_a[r, j].astype(np.float64)[:, None]
            sb = sinv_b[g][nblk, j].astype(np.float64)[None, :]
            acc += part * sa * sb
        out[sel] = acc
    return out


def grouped_abs_bound(qa, sinv_a, qb, sinv_b, m_offsets, fa="e4m3", fb="e4m3", block=128,
                      rows=None, rel: float = 1e-5) -> np.ndarray:
    """1e-5 times the grouped sum with every term replaced by its magnitude."""
    G, N, K = qb.shape
    offs = np.asarray(m_offsets, dtype=np.int64)
    row_ids = np.arange(offs[-1]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((row_ids.size, N), dtype=np.float64)
    group_of = np.searchsorted(offs, row_ids, side="right") - 1
    nblk = np.arange(N) // block
    for g in range(G):
        sel = np.flatnonzero(group_of == g)
        if sel.size == 0:
            continue
        r = row_ids[sel]
        A = np.abs(_dec(qa[r], fa))
        B = np.abs(_dec(qb[g], fb))
        acc = np.zeros((sel.size, N), dtype=np.float64)
        for j, (k0, k1) in enumerate(_blocks(K, block)):
            acc += (A[:, k0:k1] @ B[:, k0:k1].T) * np.abs(sinv_a[r, j].astype(np.float64))[:, None] \
                * np.abs(sinv_b[g][nblk, j].astype(np.float64))[None, :]
        out[sel] = acc
    return rel * out

"""FP8 gradient all-reduce with automatic scaling: the parts one GPU runs
(test infrastructure; CPU oracle).

What the pages fix
------------------
* "FP8 and low-precision formats" (use cases): E5M2 for gradient
  communication in distributed training, to cut inter-node bandwidth.
* "#fp8" tag page, discussion of FP8 LLM training: "automatic scaling" adjusts
  the tensor scaling factors dynamically so that gradient values stay inside
  FP8's representable range during the all-reduce, against underflow and
  overflow.
* "4.2 Hopper I — Transformer Engine·FP8", §4.2.4: scale = FP8_MAX / amax,
  scaled saturating cast, x(1/scale) restore, high-precision accumulation.

Readings where the pages are silent (each listed in the design notes):
* Every rank casts its gradient with ONE shared scale, s = fp32(MAX / m),
  where m is the largest amax over the ranks (a MAX all-reduce of one float
  per rank), by the rule of the delayed-scaling update; when m is 0, Inf or
  NaN (or the quotient is not finite) the scale is 1.
* The payload that travels is the E5M2 (or E4M3) codes.  The receiving rank
  sums the R payloads of its chunk in fp32, in rank order (r = 0, 1, ...),
  then restores with x(1/s): out = fp32(fp32(sum_r dec(q_r)) * sinv).  The
  sum, not the mean: averaging is a further factor 1/R the caller may fold
  into the next step.

Parity status: pinned (tests/test_oracle_allreduce.py): hand-computed shared
scales, exactly representable gradients whose sum is exact, identical ranks
(sum = R x one rank for R a power of two), and the rank-order fp32 rounding
of a sum whose order matters.
"""

from __future__ import annotations

import numpy as np

from . import codec, scaling

__all__ = ["shared_scale", "dequant_sum", "fp8_allreduce"]


def shared_scale(amaxes, fmt):
    """(scale, scale_inv) shared by every rank: the scale rule applied to the
    largest of the ranks' amax values (bit-pattern maximum, so NaN wins)."""
    f = codec._fmt(fmt)
    m = scaling.amax(np.asarray(amaxes, dtype=np.float32))
    ok, s, si = scaling.scale_from_amax(m, f.max_value)
    return (s, si) if ok else (np.float32(1.0), np.float32(1.0))


def dequant_sum(payloads, fmt, scale_inv) -> np.ndarray:
    """payloads: R uint8 arrays of one shape.  fp32 sum in rank order of the
    decoded values, then one fp32 multiply by scale_inv."""
    f = codec._fmt(fmt)
    acc = codec.decode(payloads[0], f).astype(np.float32)
    for q in payloads[1:]:
        acc = (acc + codec.decode(q, f).astype(np.float32)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return (acc * np.float32(scale_inv)).astype(np.float32)


def fp8_allreduce(grads32, fmt="e5m2") -> dict:
    """The whole exchange for R ranks' fp32 gradients of one shape: amax per
    rank, the shared scale, the cast of every rank, and the restored sum."""
    f = codec._fmt(fmt)
    amaxes = [scaling.amax(g) for g in grads32]
    s, si = shared_scale(amaxes, f)
    payloads = [scaling.quantize(g, s, f)[0] for g in grads32]
    return {"amaxes": amaxes, "scale": s, "scale_inv": si, "payloads": payloads,
            "sum": dequant_sum(payloads, f, si)}

"""Seeded synthetic workloads for the per-tensor-scaled FP8 GEMM path.

Every generator here draws from numpy's PCG64 (``numpy.random.default_rng``)
with a fixed seed, so the host oracle and the GPU path see byte-identical
inputs.  Floating-point inputs come back either as ``float32`` arrays or as
bfloat16 bit patterns held in ``uint16`` arrays (bf16 is the storage type of the
activation/weight/gradient tensors; the draw is made in fp32 and rounded to
bf16 with round-to-nearest-even, which is how a bf16 tensor is normally
produced).  Widening bf16 bits to fp32 is exact; each consumer does it itself.

The shapes and distributions follow the transformer layer used on the page
"4.2 Hopper I — Transformer Engine·FP8" (§4.2.6: hidden 4096, ffn 16384,
32 heads) and its remarks that activations change from layer to layer and
step to step (§4.2.2) and can spike (§4.2.9), that gradients mix very large
and very small magnitudes (§4.2.3), and, for the grouped case, the DeepGEMM
entry of the "#fp8" tag page (MoE grouped GEMM).  Sizes are parameters so
that tests can draw the same recipe at small shapes.
"""

from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "HostTensor",
    "bf16_bits_from_f32",
    "tiny_operands",
    "fc1_forward",
    "dgrad_hybrid",
    "stream_step",
    "stream_sigma",
    "moe_token_counts",
    "moe_grouped",
    "adversarial_f32",
]


@dataclass
class HostTensor:
    """A 2-D (or 3-D) host array plus its storage dtype tag ("f32" or "bf16").

    For "bf16" the array is ``uint16`` holding bfloat16 bit patterns; for
    "f32" it is ``float32``.  ``recipe`` records how it was drawn.
    """

    data: np.ndarray
    dtype: str
    recipe: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.data.shape


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaNs stay NaN, infinities stay infinite.  Large arrays go through PyTorch's
    CPU conversion (the same rounding, multi-threaded); small ones through the
    integer formula below.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.size < (1 << 20):
        return _bf16_bits_small(a)
    import torch
    out = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(a)
    if nan.any():                      # keep the NaN sign and payload rule of the formula
        out = out.copy()
        out[nan] = _bf16_bits_small(a[nan])
    return out


def _bf16_bits_small(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)).astype(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def _as(a32: np.ndarray, dtype: str, recipe: str, **extra) -> HostTensor:
    if dtype == "f32":
        return HostTensor(np.ascontiguousarray(a32, dtype=np.float32), "f32", recipe, extra)
    if dtype == "bf16":
        return HostTensor(bf16_bits_from_f32(a32), "bf16", recipe, extra)
    raise ValueError(f"unknown dtype {dtype!r}")


def _parallel(fn, args_list):
    """Run independent seeded draws on a few threads (numpy releases the GIL);
    results come back in argument order, so the output does not depend on timing."""
    with _cf.ThreadPoolExecutor(max_workers=min(4, len(args_list)) or 1) as ex:
        return list(ex.map(lambda a: fn(*a), args_list))


def _normal(shape, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


# ---------------------------------------------------------------------------
# Tiny case: fp32 64x128 by 128x64, N(0, 0.02), history pre-filled by 4 draws.
# ---------------------------------------------------------------------------
TINY_SEEDS = {"A": 11, "B": 12, "A_priors": (101, 102, 103, 104), "B_priors": (201, 202, 203, 204)}


def tiny_operands(m: int = 64, k: int = 128, n: int = 64) -> dict:
    """A [m x k] and B [k x n], fp32 ~N(0, 0.02), plus 4 prior draws per operand."""
    s = TINY_SEEDS
    out = {
        "A": _as(_normal((m, k), 0.02, s["A"]), "f32", "N(0,0.02) seed 11"),
        "B": _as(_normal((k, n), 0.02, s["B"]), "f32", "N(0,0.02) seed 12"),
        "A_priors": [_as(_normal((m, k), 0.02, sd), "f32", f"N(0,0.02) seed {sd}") for sd in s["A_priors"]],
        "B_priors": [_as(_normal((k, n), 0.02, sd), "f32", f"N(0,0.02) seed {sd}") for sd in s["B_priors"]],
    }
    return out


# ---------------------------------------------------------------------------
# FC1 forward: X bf16 [tokens x hidden] N(0,1) with 0.1 % outliers x100,
#              W bf16 [hidden x ffn] N(0, 0.02).
# ---------------------------------------------------------------------------
FC1_SEEDS = {"X": 21, "X_outliers": 22, "W": 23,
             "X_priors": (2101, 2102, 2103, 2104), "X_prior_outliers": (2151, 2152, 2153, 2154),
             "W_priors": (2301, 2302, 2303, 2304)}


def _normal_with_outliers(shape, value_seed: int, pos_seed: int, frac=0.001, factor=100.0) -> np.ndarray:
    x = _normal(shape, 1.0, value_seed)
    n = x.size
    count = int(round(frac * n))
    if count:
        pos = np.random.default_rng(pos_seed).choice(n, size=count, replace=False)
        flat = x.reshape(-1)
        flat[pos] *= np.float32(factor)
    return x


def fc1_forward(tokens: int = 8192, hidden: int = 4096, ffn: int = 16384, priors: bool = True) -> dict:
    """Forward FC1 operands: X [tokens x hidden] and W [hidden x ffn], both bf16."""
    s = FC1_SEEDS
    X = _as(_normal_with_outliers((tokens, hidden), s["X"], s["X_outliers"]), "bf16",
            "N(0,1), round(0.001*numel) uniform positions x100, seeds 21/22")
    W = _as(_normal((hidden, ffn), 0.02, s["W"]), "bf16", "N(0,0.02) seed 23")
    out = {"X": X, "W": W, "X_priors": [], "W_priors": []}
    if priors:
        out["X_priors"] = _parallel(
            lambda vs, ps: _as(_normal_with_outliers((tokens, hidden), vs, ps), "bf16", f"X prior seeds {vs}/{ps}"),
            list(zip(s["X_priors"], s["X_prior_outliers"])))
        out["W_priors"] = _parallel(lambda sd: _as(_normal((hidden, ffn), 0.02, sd), "bf16", f"W prior seed {sd}"),
                                    [(sd,) for sd in s["W_priors"]])
    return out


# ---------------------------------------------------------------------------
# dgrad (HYBRID): dY bf16 [tokens x ffn], |dY| = 10**U(-6, 2), random sign;
#                 W bf16 [ffn x hidden] N(0, 0.02).
# ---------------------------------------------------------------------------
DGRAD_SEEDS = {"dY_mag": 31, "dY_sign": 32, "W": 33,
               "dY_priors": (3101, 3102, 3103, 3104), "W_priors": (3301, 3302, 3303, 3304)}


def _loguniform_signed(shape, mag_seed: int, sign_seed: int, lo_exp=-6.0, hi_exp=2.0) -> np.ndarray:
    u = np.random.default_rng(mag_seed).random(size=shape, dtype=np.float32)
    u *= np.float32(hi_exp - lo_exp)
    u += np.float32(lo_exp)
    mag = np.power(np.float32(10.0), u)
    neg = np.random.default_rng(sign_seed).integers(0, 2, size=shape, dtype=np.int8)
    bits = mag.view(np.uint32)
    np.bitwise_or(bits, neg.astype(np.uint32) << np.uint32(31), out=bits)   # sign bit set with p = 1/2
    return mag


def dgrad_hybrid(tokens: int = 8192, ffn: int = 16384, hidden: int = 4096, priors: bool = True) -> dict:
    """dgrad operands: dY [tokens x ffn] (log-uniform magnitudes) and W [ffn x hidden]."""
    s = DGRAD_SEEDS
    dY = _as(_loguniform_signed((tokens, ffn), s["dY_mag"], s["dY_sign"]), "bf16",
             "|dY| = 10**U(-6,2), sign p=1/2, seeds 31/32")
    W = _as(_normal((ffn, hidden), 0.02, s["W"]), "bf16", "N(0,0.02) seed 33")
    out = {"dY": dY, "W": W, "dY_priors": [], "W_priors": []}
    if priors:
        out["dY_priors"] = _parallel(
            lambda sd: _as(_loguniform_signed((tokens, ffn), sd, sd + 100), "bf16", f"dY prior {sd}/{sd + 100}"),
            [(sd,) for sd in s["dY_priors"]])
        out["W_priors"] = _parallel(lambda sd: _as(_normal((ffn, hidden), 0.02, sd), "bf16", f"W prior seed {sd}"),
                                    [(sd,) for sd in s["W_priors"]])
    return out


# ---------------------------------------------------------------------------
# Delayed-scaling stream: 32 steps of [8192 x 4096] ~N(0, sigma_t).
# ---------------------------------------------------------------------------
STREAM_STEPS = 32
STREAM_SPIKE_STEP = 20


def stream_sigma(t: int) -> float:
    """sigma_t = 1.05**t, times 50 at the single spike step 20."""
    s = 1.05 ** t
    if t == STREAM_SPIKE_STEP:
        s *= 50.0
    return s


def stream_step(t: int, rows: int = 8192, cols: int = 4096, dtype: str = "f32") -> HostTensor:
    """Step t's activation tensor, N(0, sigma_t), seed 4000 + t."""
    return _as(_normal((rows, cols), stream_sigma(t), 4000 + t), dtype, f"N(0,{stream_sigma(t):.6g}) seed {4000 + t}")


# ---------------------------------------------------------------------------
# MoE grouped GEMM: 8 experts, token counts multiples of 128 in [128, 4096]
# summing to 16384; A bf16 [16384 x 7168] N(0,1); W_g stored [N x K] N(0,0.02).
# ---------------------------------------------------------------------------
MOE_SEEDS = {"counts": 51, "A": 52, "W_base": 53}


def moe_token_counts(experts: int = 8, total: int = 16384, unit: int = 128, cap: int = 4096,
                     seed: int = MOE_SEEDS["counts"]) -> np.ndarray:
    """Seeded token counts: each expert starts at one unit; the remaining units are
    dealt by an equal-probability multinomial, redrawn until no expert exceeds cap."""
    units_total = total // unit
    assert units_total * unit == total and units_total >= experts
    rng = np.random.default_rng(seed)
    cap_units = cap // unit
    while True:
        extra = rng.multinomial(units_total - experts, [1.0 / experts] * experts)
        counts = 1 + extra
        if counts.max() <= cap_units:
            return (counts * unit).astype(np.int64)


def moe_grouped(experts: int = 8, total: int = 16384, k: int = 7168, n: int = 4096,
                unit: int = 128, cap: int = 4096) -> dict:
    """Grouped operands: A [total x k] bf16 N(0,1); B [experts x n x k] bf16 N(0,0.02)
    (each expert's weight stored output-major, K contiguous); m_offsets [experts+1]."""
    counts = moe_token_counts(experts, total, unit, cap)
    offs = np.zeros(experts + 1, dtype=np.int64)
    offs[1:] = np.cumsum(counts)
    A = _as(_normal((total, k), 1.0, MOE_SEEDS["A"]), "bf16", "N(0,1) seed 52")
    Bs = np.empty((experts, n, k), dtype=np.uint16)
    for g in range(experts):
        Bs[g] = bf16_bits_from_f32(_normal((n, k), 0.02, MOE_SEEDS["W_base"] + g))
    B = HostTensor(Bs, "bf16", "expert g: N(0,0.02) seed 53+g")
    return {"A": A, "B": B, "counts": counts, "m_offsets": offs}


# ---------------------------------------------------------------------------
# Adversarial fp32 values for the cast: boundaries, ties, specials.
# ---------------------------------------------------------------------------
def adversarial_f32(seed: int = 7, random_count: int = 4096) -> np.ndarray:
    """A flat fp32 array mixing specials (+-0, +-Inf, NaNs, fp32 subnormals), every
    value near each E4M3/E5M2 code (the code's value, the midpoints to its
    neighbours, and one fp32 ulp either side of those), and random bit patterns."""
    vals = [0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1e-40, -3e-39, 1.0, -1.0,
            448.0, 464.0, 480.0, 57344.0, 61440.0, 65536.0, 1e30, -1e30, 3.4e38]
    pts = []
    for e, m_ in ((4, 3), (5, 2)):
        bias = (1 << (e - 1)) - 1
        for ex in range(1 - bias - m_ - 2, (1 << e) - bias + 1):
            for mant in range(1 << (m_ + 1)):
                pts.append(mant * 2.0 ** (ex - m_) if ex >= 1 - bias else mant * 2.0 ** (1 - bias - m_))
                pts.append((mant + 0.5) * 2.0 ** (ex - m_))
    p = np.unique(np.asarray(pts, dtype=np.float64))
    p = p[np.isfinite(p) & (p < 3e38)].astype(np.float32)
    up = np.nextafter(p, np.float32(np.inf))
    dn = np.nextafter(p, np.float32(0))
    base = np.concatenate([p, up, dn]).astype(np.float32)
    base = np.concatenate([base, -base, np.asarray(vals, dtype=np.float32)])
    rng = np.random.default_rng(seed)
    rbits = rng.integers(0, 2 ** 32, size=random_count, dtype=np.uint64).astype(np.uint32)
    nanbits = np.asarray([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32)
    return np.concatenate([base, rbits.view(np.float32), nanbits.view(np.float32)])

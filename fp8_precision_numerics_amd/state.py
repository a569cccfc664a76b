"""Device buffers of one tensor's delayed-scaling state, and the recipe.

"4.2 Hopper I — Transformer Engine·FP8", §4.2.6: a recipe names the FP8
format (HYBRID = E4M3 forward, E5M2 backward), the amax history length (16)
and the rule applied to the history ("max"); each FP8 tensor keeps its own
amax history and scale (§4.2.4).  This module only allocates and groups the
buffers (PyTorch is used for device memory); the cast and the history update
run in libfp8mi's kernels.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _binding as _b


@dataclass(frozen=True)
class Recipe:
    """Delayed-scaling recipe: forward / backward formats, history length, rule."""

    fmt_fwd: str = "e4m3"
    fmt_bwd: str = "e5m2"
    history_len: int = 16
    algo: str = "max"

    def __post_init__(self):
        if self.algo != "max":
            raise ValueError("only the 'max' amax rule is implemented")
        if not 1 <= self.history_len <= 4096:
            raise ValueError("history_len must be in [1, 4096]")


class DelayedScalingState:
    """history[L] (zeros), head (0), scale (1), scale_inv (1), status (0) and the
    last amax, all on one GPU.  ``quantize`` casts with the current scale and
    records amax; ``update`` pushes that amax and refreshes the scale for the
    next cast."""

    def __init__(self, fmt: str = "e4m3", history_len: int = 16, device="cuda"):
        self.fmt = fmt
        dev = torch.device(device)
        self.history = torch.zeros(history_len, dtype=torch.float32, device=dev)
        self.head = torch.zeros(1, dtype=torch.int32, device=dev)
        self.scale = torch.ones(1, dtype=torch.float32, device=dev)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.amax = torch.zeros(1, dtype=torch.float32, device=dev)
        # inverse of the scale the last quantize_update cast with (the GEMM's factor for those codes)
        self.scale_inv_used = torch.ones(1, dtype=torch.float32, device=dev)
        self.sat = torch.zeros(1, dtype=torch.int64, device=dev)
        # scratch for the per-workgroup partials of amax and the count
        self.workspace = torch.empty(_b.QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)

    def quantize(self, x, q=None, q_t=None, count_saturation=False, stream=None):
        _b.fp8_quantize(x, self.fmt, self.scale, q=q, q_t=q_t, amax=self.amax,
                        sat=self.sat if count_saturation else None, workspace=self.workspace, stream=stream)

    def quantize_update(self, x, q=None, q_t=None, count_saturation=False, stream=None):
        """quantize then update in one library call (the history step rides on the
        launch that reduces the cast's partial amaxes).  Afterwards scale_inv
        belongs to the next step; a GEMM on these codes takes scale_inv_used."""
        _b.fp8_quantize_update(x, self.fmt, self.history, self.head, self.scale, self.scale_inv, self.amax, q=q,
                               q_t=q_t, sat=self.sat if count_saturation else None, status=self.status,
                               workspace=self.workspace, scale_inv_used=self.scale_inv_used, stream=stream)

    def update(self, stream=None):
        _b.fp8_amax_update(self.history, self.head, self.amax, self.fmt, self.scale, self.scale_inv,
                           self.status, stream=stream)

    def snapshot(self) -> dict:
        """Host copies of every buffer (synchronises)."""
        return {k: getattr(self, k).detach().cpu().clone()
                for k in ("history", "head", "scale", "scale_inv", "status", "amax", "sat")}

    def restore(self, snap: dict) -> None:
        for k, v in snap.items():
            getattr(self, k).copy_(v)

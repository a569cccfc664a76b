"""One FP8 linear layer (Y = X W^T) under the HYBRID delayed-scaling recipe:
forward, data gradient and weight gradient, each GEMM on FP8 operands.

"4.2 Hopper I — Transformer Engine·FP8", §4.2.3 and §4.2.6: forward operands
are cast to E4M3, gradients to E5M2 (HYBRID); §4.2.4: each tensor is cast with
its own delayed scale and the GEMM result is restored by x(1/scale) of both
operands; §4.2.6: the amax histories and scales are refreshed after the step.

The class only sequences libfp8mi's kernels and owns the buffers (PyTorch
provides the device memory):

* forward: one cast pass of X gives X_q (forward GEMM) and X_q^T (weight
  gradient); one pass of W gives W_q (forward) and W_q^T (data gradient);
  Y = fp8_gemm(X_q, W_q).
* backward: one cast pass of dY (E5M2) gives dY_q and dY_q^T;
  dX = fp8_gemm(dY_q, W_q^T), dW = fp8_gemm(dY_q^T, X_q^T).
* forward_requant: the forward with Y re-quantised to FP8 in the GEMM's
  epilogue with the scale of Y's own delayed-scaling state (§4.2.4: the
  restore "combined with the next stage's scale"), recording Y's amax there.
* update: each state pushes the amax its cast recorded and sets the scale
  for the next step.
"""

from __future__ import annotations

import torch

from . import _binding as _b
from .state import DelayedScalingState, Recipe


class Fp8Linear:
    """Buffers and delayed-scaling states of one linear layer with
    X [tokens x in], W [out x in], dY [tokens x out]."""

    def __init__(self, tokens: int, in_features: int, out_features: int, recipe: Recipe = Recipe(),
                 accum: str = "exact", device="cuda"):
        if recipe.fmt_fwd != "e4m3" or recipe.fmt_bwd != "e5m2":
            raise ValueError("Fp8Linear implements the HYBRID recipe (E4M3 forward, E5M2 backward)")
        dev = torch.device(device)
        self.accum = accum
        self.shape = (tokens, in_features, out_features)
        self.state_x = DelayedScalingState(recipe.fmt_fwd, recipe.history_len, device=dev)
        self.state_w = DelayedScalingState(recipe.fmt_fwd, recipe.history_len, device=dev)
        self.state_g = DelayedScalingState(recipe.fmt_bwd, recipe.history_len, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.qx = torch.empty((tokens, in_features), **u8)
        self.qx_t = torch.empty((in_features, tokens), **u8)
        self.qw = torch.empty((out_features, in_features), **u8)
        self.qw_t = torch.empty((in_features, out_features), **u8)
        self.qg = torch.empty((tokens, out_features), **u8)
        self.qg_t = torch.empty((out_features, tokens), **u8)

    def _check(self, t, rows, cols, name):
        if tuple(t.shape) != (rows, cols):
            raise ValueError(f"{name} must be {rows}x{cols}, got {tuple(t.shape)}")

    def forward(self, x, w, y, stream=None):
        """Cast X and W (both orientations) with the current scales, then
        y = X W^T (y fp32 or bf16 [tokens x out])."""
        T, I, O = self.shape
        self._check(x, T, I, "X")
        self._check(w, O, I, "W")
        self._check(y, T, O, "Y")
        self.state_x.quantize(x, q=self.qx, q_t=self.qx_t, stream=stream)
        self.state_w.quantize(w, q=self.qw, q_t=self.qw_t, stream=stream)
        _b.fp8_gemm(self.qx, "e4m3", self.qw, "e4m3", self.state_x.scale_inv, self.state_w.scale_inv, y,
                    accum=self.accum, stream=stream)

    def forward_requant(self, x, w, yq, state_y: DelayedScalingState, stream=None):
        """As forward, but Y leaves the GEMM as FP8 codes yq [tokens x out] in
        state_y's format, cast with state_y's current scale; Y's amax and
        saturation count go to state_y (state_y.update() then records them)."""
        T, I, O = self.shape
        self._check(x, T, I, "X")
        self._check(w, O, I, "W")
        self._check(yq, T, O, "Yq")
        self.state_x.quantize(x, q=self.qx, q_t=self.qx_t, stream=stream)
        self.state_w.quantize(w, q=self.qw, q_t=self.qw_t, stream=stream)
        _b.fp8_gemm_requant(self.qx, "e4m3", self.qw, "e4m3", self.state_x.scale_inv, self.state_w.scale_inv,
                            state_y.fmt, state_y.scale, yq, amax=state_y.amax, sat=state_y.sat,
                            accum=self.accum, stream=stream)

    def backward(self, dy, dx, dw, stream=None):
        """Cast dY (E5M2, both orientations), then dx = dY W and dw = dY^T X from
        the forward casts of W and X (dx [tokens x in], dw [out x in])."""
        T, I, O = self.shape
        self._check(dy, T, O, "dY")
        self._check(dx, T, I, "dX")
        self._check(dw, O, I, "dW")
        self.state_g.quantize(dy, q=self.qg, q_t=self.qg_t, stream=stream)
        _b.fp8_gemm(self.qg, "e5m2", self.qw_t, "e4m3", self.state_g.scale_inv, self.state_w.scale_inv, dx,
                    accum=self.accum, stream=stream)
        _b.fp8_gemm(self.qg_t, "e5m2", self.qx_t, "e4m3", self.state_g.scale_inv, self.state_x.scale_inv, dw,
                    accum=self.accum, stream=stream)

    def update(self, stream=None):
        """Push each cast's amax into its history and set the next step's scales."""
        for st in (self.state_x, self.state_w, self.state_g):
            st.update(stream=stream)

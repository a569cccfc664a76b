"""One FP8 linear layer step (forward, data gradient, weight gradient) under the
HYBRID recipe with delayed scaling (test infrastructure; CPU oracle).

What the pages fix ("4.2 Hopper I — Transformer Engine·FP8")
-------------------------------------------------------------
* §4.2.3 / §4.2.6: HYBRID casts forward operands to E4M3 and the backward
  (gradient) operands to E5M2; inside the autocast region the linear layer's
  GEMMs run in FP8 and the backward pass follows the E5M2 path.
* §4.2.4: each FP8 tensor is cast with its own scale, the GEMM accumulates in
  FP32 and the result is restored by x(1/scale) of both operands; with delayed
  scaling the scale of this step comes from the amax history of past steps.
* §4.2.6: after the step the library updates each tensor's amax history and
  with it the scale used by the next step.

Readings where the pages are silent (each listed in the design notes):
* The layer is Y = X W^T with X [tokens x in] and W [out x in] (the usual
  linear-layer weight layout); its gradients are dX = dY W and
  dW = dY^T X, the plain calculus of that product.
* The backward GEMMs reuse the FP8 codes and inverse scales of the forward
  casts of X and W (one cast per tensor per step); dY is cast once, to E5M2,
  with its own delayed-scaling state.
* After the step each state records the amax seen by its cast and refreshes
  its scale for the next step, in the order X, W, dY (the states are
  independent, so the order does not change any value).

Parity status: pinned (tests/test_oracle_linear.py): with unit scales and
inputs that each format holds exactly, all three products equal the fp64
matrix products of the inputs themselves, which fixes every orientation and
the format given to each operand; the scales of a second step are the
closed-form 448/amax and 57344/amax values.
"""

from __future__ import annotations

from . import gemm, scaling

__all__ = ["hybrid_linear_step"]


def hybrid_linear_step(x32, w32, dy32, sx: scaling.DelayedScaling, sw: scaling.DelayedScaling,
                       sg: scaling.DelayedScaling) -> dict:
    """One step of an FP8 linear layer.

    x32 [T x I], w32 [O x I], dy32 [T x O] are fp32 (bf16 inputs widened
    exactly beforehand); sx, sw (E4M3) and sg (E5M2) are the tensors' delayed
    scaling states, updated in place after the step.  Returns the codes of the
    three casts, the inverse scales used, and the fp64 products
    Y [T x O], dX [T x I], dW [O x I].
    """
    assert sx.fmt.name == "e4m3" and sw.fmt.name == "e4m3" and sg.fmt.name == "e5m2"
    # the casts of this step use the scales the states hold now
    qx, amax_x, _ = scaling.quantize(x32, sx.scale, "e4m3")
    qw, amax_w, _ = scaling.quantize(w32, sw.scale, "e4m3")
    qg, amax_g, _ = scaling.quantize(dy32, sg.scale, "e5m2")
    six, siw, sig = sx.scale_inv, sw.scale_inv, sg.scale_inv
    # forward: Y[t,o] = sum_i X[t,i] W[o,i]
    y = gemm.dequant_gemm(qx, "e4m3", qw.T, "e4m3", six, siw)
    # data gradient: dX[t,i] = sum_o dY[t,o] W[o,i]
    dx = gemm.dequant_gemm(qg, "e5m2", qw, "e4m3", sig, siw)
    # weight gradient: dW[o,i] = sum_t dY[t,o] X[t,i]
    dw = gemm.dequant_gemm(qg.T, "e5m2", qx, "e4m3", sig, six)
    bounds = {
        "y": gemm.abs_bound(qx, "e4m3", qw.T, "e4m3", six, siw),
        "dx": gemm.abs_bound(qg, "e5m2", qw, "e4m3", sig, siw),
        "dw": gemm.abs_bound(qg.T, "e5m2", qx, "e4m3", sig, six),
    }
    sx.update(amax_x)
    sw.update(amax_w)
    sg.update(amax_g)
    return {"qx": qx, "qw": qw, "qg": qg, "scale_inv": (six, siw, sig),
            "amax": (amax_x, amax_w, amax_g), "y": y, "dx": dx, "dw": dw, "bounds": bounds}

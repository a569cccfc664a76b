"""GPU parity: one FP8 linear layer step (forward, data gradient, weight gradient)
under the HYBRID recipe against the oracle's step, and the weight-gradient
GEMM at the FC1 training shape on sampled outputs."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, mfma8_bound, to_device, u8
from oracle import codec, gemm, linear, scaling
from synth import dgrad_hybrid, fc1_forward

pytestmark = pytest.mark.gpu


def _check(got, want, bound):
    err = np.abs(got.astype(np.float64) - want)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])


def _state_equal(st, ref):
    snap = st.snapshot()
    assert np.array_equal(snap["history"].numpy().view(np.uint32), ref.history.view(np.uint32))
    assert int(snap["head"][0]) == ref.head
    assert snap["scale"].numpy().view(np.uint32)[0] == np.float32(ref.scale).view(np.uint32)
    assert snap["scale_inv"].numpy().view(np.uint32)[0] == np.float32(ref.scale_inv).view(np.uint32)


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
@pytest.mark.parametrize("T,I,O", [(208, 272, 144), (256, 128, 384)])
def test_linear_step_matches_oracle(T, I, O, accum):
    """Three steps with fresh states: every cast (both orientations) bit for bit,
    the states after each update bit for bit, and Y, dX, dW within the method's
    bound (exact mode) or the matrix-core error model (mfma_fp8 mode)."""
    dev = device()
    rng = np.random.default_rng(T + I + O)
    layer = fm.Fp8Linear(T, I, O, accum=accum, device=dev)
    refs = (scaling.DelayedScaling("e4m3"), scaling.DelayedScaling("e4m3"), scaling.DelayedScaling("e5m2"))
    y = torch.empty((T, O), dtype=torch.float32, device=dev)
    dx = torch.empty((T, I), dtype=torch.float32, device=dev)
    dw = torch.empty((O, I), dtype=torch.float32, device=dev)
    for step in range(3):
        # magnitudes drift between steps so each step's scales differ
        x = (rng.standard_normal((T, I)) * 0.5 * (1 + step)).astype(np.float32)
        w = (rng.standard_normal((O, I)) * 0.02).astype(np.float32)
        dy = (rng.standard_normal((T, O)) * 1e-3 * 10.0 ** rng.uniform(-2, 1, (T, 1))).astype(np.float32)
        announce(f"linear step {step} T={T} I={I} O={O} {accum}")
        layer.forward(to_device((x, "f32"), dev), to_device((w, "f32"), dev), y)
        layer.backward(to_device((dy, "f32"), dev), dx, dw)
        layer.update()
        torch.cuda.synchronize()
        r = linear.hybrid_linear_step(x, w, dy, *refs)
        assert np.array_equal(u8(layer.qx), r["qx"]) and np.array_equal(u8(layer.qx_t), r["qx"].T)
        assert np.array_equal(u8(layer.qw), r["qw"]) and np.array_equal(u8(layer.qw_t), r["qw"].T)
        assert np.array_equal(u8(layer.qg), r["qg"]) and np.array_equal(u8(layer.qg_t), r["qg"].T)
        for st, ref in zip((layer.state_x, layer.state_w, layer.state_g), refs):
            _state_equal(st, ref)
        six, siw, sig = r["scale_inv"]
        if accum == "exact":
            bounds = r["bounds"]
        else:
            bounds = {"y": mfma8_bound(r["qx"], "e4m3", r["qw"], "e4m3", six, siw),
                      "dx": mfma8_bound(r["qg"], "e5m2", r["qw"].T, "e4m3", sig, siw),
                      "dw": mfma8_bound(r["qg"].T, "e5m2", r["qx"].T, "e4m3", sig, six)}
        _check(f32(y), r["y"], bounds["y"])
        _check(f32(dx), r["dx"], bounds["dx"])
        _check(f32(dw), r["dw"], bounds["dw"])


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_forward_requant_within_bracket(accum):
    """The forward with Y re-quantised to E4M3 in the epilogue, with Y's own
    delayed-scaling state over three steps: codes and the recorded amax within
    the oracle's bracket of the step's exact product; Y's scale leaves 1 once
    its first amax is recorded."""
    dev = device()
    T, I, O = 208, 272, 144
    rng = np.random.default_rng(77)
    layer = fm.Fp8Linear(T, I, O, accum=accum, device=dev)
    st_y = fm.DelayedScalingState("e4m3", 16, device=dev)
    refs = (scaling.DelayedScaling("e4m3"), scaling.DelayedScaling("e4m3"), scaling.DelayedScaling("e5m2"))
    yq = torch.empty((T, O), dtype=torch.uint8, device=dev)
    dy = np.zeros((T, O), dtype=np.float32)
    for step in range(3):
        x = (rng.standard_normal((T, I)) * (1 + step)).astype(np.float32)
        w = (rng.standard_normal((O, I)) * 0.02).astype(np.float32)
        announce(f"forward requant step {step} {accum}")
        s_y = st_y.scale.item()
        layer.forward_requant(to_device((x, "f32"), dev), to_device((w, "f32"), dev), yq, st_y)
        torch.cuda.synchronize()
        amax_y = st_y.amax.item()
        layer.state_x.update()
        layer.state_w.update()
        st_y.update()
        r = linear.hybrid_linear_step(x, w, dy, *refs)
        assert np.array_equal(u8(layer.qx), r["qx"]) and np.array_equal(u8(layer.qw), r["qw"])
        six, siw, _ = r["scale_inv"]
        bound = r["bounds"]["y"] if accum == "exact" else mfma8_bound(r["qx"], "e4m3", r["qw"], "e4m3", six, siw)
        br = gemm.requant_bracket(r["y"], bound, np.float32(s_y), "e4m3")
        got = codec.decode(u8(yq), "e4m3")
        assert np.all((got >= br["lo"]) & (got <= br["hi"]))
        assert br["amax"][0] <= amax_y <= br["amax"][1]
    # step 0 cast Y with scale 1; later steps with 448 / (max amax so far)
    assert st_y.scale.item() != 1.0


def test_linear_rejects_wrong_shapes():
    dev = device()
    layer = fm.Fp8Linear(64, 128, 32, device=dev)
    with pytest.raises(ValueError):
        layer.forward(torch.zeros((64, 127), device=dev), torch.zeros((32, 128), device=dev),
                      torch.empty((64, 32), device=dev))
    with pytest.raises(ValueError):
        fm.Fp8Linear(64, 128, 32, recipe=fm.Recipe(fmt_fwd="e5m2"), device=dev)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_wgrad_hybrid_full_size(accum):
    """dW = dY^T X at the FC1 training shape: dY bf16 8192x16384 (E5M2,
    cast-transposed) and X bf16 8192x4096 (E4M3, cast-transposed), K = 8192
    tokens -> fp32 16384x4096; sampled outputs against exact dot products,
    within the method's bound (exact mode) or the error model (mfma_fp8)."""
    dev = device()
    dg = dgrad_hybrid(priors=False)
    dfx = fc1_forward(priors=False)
    G, X = to_device(dg["dY"], dev), to_device(dfx["X"], dev)
    del dg, dfx
    stG = fm.DelayedScalingState("e5m2", 16, device=dev)
    stX = fm.DelayedScalingState("e4m3", 16, device=dev)
    qg_t = torch.empty((16384, 8192), dtype=torch.uint8, device=dev)
    qx_t = torch.empty((4096, 8192), dtype=torch.uint8, device=dev)
    announce(f"wgrad full size: cast-transpose + gemm ({accum})")
    for _ in range(2):                     # the second cast uses the amax-derived scales
        stG.quantize(G, q_t=qg_t)
        stG.update()
        stX.quantize(X, q_t=qx_t)
        stX.update()
    c = torch.empty((16384, 4096), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qg_t, "e5m2", qx_t, "e4m3", stG.scale_inv, stX.scale_inv, c, accum=accum)
    torch.cuda.synchronize()
    qa, qbT = u8(qg_t), u8(qx_t)
    sa, sb = stG.scale_inv.item(), stX.scale_inv.item()
    got = f32(c)
    rng = np.random.default_rng(41)
    ms = np.concatenate([rng.integers(0, 16384, 512), [0, 16383]])
    ns = np.concatenate([rng.integers(0, 4096, 512), [4095, 0]])
    for m, n in zip(ms, ns):
        num, sh = gemm.exact_dot(qa[m], "e5m2", qbT[n], "e4m3")
        exact = np.ldexp(float(num), -sh) * sa * sb
        if accum == "exact":
            bound = float(gemm.abs_bound(qa[m:m + 1], "e5m2", qbT[n:n + 1].T, "e4m3", sa, sb)[0, 0])
        else:
            bound = float(mfma8_bound(qa[m:m + 1], "e5m2", qbT[n:n + 1], "e4m3", sa, sb)[0, 0])
        assert abs(float(got[m, n]) - exact) <= bound, (m, n, float(got[m, n]), exact, bound)

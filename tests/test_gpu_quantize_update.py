"""GPU parity: fp8_quantize_update (cast and history step in one call) equals
fp8_quantize followed by fp8_amax_update, bit for bit, with and without a
workspace, and both equal the oracle's delayed-scaling sequence."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, u8
from oracle import scaling
from synth import HostTensor, bf16_bits_from_f32

pytestmark = pytest.mark.gpu

KEYS = ("history", "head", "scale", "scale_inv", "status", "amax", "sat")


def _snap(st):
    return {k: getattr(st, k).detach().cpu().numpy().copy() for k in KEYS}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fused_step_equals_separate_calls_and_oracle(fmt, dtype):
    dev = device()
    rng = np.random.default_rng(5 if fmt == "e4m3" else 6)
    rows, cols = 512, 1024
    fused = fm.DelayedScalingState(fmt, 16, device=dev)
    fused_nows = fm.DelayedScalingState(fmt, 16, device=dev)
    fused_nows.workspace = None                    # the atomics path, then a separate update launch
    sep = fm.DelayedScalingState(fmt, 16, device=dev)
    ref = scaling.DelayedScaling(fmt, 16)
    bufs = {name: (torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                   torch.empty((cols, rows), dtype=torch.uint8, device=dev)) for name in ("f", "n", "s")}
    for step in range(7):
        sigma = 1.05 ** step * (50.0 if step == 3 else 1.0)
        x32 = (rng.standard_normal((rows, cols)) * sigma).astype(np.float32)
        if step == 5:
            x32[7, 9] = np.inf                     # a non-finite amax: the scale is held, status bit 0 set
        h = HostTensor(x32, "f32") if dtype == "f32" else HostTensor(bf16_bits_from_f32(x32), "bf16")
        x = torch.from_numpy(h.data if dtype == "f32" else h.data.view(np.int16)).to(dev)
        if dtype == "bf16":
            x = x.view(torch.bfloat16)
        announce(f"quantize_update step {step} {fmt} {dtype}")
        used = sep.scale_inv.detach().cpu().numpy().copy()      # the inverse scale this step's cast uses
        fused.quantize_update(x, q=bufs["f"][0], q_t=bufs["f"][1], count_saturation=True)
        fused_nows.quantize_update(x, q=bufs["n"][0], q_t=bufs["n"][1], count_saturation=True)
        sep.quantize(x, q=bufs["s"][0], q_t=bufs["s"][1], count_saturation=True)
        sep.update()
        torch.cuda.synchronize()
        xw = scaling.widen(h.data, dtype)
        wq, wamax, wsat = scaling.quantize(xw, ref.scale, fmt)
        ref.update(wamax)
        a, b, c = _snap(fused), _snap(fused_nows), _snap(sep)
        for k in KEYS:
            assert np.array_equal(a[k].view(np.uint8), c[k].view(np.uint8)), (step, k)
            assert np.array_equal(b[k].view(np.uint8), c[k].view(np.uint8)), (step, k)
        for name in ("f", "n"):
            assert torch.equal(bufs[name][0], bufs["s"][0]) and torch.equal(bufs[name][1], bufs["s"][1])
        for st in (fused, fused_nows):
            assert f32(st.scale_inv_used).view(np.uint32)[0] == used.view(np.uint32)[0], step
        assert np.array_equal(u8(bufs["f"][0]), wq)
        assert np.array_equal(a["history"].view(np.uint32), ref.history.view(np.uint32))
        assert int(a["head"][0]) == ref.head and int(a["status"][0]) == ref.status
        assert a["scale"].view(np.uint32)[0] == np.float32(ref.scale).view(np.uint32)
        assert a["scale_inv"].view(np.uint32)[0] == np.float32(ref.scale_inv).view(np.uint32)
        assert int(a["sat"][0]) == wsat


def test_fused_step_on_an_empty_tensor():
    """No elements: amax 0 goes into the history like any other step."""
    dev = device()
    st = fm.DelayedScalingState("e4m3", 4, device=dev)
    x = torch.empty((0, 16), dtype=torch.float32, device=dev)
    st.quantize_update(x, q=torch.empty((0, 16), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    snap = _snap(st)
    assert snap["amax"][0] == 0.0 and int(snap["head"][0]) == 1 and (int(snap["status"][0]) & 1) == 1
    assert snap["scale"][0] == 1.0

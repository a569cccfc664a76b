"""GPU parity: the GEMM whose epilogue re-quantises its result to FP8
(fp8_gemm_requant) against the oracle's bracket, and against the unfused
device path (fp32 GEMM, then the cast) bit for bit."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, mfma8_bound, to_device, u8
from oracle import codec, gemm
from synth import fc1_forward

pytestmark = pytest.mark.gpu


def rand_codes(rng, shape, fmt):
    f = codec.FORMATS[fmt]
    mag = rng.integers(0, f.max_code + 1, size=shape)
    return (mag | (rng.integers(0, 2, size=shape) << 7)).astype(np.uint8)


def _dev_scalar(v, dev):
    return torch.tensor([float(v)], dtype=torch.float32, device=dev)


def _run_both(qa, fa, qbT, fb, sa, sb, out_fmt, s_out, accum):
    """Fused re-quantising GEMM, and the fp32 GEMM followed by the cast."""
    dev = device()
    a, b = torch.from_numpy(qa).to(dev), torch.from_numpy(qbT).to(dev)
    sa_d, sb_d, so_d = _dev_scalar(sa, dev), _dev_scalar(sb, dev), _dev_scalar(s_out, dev)
    M, N = qa.shape[0], qbT.shape[0]
    cq = torch.full((M, N), 0xA5, dtype=torch.uint8, device=dev)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    sat = torch.full((1,), 12345, dtype=torch.int64, device=dev)
    fm.fp8_gemm_requant(a, fa, b, fb, sa_d, sb_d, out_fmt, so_d, cq, amax=amax, sat=sat, accum=accum)
    c32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    fm.fp8_gemm(a, fa, b, fb, sa_d, sb_d, c32, accum=accum)
    q2 = torch.empty((M, N), dtype=torch.uint8, device=dev)
    amax2 = torch.empty((1,), dtype=torch.float32, device=dev)
    sat2 = torch.empty((1,), dtype=torch.int64, device=dev)
    fm.fp8_quantize(c32, out_fmt, so_d, q=q2, amax=amax2, sat=sat2)
    torch.cuda.synchronize()
    return (u8(cq), f32(amax)[0], int(sat.item())), (u8(q2), f32(amax2)[0], int(sat2.item()))


# (1100, 1030, 400) and (1024, 1040, 144): the 256x256-tile path with edge
# tiles and a ragged last K step.
SHAPES = [(64, 64, 128), (1, 1, 16), (300, 260, 272), (257, 513, 144), (1100, 1030, 384), (1024, 1040, 256),
          (1100, 1030, 400), (1024, 1040, 144)]


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
@pytest.mark.parametrize("out_fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_requant_within_bracket_and_equal_to_unfused(M, N, K, out_fmt, accum):
    """Random codes; an output scale that saturates the largest results and
    pushes the smallest into subnormals.  Codes, amax and the saturation count
    lie in the oracle's bracket, and equal the unfused device path exactly."""
    announce(f"requant {M}x{N}x{K} -> {out_fmt} {accum}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    fa, fb = ("e5m2", "e4m3") if out_fmt == "e5m2" else ("e4m3", "e4m3")
    qa, qbT = rand_codes(rng, (M, K), fa), rand_codes(rng, (N, K), fb)
    sa, sb = np.float32(0.125), np.float32(0.0625)
    c64 = gemm.dequant_gemm(qa, fa, qbT.T, fb, sa, sb)
    mx = float(np.max(np.abs(c64)))
    s_out = np.float32(codec.FORMATS[out_fmt].max_value / (0.6 * mx)) if mx > 0 else np.float32(1.0)
    fused, unfused = _run_both(qa, fa, qbT, fb, sa, sb, out_fmt, s_out, accum)
    assert np.array_equal(fused[0], unfused[0])
    assert fused[1].view(np.uint32) == unfused[1].view(np.uint32) and fused[2] == unfused[2]
    bound = (gemm.abs_bound(qa, fa, qbT.T, fb, sa, sb) if accum == "exact"
             else mfma8_bound(qa, fa, qbT, fb, sa, sb))
    r = gemm.requant_bracket(c64, bound, s_out, out_fmt)
    got = codec.decode(fused[0], out_fmt)
    ok = (got >= r["lo"]) & (got <= r["hi"])
    assert ok.all(), np.argwhere(~ok)[:5]
    assert r["amax"][0] <= float(fused[1]) <= r["amax"][1]
    assert r["sat"][0] <= fused[2] <= r["sat"][1]
    if M * N >= 4096:
        assert fused[2] > 0                   # the scale does saturate some outputs


def test_requant_empty_clears_stats():
    dev = device()
    a = torch.zeros((0, 32), dtype=torch.uint8, device=dev)
    b = torch.zeros((16, 32), dtype=torch.uint8, device=dev)
    one = _dev_scalar(1.0, dev)
    cq = torch.zeros((0, 16), dtype=torch.uint8, device=dev)
    amax = torch.full((1,), 7.0, dtype=torch.float32, device=dev)
    sat = torch.full((1,), 9, dtype=torch.int64, device=dev)
    fm.fp8_gemm_requant(a, "e4m3", b, "e4m3", one, one, "e4m3", one, cq, amax=amax, sat=sat)
    torch.cuda.synchronize()
    assert amax.item() == 0.0 and sat.item() == 0


def test_requant_without_stats_outputs():
    """amax and sat are optional; the codes do not depend on them."""
    dev = device()
    rng = np.random.default_rng(5)
    qa, qbT = rand_codes(rng, (200, 144), "e4m3"), rand_codes(rng, (136, 144), "e4m3")
    a, b = torch.from_numpy(qa).to(dev), torch.from_numpy(qbT).to(dev)
    s = _dev_scalar(0.01, dev)
    c1 = torch.empty((200, 136), dtype=torch.uint8, device=dev)
    c2 = torch.empty_like(c1)
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    fm.fp8_gemm_requant(a, "e4m3", b, "e4m3", s, s, "e4m3", _dev_scalar(3.0, dev), c1)
    fm.fp8_gemm_requant(a, "e4m3", b, "e4m3", s, s, "e4m3", _dev_scalar(3.0, dev), c2, amax=amax)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


@pytest.mark.timeout(400)
def test_fc1_forward_requant_full_size():
    """The FC1 forward at full size with its output re-quantised to E4M3 with
    a delayed-style scale (448 / the amax of a first fp32 run): equal to the
    unfused device path; sampled codes within the oracle's bracket."""
    dev = device()
    d = fc1_forward(priors=False)
    X, W = to_device(d["X"], dev), to_device(d["W"], dev)
    stX = fm.DelayedScalingState("e4m3", 16, device=dev)
    stW = fm.DelayedScalingState("e4m3", 16, device=dev)
    qx = torch.empty((8192, 4096), dtype=torch.uint8, device=dev)
    qwT = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
    for _ in range(2):
        stX.quantize(X, q=qx)
        stX.update()
        stW.quantize(W, q_t=qwT)
        stW.update()
    announce("fc1 full size requant")
    c32 = torch.empty((8192, 16384), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv, stW.scale_inv, c32)
    amax0 = torch.empty((1,), dtype=torch.float32, device=dev)
    fm.fp8_quantize(c32, "e4m3", None, amax=amax0)
    torch.cuda.synchronize()
    s_out = np.float32(448.0 / float(amax0.item()))
    so = _dev_scalar(s_out, dev)
    cq = torch.empty((8192, 16384), dtype=torch.uint8, device=dev)
    amax = torch.empty((1,), dtype=torch.float32, device=dev)
    sat = torch.empty((1,), dtype=torch.int64, device=dev)
    fm.fp8_gemm_requant(qx, "e4m3", qwT, "e4m3", stX.scale_inv, stW.scale_inv, "e4m3", so, cq, amax=amax, sat=sat)
    q2 = torch.empty_like(cq)
    amax2 = torch.empty_like(amax)
    sat2 = torch.empty_like(sat)
    fm.fp8_quantize(c32, "e4m3", so, q=q2, amax=amax2, sat=sat2)
    torch.cuda.synchronize()
    assert torch.equal(cq, q2)
    assert amax.item() == amax2.item() == amax0.item() and sat.item() == sat2.item()
    qa, qbT, got = u8(qx), u8(qwT), u8(cq)
    sa, sb = stX.scale_inv.item(), stW.scale_inv.item()
    rng = np.random.default_rng(61)
    ms, ns = rng.integers(0, 8192, 1024), rng.integers(0, 16384, 1024)
    floor = 0.0
    for m, n in zip(ms, ns):
        num, sh = gemm.exact_dot(qa[m], "e4m3", qbT[n], "e4m3")
        exact = np.ldexp(float(num), -sh) * sa * sb
        bound = gemm.abs_bound(qa[m:m + 1], "e4m3", qbT[n:n + 1].T, "e4m3", sa, sb)[0]
        r = gemm.requant_bracket(np.array([exact]), bound, s_out, "e4m3")
        v = codec.decode(got[m:m + 1, n], "e4m3")[0]
        assert r["lo"][0] <= v <= r["hi"][0], (m, n, v, r["lo"][0], r["hi"][0])
        floor = max(floor, r["amax"][0])
    # the recorded amax covers every result, so it is at least the sampled results' lower brackets
    assert float(amax.item()) >= floor > 0.0


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_requant_nonfinite_results_equal_unfused(accum):
    """Rows of A holding a NaN code (E4M3 0x7F) or an Inf code (E5M2 0x7C): the
    codes, the amax (NaN above everything) and the count (Inf counts, NaN does
    not) equal the unfused path's, on a ragged shape so edge tiles take the
    bounds tests.  In the exact mode those rows are NaN / +-Inf results, coded
    sign|0x7F and +-max."""
    announce(f"requant non-finite {accum}")
    rng = np.random.default_rng(17)
    M, N, K = 300, 260, 272
    for fa, bad_code in (("e4m3", 0x7F), ("e5m2", 0x7C)):
        qa, qbT = rand_codes(rng, (M, K), fa), rand_codes(rng, (N, K), "e4m3")
        qa[3, 5] = bad_code
        qa[299, 0] = bad_code | 0x80
        for out_fmt in ("e4m3", "e5m2"):
            fused, unfused = _run_both(qa, fa, qbT, "e4m3", np.float32(0.125), np.float32(0.0625), out_fmt,
                                       np.float32(1e-3), accum)
            assert np.array_equal(fused[0], unfused[0])
            assert fused[1].view(np.uint32) == unfused[1].view(np.uint32) and fused[2] == unfused[2]
            got = fused[0]
            if accum != "exact":
                continue      # how the FP8 matrix cores treat NaN / Inf inputs is not specified here
            if bad_code == 0x7F:
                assert np.all((got[3] & 0x7F) == 0x7F) and np.isnan(fused[1])
            else:
                mx = 0x7E if out_fmt == "e4m3" else 0x7B
                assert np.all(((got[3] & 0x7F) == mx) | ((got[3] & 0x7F) == 0x7F))
                assert fused[2] >= N

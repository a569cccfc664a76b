"""GPU parity: fp8_gemm against the oracle's exact / fp64 dequantised GEMM.

fp32 outputs must satisfy |C_gpu - C64| <= 1e-5 * sum_k |a b| * sinv_a * sinv_b;
bf16 outputs must lie between the bf16 roundings of C64 -+ that bound (round to
nearest even is monotone, so this is "some fp32 value within the bound rounds
to the bf16 result").  Closed-form cases are checked exactly."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, mfma8_bound, to_device, u8
from oracle import codec, gemm, scaling
from synth import dgrad_hybrid, fc1_forward, tiny_operands

pytestmark = pytest.mark.gpu


def rand_codes(rng, shape, fmt):
    f = codec.FORMATS[fmt]
    mag = rng.integers(0, f.max_code + 1, size=shape)
    return (mag | (rng.integers(0, 2, size=shape) << 7)).astype(np.uint8)


ACCUMS = ["exact", "mfma_fp8"]


def run_gemm(qa, fa, qbT, fb, sa, sb, out="f32", accum="exact", b_trans=False):
    """qbT is B as [N x K]; with b_trans the library is handed B as [K x N] instead."""
    dev = device()
    a = torch.from_numpy(np.ascontiguousarray(qa)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(qbT.T if b_trans else qbT)).to(dev)
    c = torch.empty((qa.shape[0], qbT.shape[0]), dtype=torch.float32 if out == "f32" else torch.bfloat16,
                    device=dev)
    fm.fp8_gemm(a, fa, b, fb, torch.tensor([float(sa)], dtype=torch.float32, device=dev),
                torch.tensor([float(sb)], dtype=torch.float32, device=dev), c, accum=accum, b_trans=b_trans)
    torch.cuda.synchronize()
    return f32(c)


def check_within_bound(c_gpu, qa, fa, qb, fb, sa, sb, out, bound=None):
    """Element-wise: |C_gpu - C64| <= bound (default: the method's 1e-5 * sum|ab|)."""
    c64 = gemm.dequant_gemm(qa, fa, qb, fb, sa, sb)
    if bound is None:
        bound = gemm.abs_bound(qa, fa, qb, fb, sa, sb)
    if out == "f32":
        err = np.abs(c_gpu.astype(np.float64) - c64)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])
    else:
        lo, hi = gemm.bf16_bracket(c64, bound)
        ok = (c_gpu >= lo) & (c_gpu <= hi)
        assert ok.all(), np.argwhere(~ok)[:5]


# The last three take the 256x256-tile path (M, N >= 1024) with edge tiles in
# both M and N; (1100, 1030, 400) and (1024, 1040, 144) also end on a ragged K
# step (K % 128 != 0), which that path stages through registers.
SHAPES = [(64, 64, 128), (1, 1, 16), (300, 260, 272), (257, 513, 144), (128, 2048, 256), (1100, 1030, 384),
          (1100, 1030, 400), (1024, 1040, 144)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_codes_exact_mode_within_method_bound(M, N, K, fa, fb, out):
    """Codes drawn uniformly over every finite value (the widest dynamic range
    the formats allow): the exact mode meets 1e-5 * sum|ab| everywhere."""
    rng = np.random.default_rng(M * 131 + N * 17 + K)
    qa = rand_codes(rng, (M, K), fa)
    qbT = rand_codes(rng, (N, K), fb)
    sa, sb = np.float32(0.37), np.float32(2.5e-3)
    announce(f"gemm exact M={M} N={N} K={K} {fa}x{fb}->{out}")
    c = run_gemm(qa, fa, qbT, fb, sa, sb, out, "exact")
    check_within_bound(c, qa, fa, qbT.T, fb, sa, sb, out)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_codes_mfma8_mode_within_hardware_bound(M, N, K, fa, fb, out):
    """The native FP8 matrix-core mode on the same adversarial codes stays within
    the error model of its arithmetic (see gpu_helpers.mfma8_bound)."""
    rng = np.random.default_rng(M * 131 + N * 17 + K)
    qa = rand_codes(rng, (M, K), fa)
    qbT = rand_codes(rng, (N, K), fb)
    sa, sb = np.float32(0.37), np.float32(2.5e-3)
    announce(f"gemm mfma8 M={M} N={N} K={K} {fa}x{fb}->{out}")
    c = run_gemm(qa, fa, qbT, fb, sa, sb, out, "mfma_fp8")
    check_within_bound(c, qa, fa, qbT.T, fb, sa, sb, out, bound=mfma8_bound(qa, fa, qbT, fb, sa, sb))


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("K", [4096, 16384])
def test_all_max_codes_exact(K, accum):
    """448^2 = 49 * 2^12 (and 448 * 57344 = 49 * 2^19): every partial sum is exact
    in fp32, in any order, so C = K * 448^2 bit for bit."""
    M, N = 256, 256
    for fa, ca in (("e4m3", 0x7E), ("e5m2", 0x7B)):
        qa = np.full((M, K), ca, dtype=np.uint8)
        qa[::2] |= 0x80
        qbT = np.full((N, K), 0x7E, dtype=np.uint8)
        announce(f"all-max K={K} {fa}")
        c = run_gemm(qa, fa, qbT, "e4m3", np.float32(1), np.float32(1), accum=accum)
        val = K * float(codec.decode(ca, fa)) * 448.0
        assert np.all(c[1::2] == val) and np.all(c[::2] == -val)


def all_finite_codes(fmt):
    """Every finite code of the format, both signs (E4M3: 254, E5M2: 248),
    subnormals 0x01.. and 0x81.. included."""
    f = codec.FORMATS[fmt]
    mags = np.arange(0, f.max_code + 1, dtype=np.uint8)
    return np.concatenate([mags, mags | 0x80]).astype(np.uint8)


PAIRS = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")]


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_permutation_selects_columns_exactly(fa, fb, accum):
    """B is a permutation whose nonzero entries cycle through every finite code
    of its format; A holds every finite code of its format in every row
    (shifted per row).  Each output is one exact product, so C must equal
    dec(A[m, perm[n]]) * dec(b_n) * sinv_a bit for bit: FP8 subnormals of
    either operand (E5M2 0x01-0x03, E4M3 0x01-0x07) must survive the
    contraction unflushed."""
    rng = np.random.default_rng(4)
    M, K = 200, 256
    codes_a = all_finite_codes(fa)
    qa = np.stack([np.resize(np.roll(codes_a, 3 * m), K) for m in range(M)]).astype(np.uint8)
    perm = rng.permutation(K)
    codes_b = all_finite_codes(fb)
    codes_b = codes_b[(codes_b & 0x7F) != 0]            # nonzero entries only
    cb = np.resize(codes_b, K)
    qbT = np.zeros((K, K), dtype=np.uint8)              # B^T[n, k] = dec(cb[n]) iff k == perm[n]
    qbT[np.arange(K), perm] = cb
    announce(f"permutation {fa}x{fb} {accum}")
    c = run_gemm(qa, fa, qbT, fb, np.float32(0.5), np.float32(1), accum=accum)
    want = codec.decode(qa, fa)[:, perm] * codec.decode(cb, fb)[None, :] * 0.5
    assert np.array_equal(c.astype(np.float64), want)


# B handed over as [K x N] (N a multiple of 16): small tiles, the 256x256 path
# with edge tiles, ragged last K steps (400, 144, 272) and a long K.
BT_SHAPES = [(64, 64, 128), (16, 16, 16), (300, 272, 272), (257, 528, 144), (128, 2048, 256),
             (1100, 1040, 400), (1024, 1040, 144), (1030, 1024, 4096)]


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("M,N,K", BT_SHAPES)
def test_b_trans_equals_the_k_contiguous_path(M, N, K, fa, fb, out, accum):
    """B stored [K x N] (b_trans): the kernels read it through the LDS transpose
    path in the same K order as the [N x K] layout, so both give the same bits;
    in the exact mode both lie within the method's bound."""
    rng = np.random.default_rng(M * 7 + N * 5 + K * 3)
    qa = rand_codes(rng, (M, K), fa)
    qbT = rand_codes(rng, (N, K), fb)
    sa, sb = np.float32(0.37), np.float32(2.5e-3)
    announce(f"b_trans M={M} N={N} K={K} {fa}x{fb}->{out} {accum}")
    c_nk = run_gemm(qa, fa, qbT, fb, sa, sb, out, accum)
    c_kn = run_gemm(qa, fa, qbT, fb, sa, sb, out, accum, b_trans=True)
    assert np.array_equal(c_kn.view(np.uint32), c_nk.view(np.uint32))
    if accum == "exact" and M * N * K <= (1 << 30):
        check_within_bound(c_kn, qa, fa, qbT.T, fb, sa, sb, out)


def test_b_trans_full_fc1_weight_layout():
    """The FC1 product with W handed over as stored, [K x N] = 4096 x 16384
    (no cast-transpose): equal to the product on the cast-transposed weight."""
    dev = device()
    rng = np.random.default_rng(99)
    M, K, N = 8192, 4096, 16384
    qa = torch.from_numpy(rand_codes(rng, (M, K), "e4m3")).to(dev)
    qkn = torch.from_numpy(rand_codes(rng, (K, N), "e4m3")).to(dev)
    qnk = qkn.t().contiguous()
    one = torch.ones(1, dtype=torch.float32, device=dev)
    announce("b_trans fc1 full size")
    for accum in ACCUMS:
        c1 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        c2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fm.fp8_gemm(qa, "e4m3", qnk, "e4m3", one, one, c1, accum=accum)
        fm.fp8_gemm(qa, "e4m3", qkn, "e4m3", one, one, c2, accum=accum, b_trans=True)
        torch.cuda.synchronize()
        assert torch.equal(c1.view(torch.int16), c2.view(torch.int16)), accum


@pytest.mark.parametrize("fa", ["e4m3", "e5m2"])
def test_fp8_matrix_cores_miss_the_method_bound_where_exact_mode_meets_it(fa):
    """Why the headline GEMM contracts on the bf16 matrix cores.  Every run of 8
    consecutive K products holds one product 448*448 (E4M3) or 57344*448 (E5M2
    times E4M3) and seven products 2^-10 of it.  The native FP8 instruction sums
    a run in fixed point 13 bits below its largest product, so each small
    product (binary 1100 0100 times a power of two, 4 bits below that grid) is
    cut by 4/196 of itself: the result misses 1e-5 * sum|ab| by an order of
    magnitude.  The exact mode (FP8 widened to bf16, fp32 sums) returns the
    exact sum, which is representable here."""
    K = 256
    M = N = 64
    big = 0x7E if fa == "e4m3" else 0x7B                    # 448 / 57344
    small = 0x2E if fa == "e4m3" else 0x53                  # 0.4375 = 448 * 2^-10 / 56 = 57344 * 2^-10
    qa = np.full((M, K), small, dtype=np.uint8)
    qa[:, ::8] = big
    qa[1::2] |= 0x80                                        # half the rows negative (all products of a row alike)
    qbT = np.full((N, K), 0x7E, dtype=np.uint8)             # B = 448 everywhere
    sa, sb = np.float32(1), np.float32(1)
    c64 = gemm.dequant_gemm(qa, fa, qbT.T, "e4m3", sa, sb)
    bound = gemm.abs_bound(qa, fa, qbT.T, "e4m3", sa, sb)
    announce(f"fp8 cores vs the bound ({fa})")
    exact = run_gemm(qa, fa, qbT, "e4m3", sa, sb, accum="exact").astype(np.float64)
    native = run_gemm(qa, fa, qbT, "e4m3", sa, sb, accum="mfma_fp8").astype(np.float64)
    assert np.array_equal(exact, c64)
    excess = np.abs(native - c64) / bound
    print(f"mfma_fp8 |err| / (1e-5 sum|ab|): min {excess.min():.3g} max {excess.max():.3g}", flush=True)
    assert np.all(excess > 1.0)
    # and it stays inside the hardware model the mfma_fp8 tests use
    assert np.all(np.abs(native - c64) <= mfma8_bound(qa, fa, qbT, "e4m3", sa, sb))


@pytest.mark.parametrize("accum", ACCUMS)
def test_zero_operand_gives_zero(accum):
    rng = np.random.default_rng(5)
    qa = np.zeros((130, 160), dtype=np.uint8)
    qbT = rand_codes(rng, (70, 160), "e4m3")
    c = run_gemm(qa, "e4m3", qbT, "e4m3", np.float32(3), np.float32(3), accum=accum)
    assert not c.any()


def test_nan_code_propagates_in_exact_mode():
    rng = np.random.default_rng(6)
    qa = rand_codes(rng, (64, 128), "e4m3")
    qbT = rand_codes(rng, (64, 128), "e4m3")
    qa[3, 17] = 0x7F                                   # E4M3 NaN
    c = run_gemm(qa, "e4m3", qbT, "e4m3", np.float32(1), np.float32(1), accum="exact")
    assert np.isnan(c[3]).all() and not np.isnan(np.delete(c, 3, axis=0)).any()


def _gpu_pipeline_scales(priors, fmt, dev):
    st = fm.DelayedScalingState(fmt, 16, device=dev)
    ref = scaling.DelayedScaling(fmt, 16)
    for p in priors:
        xd = to_device(p, dev)
        st.quantize(xd)
        st.update()
        ref.update(scaling.amax(scaling.widen(p.data, p.dtype)))
    return st, ref


@pytest.mark.parametrize("accum", ACCUMS)
def test_tiny_delayed_scaling_matmul_end_to_end(accum):
    """fp32 A 64x128, B 128x64 ~N(0,0.02); history pre-filled by 4 prior draws per
    operand; cast both E4M3; GEMM fp32 out; every element against exact dots
    (the method's bound for the exact mode, the hardware model for mfma_fp8)."""
    dev = device()
    d = tiny_operands()
    stA, refA = _gpu_pipeline_scales(d["A_priors"], "e4m3", dev)
    stB, refB = _gpu_pipeline_scales(d["B_priors"], "e4m3", dev)
    A, B = to_device(d["A"], dev), to_device(d["B"], dev)
    qa = torch.empty((64, 128), dtype=torch.uint8, device=dev)
    qbT = torch.empty((64, 128), dtype=torch.uint8, device=dev)
    stA.quantize(A, q=qa)
    stB.quantize(B, q_t=qbT)
    c = torch.empty((64, 64), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qa, "e4m3", qbT, "e4m3", stA.scale_inv, stB.scale_inv, c, accum=accum)
    torch.cuda.synchronize()
    wqa, wam, _ = scaling.quantize(d["A"].data, refA.scale, "e4m3")
    wqb, wbm, _ = scaling.quantize(d["B"].data, refB.scale, "e4m3")
    assert np.array_equal(u8(qa), wqa)
    assert np.array_equal(u8(qbT), wqb.T)
    assert stA.scale_inv.item() == refA.scale_inv and stB.scale_inv.item() == refB.scale_inv
    exact = gemm.exact_gemm_small(wqa, "e4m3", wqb, "e4m3")
    c64 = exact * np.float64(refA.scale_inv) * np.float64(refB.scale_inv)
    if accum == "exact":
        bound = gemm.abs_bound(wqa, "e4m3", wqb, "e4m3", refA.scale_inv, refB.scale_inv)
    else:
        bound = mfma8_bound(wqa, "e4m3", wqb.T, "e4m3", refA.scale_inv, refB.scale_inv)
    assert np.all(np.abs(f32(c).astype(np.float64) - c64) <= bound)
    # the FP8 result tracks the fp64 product of the unquantised inputs
    ref = d["A"].data.astype(np.float64) @ d["B"].data.astype(np.float64)
    assert np.max(np.abs(f32(c) - ref)) < 0.1 * np.max(np.abs(ref))
    # the history step after the GEMM: amax of this step enters the ring
    stA.update()
    stB.update()
    refA.update(wam)
    refB.update(wbm)
    torch.cuda.synchronize()
    assert stA.scale.item() == refA.scale and stB.scale.item() == refB.scale


def _sampled_check(c_gpu, qa, fa, qbT, fb, sa, sb, out, samples, seed):
    rng = np.random.default_rng(seed)
    M, N = c_gpu.shape
    ms = np.concatenate([rng.integers(0, M, samples), [0, M - 1, M - 1, 0]])
    ns = np.concatenate([rng.integers(0, N, samples), [0, N - 1, 0, N - 1]])
    da = {}
    db = {}
    for m, n in zip(ms, ns):
        num, sh = gemm.exact_dot(qa[m], fa, qbT[n], fb)
        exact = np.ldexp(float(num), -sh) * np.float64(sa) * np.float64(sb)
        if m not in da:
            da[m] = np.abs(codec.decode(qa[m], fa))
        if n not in db:
            db[n] = np.abs(codec.decode(qbT[n], fb))
        bound = 1e-5 * float(np.dot(da[m], db[n])) * np.float64(sa) * np.float64(sb)
        got = float(c_gpu[m, n])
        if out == "f32":
            assert abs(got - exact) <= bound, (m, n, got, exact, bound)
        else:
            lo, hi = gemm.bf16_bracket(np.float64([exact]), np.float64([bound]))
            assert lo[0] <= got <= hi[0], (m, n, got, exact, bound)


def test_fc1_forward_full_size():
    """X bf16 8192x4096 @ W bf16 4096x16384 -> bf16, the whole path: delayed-scaled
    casts (W cast-transposed), GEMM in the exact mode, sampled outputs against
    exact dot products within the method's bound."""
    accum = "exact"
    dev = device()
    d = fc1_forward()
    stX, refX = _gpu_pipeline_scales(d["X_priors"], "e4m3", dev)
    stW, refW = _gpu_pipeline_scales(d["W_priors"], "e4m3", dev)
    X, W = to_device(d["X"], dev), to_device(d["W"], dev)
    qx = torch.empty((8192, 4096), dtype=torch.uint8, device=dev)
    qwT = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
    announce("fc1 full size: quantize + gemm")
    stX.quantize(X, q=qx)
    stW.quantize(W, q_t=qwT)
    c = torch.empty((8192, 16384), dtype=torch.bfloat16, device=dev)
    fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv, stW.scale_inv, c, accum=accum)
    torch.cuda.synchronize()
    assert stX.scale_inv.item() == refX.scale_inv and stW.scale_inv.item() == refW.scale_inv
    qa, qbT = u8(qx), u8(qwT)
    # codes of a band of rows are re-derived by the oracle to tie the GEMM inputs to the path
    x32 = scaling.widen(d["X"].data[:64], "bf16")
    assert np.array_equal(qa[:64], scaling.quantize(x32, refX.scale, "e4m3")[0])
    _sampled_check(f32(c), qa, "e4m3", qbT, "e4m3", refX.scale_inv, refW.scale_inv, "bf16", 4096, 21)


def test_fc1_forward_full_size_mfma8_error_model():
    """The same FC1 product in the native FP8 matrix-core mode.  It does NOT meet
    the method's 1e-5 * sum|ab| bound everywhere on this workload (measured), so
    it is held to the error model of its arithmetic on sampled outputs instead."""
    dev = device()
    d = fc1_forward(priors=False)
    X, W = to_device(d["X"], dev), to_device(d["W"], dev)
    stX = fm.DelayedScalingState("e4m3", 16, device=dev)
    stW = fm.DelayedScalingState("e4m3", 16, device=dev)
    qx = torch.empty((8192, 4096), dtype=torch.uint8, device=dev)
    qwT = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
    for _ in range(2):                     # the second cast uses the amax-derived scale
        stX.quantize(X, q=qx)
        stX.update()
        stW.quantize(W, q_t=qwT)
        stW.update()
    c = torch.empty((8192, 16384), dtype=torch.float32, device=dev)
    announce("fc1 full size, mfma_fp8 mode")
    fm.fp8_gemm(qx, "e4m3", qwT, "e4m3", stX.scale_inv, stW.scale_inv, c, accum="mfma_fp8")
    torch.cuda.synchronize()
    qa, qbT = u8(qx), u8(qwT)
    sa, sb = stX.scale_inv.item(), stW.scale_inv.item()
    rng = np.random.default_rng(77)
    ms, ns = rng.integers(0, 8192, 256), rng.integers(0, 16384, 256)
    got = f32(c)[ms, ns].astype(np.float64)
    for i, (m, n) in enumerate(zip(ms, ns)):
        num, sh = gemm.exact_dot(qa[m], "e4m3", qbT[n], "e4m3")
        exact = np.ldexp(float(num), -sh) * sa * sb
        bound = mfma8_bound(qa[m:m + 1], "e4m3", qbT[n:n + 1], "e4m3", sa, sb)[0, 0]
        assert abs(got[i] - exact) <= bound, (m, n, got[i], exact, bound)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("accum", ACCUMS)
def test_dgrad_hybrid_full_size(accum):
    """dY bf16 8192x16384 (log-uniform magnitudes) as E5M2 @ W 16384x4096 as E4M3
    (cast-transposed) -> fp32; sampled outputs against exact dot products."""
    dev = device()
    d = dgrad_hybrid()
    stG, refG = _gpu_pipeline_scales(d["dY_priors"], "e5m2", dev)
    stW, refW = _gpu_pipeline_scales(d["W_priors"], "e4m3", dev)
    G, W = to_device(d["dY"], dev), to_device(d["W"], dev)
    qg = torch.empty((8192, 16384), dtype=torch.uint8, device=dev)
    qwT = torch.empty((4096, 16384), dtype=torch.uint8, device=dev)
    announce("dgrad full size: quantize + gemm")
    stG.quantize(G, q=qg)
    stW.quantize(W, q_t=qwT)
    c = torch.empty((8192, 4096), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qg, "e5m2", qwT, "e4m3", stG.scale_inv, stW.scale_inv, c, accum=accum)
    torch.cuda.synchronize()
    assert stG.scale_inv.item() == refG.scale_inv and stW.scale_inv.item() == refW.scale_inv
    _sampled_check(f32(c), u8(qg), "e5m2", u8(qwT), "e4m3", refG.scale_inv, refW.scale_inv, "f32", 2048, 31)

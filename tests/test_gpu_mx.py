"""GPU parity: MXFP8 quantisation (fp8_quantize_mx) bit for bit against the
oracle; the MXFP8 GEMM (fp8_gemm_mx) in the exact mode within the method's
1e-5 * sum|ab| of the oracle's product, and in the FP8-matrix-core mode within
the error model of that instruction."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, mx_mfma8_bound, to_device, u8
from oracle import codec, gemm, mx, scaling
from synth import HostTensor, bf16_bits_from_f32, fc1_forward

pytestmark = pytest.mark.gpu


def _special_rows(x):
    """Blocks the exponent rule treats specially (needs >= 8 rows and 256 columns)."""
    x[0, 0:32] = 0.0                                      # all zero -> exponent code 127
    x[1, 32:64] = np.float32(448.0)                       # amax exactly MAX -> e = 0
    x[1, 64:96] *= np.float32(0.0)
    x[1, 64] = np.float32(448.5)                          # just above MAX -> e = 1
    x[2, 0:32] = np.float32(1e-42)                        # subnormal amax -> clamped to -127
    x[3, 32] = np.inf                                     # Inf -> e = 0, full encoder
    x[4, 96] = np.nan                                     # NaN -> e = 0, NaN code
    x[5, 0:32] = np.float32(2.0 ** 100) * np.float32(1.75)
    x[6, 128:160] = -x[6, 128:160]
    x[7, 0:32] = np.float32(-0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (130, 256), (300, 1024), (17, 4096), (128, 544)])
def test_quantize_mx_bit_exact(shape, fmt, dtype):
    announce(f"quantize_mx {shape} {fmt} {dtype}")
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-30, 30, size=(shape[0], 1))).astype(np.float32)
    if shape[0] >= 8 and shape[1] >= 256:
        _special_rows(x)
    h = HostTensor(x, "f32") if dtype == "f32" else HostTensor(bf16_bits_from_f32(x), "bf16")
    xw = scaling.widen(h.data, dtype)
    dev = device()
    q = torch.empty(shape, dtype=torch.uint8, device=dev)
    s = torch.full((shape[1] // 32, fm.mx_scale_ld(shape[0])), 0xA5, dtype=torch.uint8, device=dev)
    fm.fp8_quantize_mx(to_device(h, dev), fmt, q, s)
    torch.cuda.synchronize()
    wq, ws = mx.quantize_mx(xw, fmt)
    pos = fm.mx_scale_pos(np.arange(shape[0]))
    assert np.array_equal(u8(s)[:, pos].T, ws)   # K-block major, rows permuted
    assert np.array_equal(u8(q), wq)
    pad = np.ones(s.shape[1], dtype=bool)
    pad[pos] = False
    assert (u8(s)[:, pad] == 0xA5).all()          # positions of rows past the end are not written


def test_quantize_mx_more_tiles_than_workgroups():
    """8293 x 4128 bf16: 130 row groups x 9 block columns = 1170 tiles of 64
    rows x 16 blocks, more than the 1024 workgroups launched, the last block
    column one block wide and the last row group 37 rows: sampled rows from
    every region (first pass, second pass, the cut group) bit for bit, and
    the padding positions untouched."""
    rows, cols = 8293, 4128
    announce(f"quantize_mx {rows}x{cols} bf16 e4m3, sampled rows")
    rng = np.random.default_rng(8293)
    x = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3, size=(rows, 1))).astype(np.float32)
    h = HostTensor(bf16_bits_from_f32(x), "bf16")
    dev = device()
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s = torch.full((cols // 32, fm.mx_scale_ld(rows)), 0xA5, dtype=torch.uint8, device=dev)
    fm.fp8_quantize_mx(to_device(h, dev), "e4m3", q, s)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([[0, 63, 64, 7295, 8191, 8255, 8256, 8292],
                                       rng.choice(rows, 24, replace=False)]))
    wq, ws = mx.quantize_mx(scaling.widen(h.data[sample], "bf16"), "e4m3")
    assert np.array_equal(u8(q)[sample], wq)
    assert np.array_equal(u8(s)[:, fm.mx_scale_pos(sample)].T, ws)
    pad = np.ones(s.shape[1], dtype=bool)
    pad[fm.mx_scale_pos(np.arange(rows))] = False
    assert pad.sum() == fm.mx_scale_ld(rows) - rows and (u8(s)[:, pad] == 0xA5).all()


def _rand_mx(rng, rows, K, fmt, lo=112, hi=142):
    f = codec.FORMATS[fmt]
    q = (rng.integers(0, f.max_code + 1, size=(rows, K)) | (rng.integers(0, 2, size=(rows, K)) << 7)).astype(np.uint8)
    s = rng.integers(lo, hi, size=(rows, K // 32)).astype(np.uint8)
    return q, s


def _dev_scales(s, dev, pad=127):
    """Row-major [rows x K/32] exponent codes -> the library's layout on the
    device: [K/32 x mx_scale_ld(rows)], row r at position mx_scale_pos(r)
    (pad bytes = `pad`)."""
    rows, nb = s.shape
    out = np.full((nb, fm.mx_scale_ld(rows)), pad, dtype=np.uint8)
    out[:, fm.mx_scale_pos(np.arange(rows))] = s.T
    return torch.from_numpy(out).to(dev)


def _check_mx(c_gpu, qa, sa, fa, qb, sb, fb, out):
    c64 = mx.mx_gemm(qa, sa, fa, qb, sb, fb)
    bound = mx_mfma8_bound(qa, sa, fa, qb, sb, fb)
    if out == "f32":
        err = np.abs(c_gpu.astype(np.float64) - c64)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])
    else:
        lo, hi = gemm.bf16_bracket(c64, bound)
        ok = (c_gpu >= lo) & (c_gpu <= hi)
        assert ok.all(), np.argwhere(~ok)[:5]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (1, 1, 128), (300, 260, 256), (257, 513, 384), (1100, 1030, 512)])
def test_gemm_mx_within_error_model(M, N, K, fa, fb, out):
    """Random codes over the whole range with random block exponents (2^-15 ..
    2^14) on both operands."""
    announce(f"gemm_mx {M}x{N}x{K} {fa}x{fb} {out}")
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    qa, sa = _rand_mx(rng, M, K, fa)
    qb, sb = _rand_mx(rng, N, K, fb)
    dev = device()
    c = torch.empty((M, N), dtype=torch.float32 if out == "f32" else torch.bfloat16, device=dev)
    fm.fp8_gemm_mx(torch.from_numpy(qa).to(dev), fa, _dev_scales(sa, dev), torch.from_numpy(qb).to(dev), fb,
                   _dev_scales(sb, dev, pad=255), c, accum="mfma_fp8")
    torch.cuda.synchronize()
    _check_mx(f32(c), qa, sa, fa, qb, sb, fb, out)


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_gemm_mx_block_scales_select_blocks(accum):
    """Closed form: all codes 1.0; A's block b of row m has exponent code 127 + b,
    B's block b of row n has 127 - b + (n % 3): C[m, n] = 32 * nb * 2^(n % 3),
    exact (every product a power of two, sums of equal terms)."""
    dev = device()
    M, N, K = 200, 136, 512
    nb = K // 32
    qa = np.full((M, K), 0x38, dtype=np.uint8)
    qb = np.full((N, K), 0x38, dtype=np.uint8)
    sa = np.tile(127 + np.arange(nb), (M, 1)).astype(np.uint8)
    sb = (127 - np.arange(nb)[None, :] + (np.arange(N) % 3)[:, None]).astype(np.uint8)
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    fm.fp8_gemm_mx(torch.from_numpy(qa).to(dev), "e4m3", _dev_scales(sa, dev), torch.from_numpy(qb).to(dev),
                   "e4m3", _dev_scales(sb, dev), c, accum=accum)
    torch.cuda.synchronize()
    want = 32.0 * nb * 2.0 ** (np.arange(N) % 3)
    assert np.array_equal(f32(c), np.tile(want, (M, 1)).astype(np.float32))


@pytest.mark.timeout(400)
def test_fc1_mx_full_size():
    """FC1 at full size with MXFP8 operands: X bf16 8192x4096 and W^T
    16384x4096 (rows = output features, K contiguous), both E4M3 MX-quantised
    on the GPU; codes and exponents of sampled rows bit for bit, sampled GEMM
    outputs within the error model of the oracle's exact product."""
    dev = device()
    d = fc1_forward(priors=False)
    X = d["X"]
    W = HostTensor(np.ascontiguousarray(d["W"].data.T), "bf16")     # 16384 x 4096: rows = output features
    qx = torch.empty((8192, 4096), dtype=torch.uint8, device=dev)
    sx = torch.empty((128, 8192), dtype=torch.uint8, device=dev)
    qw = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
    sw = torch.empty((128, 16384), dtype=torch.uint8, device=dev)
    announce("fc1 mx full size: quantize + gemm")
    fm.fp8_quantize_mx(to_device(X, dev), "e4m3", qx, sx)
    fm.fp8_quantize_mx(to_device(W, dev), "e4m3", qw, sw)
    c = torch.empty((8192, 16384), dtype=torch.float32, device=dev)
    fm.fp8_gemm_mx(qx, "e4m3", sx, qw, "e4m3", sw, c, accum="mfma_fp8")
    ce = torch.empty((8192, 16384), dtype=torch.bfloat16, device=dev)
    fm.fp8_gemm_mx(qx, "e4m3", sx, qw, "e4m3", sw, ce, accum="exact")
    torch.cuda.synchronize()
    rng = np.random.default_rng(71)
    rows_x = np.concatenate([rng.choice(8192, 24, replace=False), [0, 8191]])
    rows_w = np.concatenate([rng.choice(16384, 24, replace=False), [0, 16383]])
    wqx, wsx = mx.quantize_mx(scaling.widen(X.data[rows_x], "bf16"), "e4m3")
    wqw, wsw = mx.quantize_mx(scaling.widen(W.data[rows_w], "bf16"), "e4m3")
    qx_h, qw_h = u8(qx)[rows_x], u8(qw)[rows_w]
    sx_h, sw_h = u8(sx)[:, fm.mx_scale_pos(rows_x)].T, u8(sw)[:, fm.mx_scale_pos(rows_w)].T
    assert np.array_equal(qx_h, wqx) and np.array_equal(sx_h, wsx)
    assert np.array_equal(qw_h, wqw) and np.array_equal(sw_h, wsw)
    got = f32(c)[np.ix_(rows_x, rows_w)]
    _check_mx(got, wqx, wsx, "e4m3", wqw, wsw, "e4m3", "f32")
    # the exact mode on the same operands: the method's bound (bf16 output)
    _check_mx_exact(f32(ce)[np.ix_(rows_x, rows_w)], wqx, wsx, "e4m3", wqw, wsw, "e4m3", "bf16")


def _check_mx_exact(c_gpu, qa, sa, fa, qb, sb, fb, out, nan_rows=(), nan_cols=()):
    """The method's tolerance on the dequantised operands: |C - C64| <= 1e-5 *
    sum_k |a_k b_k| (bf16: the bracket of C64 -+ that bound); rows / columns
    listed as outside the exact path's exponent window must be NaN."""
    c64 = mx.mx_gemm(qa, sa, fa, qb, sb, fb)
    bound = 1e-5 * (np.abs(mx.dequant_mx(qa, sa, fa)) @ np.abs(mx.dequant_mx(qb, sb, fb)).T)
    mask = np.zeros(c64.shape, dtype=bool)
    mask[list(nan_rows), :] = True
    mask[:, list(nan_cols)] = True
    assert np.isnan(c_gpu[mask]).all()
    c_gpu, c64, bound = c_gpu[~mask], c64[~mask], bound[~mask]
    if out == "f32":
        err = np.abs(c_gpu.astype(np.float64) - c64)
        bad = np.flatnonzero(err > bound)
        assert bad.size == 0, (bad[:5], err[bad[0]], bound[bad[0]])
    else:
        lo, hi = gemm.bf16_bracket(c64, bound)
        ok = (c_gpu >= lo) & (c_gpu <= hi)
        assert ok.all(), np.flatnonzero(~ok)[:5]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (1, 1, 128), (300, 260, 256), (257, 513, 384), (1100, 1030, 512),
                                   (1024, 1040, 640)])
def test_gemm_mx_exact_within_method_bound(M, N, K, fa, fb, out):
    """Exact mode: random codes over every finite value (subnormals included)
    with random block exponents 2^-15 .. 2^14 on both operands (the window of
    the exact path is 47 binades per row): within 1e-5 * sum|ab| everywhere."""
    announce(f"gemm_mx exact {M}x{N}x{K} {fa}x{fb} {out}")
    rng = np.random.default_rng(M + 3 * N + 7 * K + 1)
    qa, sa = _rand_mx(rng, M, K, fa)
    qb, sb = _rand_mx(rng, N, K, fb)
    dev = device()
    c = torch.empty((M, N), dtype=torch.float32 if out == "f32" else torch.bfloat16, device=dev)
    fm.fp8_gemm_mx(torch.from_numpy(qa).to(dev), fa, _dev_scales(sa, dev), torch.from_numpy(qb).to(dev), fb,
                   _dev_scales(sb, dev, pad=255), c, accum="exact")
    torch.cuda.synchronize()
    _check_mx_exact(f32(c), qa, sa, fa, qb, sb, fb, out)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e5m2")])
def test_gemm_mx_exact_window_edges_zero_blocks_and_nan_rows(fa, fb):
    """Rows whose block exponents span exactly 47 (the window's edge) stay
    within the bound; all-zero blocks (code 127) next to small blocks inside the
    window are harmless; a row of A and a row of B spanning 48 are reported as
    NaN rows / columns, every other output within the bound."""
    M, N, K = 260, 300, 512
    rng = np.random.default_rng(47)
    qa, sa = _rand_mx(rng, M, K, fa, 110, 140)
    qb, sb = _rand_mx(rng, N, K, fb, 110, 140)
    sa[5, :] = 120
    sa[5, 3], sa[5, 9] = 160, 113                # span 47 exactly
    sb[7, :] = 130
    sb[7, 0], sb[7, 15] = 90, 137                # span 47
    qa[11, 64:96] = 0
    sa[11, :] = 100
    sa[11, 2] = 127                               # an all-zero block with code 127, others 27 below
    sa[200, 0], sa[200, 1] = 170, 122            # span 48: outside
    sb[250, 4], sb[250, 5] = 100, 148            # span 48: outside
    dev = device()
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    fm.fp8_gemm_mx(torch.from_numpy(qa).to(dev), fa, _dev_scales(sa, dev), torch.from_numpy(qb).to(dev), fb,
                   _dev_scales(sb, dev), c, accum="exact")
    torch.cuda.synchronize()
    _check_mx_exact(f32(c), qa, sa, fa, qb, sb, fb, "f32", nan_rows=[200], nan_cols=[250])

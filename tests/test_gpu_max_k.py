"""GEMMs at the largest K each entry point accepts (include/fp8mi.h): dense
2^23, dense with B stored [K x N] at K * N = 2^31 - 32768, grouped 2^22; and a
cast of more than 2^31 elements.

At these depths the slab loads' 32-bit buffer offsets come within a few MiB
of 2^31 (the host replays in test_load_bounds.py check every one of them).
The operands make the exact result a closed form: every code of a row is the
same power of two and the scales are powers of two, so each product is a power
of two, every partial sum is an exact multiple of it far below 2^24 of it, and
both accumulation modes (bf16 matrix cores; FP8 matrix cores, whose groups of
eight equal products are summed exactly) must return it bit for bit.  For the
grouped GEMM the expected value is the two-level sum of "#fp8" tag page,
DeepGEMM entry, written out per 128-deep block."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32
from oracle import codec

pytestmark = pytest.mark.gpu


def _rows_of_codes(values, K, dev):
    """[len(values) x K] uint8 on the device, row r filled with the E4M3 code of values[r]."""
    codes = codec.encode(np.asarray(values, dtype=np.float32), "e4m3")
    t = torch.empty((len(values), K), dtype=torch.uint8, device=dev)
    t.copy_(torch.from_numpy(codes).to(dev).view(-1, 1).expand(-1, K))
    return t


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
@pytest.mark.parametrize("M,N", [(64, 48), (1024, 1040)])      # 128x128 tiles; 256x256 tiles with a ragged N
def test_dense_gemm_at_the_largest_k(M, N, accum):
    dev = device()
    K = 1 << 23
    announce(f"dense GEMM {M}x{N}x{K} {accum}")
    a_vals = 2.0 ** (np.arange(M) % 4 - 2)                       # 0.25, 0.5, 1, 2
    b_vals = 2.0 ** (np.arange(N) % 3 - 1)                       # 0.5, 1, 2
    qa = _rows_of_codes(a_vals, K, dev)
    qb = _rows_of_codes(b_vals, K, dev)
    sa = torch.tensor([2.0 ** -3], device=dev)
    sb = torch.tensor([2.0 ** -2], device=dev)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qa, "e4m3", qb, "e4m3", sa, sb, c, accum=accum)
    torch.cuda.synchronize()
    want = (K * np.outer(a_vals, b_vals) * 2.0 ** -5).astype(np.float32)
    got = f32(c)
    del qa, qb, c
    torch.cuda.empty_cache()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_dense_gemm_b_trans_at_the_largest_k_times_n(accum):
    """B stored [K x N] with K * N = 2^31 - 32768 (the entry point allows 2^31 - 1):
    column j of B holds b_j in every K row."""
    dev = device()
    M, N, K = 64, 256, (1 << 23) - 128
    announce(f"dense GEMM b_trans {M}x{N}x{K} {accum}")
    a_vals = 2.0 ** (np.arange(M) % 4 - 2)
    b_vals = 2.0 ** (np.arange(N) % 3 - 1)
    qa = _rows_of_codes(a_vals, K, dev)
    b_codes = codec.encode(b_vals.astype(np.float32), "e4m3")
    qb = torch.empty((K, N), dtype=torch.uint8, device=dev)
    qb.copy_(torch.from_numpy(b_codes).to(dev).view(1, -1).expand(K, -1))
    one = torch.ones(1, device=dev)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    fm.fp8_gemm(qa, "e4m3", qb, "e4m3", one, one, c, accum=accum, b_trans=True)
    torch.cuda.synchronize()
    want = (K * np.outer(a_vals, b_vals)).astype(np.float32)
    got = f32(c)
    del qa, qb, c
    torch.cuda.empty_cache()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_grouped_gemm_at_the_largest_k(accum):
    """Two experts of 128 and 64 rows, N = 512, K = 2^22 (32768 blocks of 128):
    A row m holds a_m, B row (g, n) holds b_gn, and the block scales are powers
    of two that vary with the row, the column block and the K block, so each
    output is sum over blocks kb of 128 * a_m * b_gn * sinv_a[m, kb] * sinv_b[g, n/128, kb]."""
    dev = device()
    counts, N, K = [128, 64], 512, 1 << 22
    G, total, nk = len(counts), sum(counts), (1 << 22) // 128
    announce(f"grouped GEMM counts={counts} N={N} K={K} {accum}")
    offs = np.array([0, counts[0], total], dtype=np.int32)
    a_vals = 2.0 ** (np.arange(total) % 2)                      # 1, 2
    b_vals = 2.0 ** -(np.arange(G * N) % 2)                     # 1, 0.5
    qa = _rows_of_codes(a_vals, K, dev)
    qb = _rows_of_codes(b_vals, K, dev).view(G, N, K)
    kb = np.arange(nk)
    sa_h = (2.0 ** ((np.arange(total)[:, None] + kb[None, :]) % 3 - 1)).astype(np.float32)        # 0.5, 1, 2
    gi, nbi = np.meshgrid(np.arange(G), np.arange(N // 128), indexing="ij")
    sb_h = (2.0 ** ((gi[..., None] + nbi[..., None] + kb[None, None, :]) % 2)).astype(np.float32)  # 1, 2
    c = torch.full((total, N), float("nan"), dtype=torch.float32, device=dev)
    fm.fp8_grouped_gemm(qa, torch.from_numpy(sa_h).to(dev), qb, torch.from_numpy(sb_h).to(dev),
                        torch.from_numpy(offs).to(dev), c, accum=accum)
    torch.cuda.synchronize()
    got = f32(c)
    del qa, qb, c
    torch.cuda.empty_cache()
    want = np.empty((total, N), dtype=np.float64)
    for g in range(G):
        rows = np.arange(offs[g], offs[g + 1])
        for nb in range(N // 128):
            cols = np.arange(nb * 128, (nb + 1) * 128)
            s = sa_h[rows].astype(np.float64) @ sb_h[g, nb].astype(np.float64)       # sum over kb
            want[np.ix_(rows, cols)] = 128.0 * np.outer(a_vals[rows] * s, b_vals[g * N + cols])
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("transposed", [False, True])
def test_cast_of_more_than_2_31_elements(transposed):
    """bf16 131136 x 16384 (2^31 + 2^20 elements): zeros except four planted
    values, one of them the very last element.  The flat cast (q only) and the
    cast-transpose (q and q_t) must put each planted code at its place and
    nothing else anywhere, and report the planted amax and saturation count."""
    dev = device()
    rows, cols = 131136, 16384
    announce(f"cast of {rows}x{cols} bf16 (transposed={transposed})")
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device=dev)
    plant = {(rows - 1, cols - 1): 1000.0, (rows - 1, 0): -3.5, (rows // 2, 7): 0.1, (0, cols - 1): 2.0}
    for (r, c), v in plant.items():
        x[r, c] = v
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev) if transposed else None
    scale = torch.tensor([1.0], device=dev)
    amax = torch.full((1,), 7.0, device=dev)
    sat = torch.full((1,), 5, dtype=torch.int64, device=dev)
    ws = torch.empty(fm.QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    fm.fp8_quantize(x, "e4m3", scale, q=q, q_t=q_t, amax=amax, sat=sat, workspace=ws)
    torch.cuda.synchronize()
    vals = np.array([float(x[r, c].float().item()) for (r, c) in plant], dtype=np.float32)   # as stored in bf16
    want = codec.encode(vals, "e4m3")
    for (r, c), code in zip(plant, want):
        assert int(q[r, c].item()) == int(code), (r, c)
        if transposed:
            assert int(q_t[c, r].item()) == int(code), (r, c)
    assert int(torch.count_nonzero(q).item()) == np.count_nonzero(want)
    if transposed:
        assert int(torch.count_nonzero(q_t).item()) == np.count_nonzero(want)
    assert f32(amax).view(np.uint32)[0] == np.float32(np.abs(vals).max()).view(np.uint32)
    assert int(sat.item()) == int(np.count_nonzero(np.abs(vals) > 448.0))

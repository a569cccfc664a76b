"""GPU parity: per-block quantisation (fp8_quantize_blockwise) bit for bit, and
the fine-grained grouped GEMM (fp8_grouped_gemm) within the error bound."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device, f32, grouped_mfma8_bound, to_device, u8
from oracle import gemm, scaling
from synth import HostTensor, bf16_bits_from_f32, moe_grouped

pytestmark = pytest.mark.gpu


def gpu_blockwise(xd, block_rows, fmt="e4m3"):
    rows, cols = xd.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=xd.device)
    si = torch.empty(((rows + block_rows - 1) // block_rows, (cols + 127) // 128), dtype=torch.float32,
                     device=xd.device)
    fm.fp8_quantize_blockwise(xd, block_rows, fmt, q, si)
    return q, si


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("block_rows", [1, 128])
@pytest.mark.parametrize("shape", [(1, 16), (5, 304), (130, 272), (300, 1040), (128, 128)])
def test_blockwise_bit_exact(shape, block_rows, dtype):
    rng = np.random.default_rng(shape[0] * 1000 + shape[1] + block_rows)
    x32 = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-4, 4, size=(shape[0], 1))).astype(np.float32)
    if shape[0] > 2:
        x32[1, :] = 0.0                          # all-zero row tiles -> scale 1
        x32[2, 3] = np.inf                       # non-finite block amax -> scale 1
    h = HostTensor(x32, "f32") if dtype == "f32" else HostTensor(bf16_bits_from_f32(x32), "bf16")
    xw = scaling.widen(h.data, dtype)
    announce(f"blockwise {shape} br={block_rows} {dtype}")
    for fmt in ("e4m3", "e5m2"):
        q, si = gpu_blockwise(to_device(h), block_rows, fmt)
        torch.cuda.synchronize()
        wq, wsi = scaling.quantize_blockwise(xw, block_rows, 128, fmt)
        assert np.array_equal(u8(q), wq)
        assert np.array_equal(f32(si).view(np.uint32), wsi.view(np.uint32))


def test_blockwise_rowtiles_beyond_one_pass_of_the_grid():
    """8200 x 16384 bf16 in 1 x 128 tiles: 1,049,600 tiles against the capped
    grid's 262,144 sixteen-lane groups (16384 workgroups x 16), so every group
    takes several tiles and the rows past 8192 come from a fifth pass:
    sampled rows from the first and the last passes bit for bit, codes and
    scales."""
    rows, cols = 8200, 16384
    rng = np.random.default_rng(8200)
    x32 = (rng.standard_normal((rows, cols), dtype=np.float32)
           * np.float32(10.0) ** rng.uniform(-3, 3, size=(rows, 1)).astype(np.float32))
    h = HostTensor(bf16_bits_from_f32(x32), "bf16")
    del x32
    announce(f"blockwise rowtiles {rows}x{cols} bf16, sampled rows")
    q, si = gpu_blockwise(to_device(h), 1, "e4m3")
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([[0, 8191, 8192, 8199], rng.choice(rows, 12, replace=False)]))
    wq, wsi = scaling.quantize_blockwise(scaling.widen(h.data[sample], "bf16"), 1, 128, "e4m3")
    assert np.array_equal(u8(q)[sample], wq)
    assert np.array_equal(f32(si).reshape(rows, -1)[sample].view(np.uint32), wsi.view(np.uint32))


def test_blockwise_rejects_columns_not_multiple_of_16():
    x = torch.zeros((5, 300), dtype=torch.float32, device=device())
    q = torch.empty((5, 300), dtype=torch.uint8, device=x.device)
    si = torch.empty((5, 3), dtype=torch.float32, device=x.device)
    with pytest.raises(fm.Fp8Error):
        fm.fp8_quantize_blockwise(x, 1, "e4m3", q, si)


def _grouped_case(counts, K, N, seed, out="bf16", accum="exact"):
    dev = device()
    rng = np.random.default_rng(seed)
    total = int(sum(counts))
    offs = np.zeros(len(counts) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    A32 = rng.standard_normal((total, K)).astype(np.float32)
    B32 = (rng.standard_normal((len(counts), N, K)) * 0.02).astype(np.float32)
    Ad, Bd = to_device((A32, "f32"), dev), to_device((B32.reshape(-1, K), "f32"), dev)
    qa, sa = gpu_blockwise(Ad, 1)
    qb, sb = gpu_blockwise(Bd, 128) if N % 128 == 0 else (None, None)
    if qb is None:                                # per-expert blocks when N is ragged
        qb = torch.empty((len(counts) * N, K), dtype=torch.uint8, device=dev)
        sb = torch.empty((len(counts), (N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device=dev)
        for g in range(len(counts)):
            q_g, s_g = gpu_blockwise(Bd[g * N:(g + 1) * N], 128)
            qb[g * N:(g + 1) * N] = q_g
            sb[g] = s_g
    c = torch.full((total, N), float("nan"), dtype=torch.float32 if out == "f32" else torch.bfloat16, device=dev)
    fm.fp8_grouped_gemm(qa, sa, qb.view(len(counts), N, K), sb.view(len(counts), -1, (K + 127) // 128),
                        torch.from_numpy(offs).to(dev), c, accum=accum)
    torch.cuda.synchronize()
    qa_h, sa_h = u8(qa), f32(sa)
    qb_h = u8(qb).reshape(len(counts), N, K)
    sb_h = f32(sb).reshape(len(counts), (N + 127) // 128, (K + 127) // 128)
    return f32(c), qa_h, sa_h, qb_h, sb_h, offs


def _check_grouped(c, qa, sa, qb, sb, offs, out, rows=None, bound=None):
    c64 = gemm.grouped_gemm(qa, sa, qb, sb, offs, rows=rows)
    if bound is None:
        bound = gemm.grouped_abs_bound(qa, sa, qb, sb, offs, rows=rows)
    got = c if rows is None else c[rows]
    if out == "f32":
        assert np.all(np.abs(got.astype(np.float64) - c64) <= bound)
    else:
        lo, hi = gemm.bf16_bracket(c64, bound)
        ok = (got >= lo) & (got <= hi)
        assert ok.all(), np.argwhere(~ok)[:5]


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("counts,K,N", [([64, 0, 200, 17], 272, 256), ([1], 128, 128), ([300, 129], 144, 260),
                                        ([128] * 8, 512, 384), ([130, 0, 0, 1, 1000, 7, 256], 256, 1040),
                                        ([200, 0, 77, 300], 1200, 384), ([129, 256], 2176, 256),
                                        ([3, 130], 16, 256)])
def test_grouped_small_within_bound(counts, K, N, out, accum):
    """Per-block-scaled N(0,1) activations and N(0,0.02) weights: the exact mode
    within the method's per-block bound, the FP8 matrix-core mode within the
    error model of its arithmetic."""
    announce(f"grouped counts={counts} K={K} N={N} {out} {accum}")
    c, qa, sa, qb, sb, offs = _grouped_case(counts, K, N, seed=len(counts) * 7 + K, out=out, accum=accum)
    bound = None if accum == "exact" else grouped_mfma8_bound(qa, sa, qb, sb, offs)
    _check_grouped(c, qa, sa, qb, sb, offs, out, bound=bound)


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_grouped_offsets_not_monotone(accum):
    """Offsets [20, 250, 100, 400, 380, 550] over 600 rows: each expert's interval
    is clamped to [end of the previous one, total rows], giving [20, 250),
    empty, [250, 400), empty, [400, 550); rows 0-19 and 550-599 belong to no
    expert and keep what the output held.  The written rows are checked against
    the oracle on the clamped offsets."""
    dev = device()
    rng = np.random.default_rng(24)
    total, K, N = 600, 272, 256
    raw = np.array([20, 250, 100, 400, 380, 550], dtype=np.int32)
    eff = np.array([20, 250, 250, 400, 400, 550], dtype=np.int32)
    G = raw.size - 1
    announce(f"grouped non-monotone offsets {raw.tolist()} {accum}")
    A32 = rng.standard_normal((total, K)).astype(np.float32)
    B32 = (rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)
    qa, sa = gpu_blockwise(to_device((A32, "f32"), dev), 1)
    qb, sb = gpu_blockwise(to_device((B32, "f32"), dev), 128)
    c = torch.full((total, N), float("nan"), dtype=torch.float32, device=dev)
    fm.fp8_grouped_gemm(qa, sa, qb.view(G, N, K), sb.view(G, N // 128, -1), torch.from_numpy(raw).to(dev), c,
                        accum=accum)
    torch.cuda.synchronize()
    got = f32(c)
    assert np.isnan(got[:20]).all() and np.isnan(got[550:]).all()
    qa_h, sa_h = u8(qa), f32(sa)
    qb_h = u8(qb).reshape(G, N, K)
    sb_h = f32(sb).reshape(G, N // 128, -1)
    rows = np.arange(20, 550)
    bound = None if accum == "exact" else grouped_mfma8_bound(qa_h, sa_h, qb_h, sb_h, eff, rows=rows)
    _check_grouped(got, qa_h, sa_h, qb_h, sb_h, eff, "f32", rows=rows, bound=bound)


def test_grouped_equal_scales_reduce_to_dense_gemm():
    """With every block scale equal, expert g's rows equal fp8_gemm of those rows.
    Codes are small integers (0..4) so every partial sum is exact in fp32 and
    both results must agree bit for bit."""
    dev = device()
    rng = np.random.default_rng(3)
    counts, K, N = [100, 156], 256, 256
    offs = np.array([0, 100, 256], dtype=np.int32)
    small = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0], dtype=np.uint8)   # 0, 1, 2, 3, 4, -1, -2
    qa = torch.from_numpy(small[rng.integers(0, small.size, size=(256, K))]).to(dev)
    qb = torch.from_numpy(small[rng.integers(0, small.size, size=(2, N, K))]).to(dev)
    sa = torch.full((256, 2), 0.125, device=dev)
    sb = torch.full((2, 2, 2), 0.5, device=dev)
    c = torch.empty((256, N), dtype=torch.float32, device=dev)
    fm.fp8_grouped_gemm(qa, sa, qb, sb, torch.from_numpy(offs).to(dev), c)
    for g in range(2):
        r0, r1 = offs[g], offs[g + 1]
        d = torch.empty((r1 - r0, N), dtype=torch.float32, device=dev)
        fm.fp8_gemm(qa[r0:r1].contiguous(), "e4m3", qb[g].contiguous(), "e4m3",
                    torch.tensor([0.125], device=dev), torch.tensor([0.5], device=dev), d)
        torch.cuda.synchronize()
        # both are exact here: small integer-valued partials times powers of two
        assert torch.equal(c[r0:r1], d)


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_moe_full_size_blockwise_and_sampled_grouped(accum):
    """8 experts, seeded token counts (multiples of 128 in [128, 4096], sum 16384),
    K=7168, N=4096; A per 1x128, W per 128x128, E4M3; bf16 out.  Quantisation is
    checked bit for bit per expert; the GEMM on sampled rows of every expert,
    within the method's per-block bound in both accumulation modes."""
    dev = device()
    d = moe_grouped()
    G, N, K = d["B"].shape
    A = to_device(d["A"], dev)
    announce("moe full size: blockwise A")
    qa, sa = gpu_blockwise(A, 1)
    Bd = to_device((d["B"].data.reshape(G * N, K), "bf16"), dev)
    announce("moe full size: blockwise B")
    qb, sb = gpu_blockwise(Bd, 128)
    offs = d["m_offsets"].astype(np.int32)
    c = torch.empty((int(offs[-1]), N), dtype=torch.bfloat16, device=dev)
    announce("moe full size: grouped gemm")
    fm.fp8_grouped_gemm(qa, sa, qb.view(G, N, K), sb.view(G, N // 128, K // 128), torch.from_numpy(offs).to(dev), c,
                        accum=accum)
    torch.cuda.synchronize()
    qa_h, sa_h, qb_h, sb_h = u8(qa), f32(sa), u8(qb).reshape(G, N, K), f32(sb).reshape(G, N // 128, K // 128)
    rng = np.random.default_rng(55)
    rows = []
    for g in range(G):
        rows += sorted(rng.choice(np.arange(offs[g], offs[g + 1]), size=4, replace=False).tolist())
        rows += [int(offs[g]), int(offs[g + 1]) - 1]
    rows = np.array(rows)
    x32 = scaling.widen(d["A"].data[rows], "bf16")
    wq, wsi = scaling.quantize_blockwise(x32, 1, 128)
    assert np.array_equal(qa_h[rows], wq) and np.array_equal(sa_h[rows].view(np.uint32), wsi.view(np.uint32))
    for g in (0, G - 1):
        w32 = scaling.widen(d["B"].data[g], "bf16")
        wq, wsi = scaling.quantize_blockwise(w32, 128, 128)
        assert np.array_equal(qb_h[g], wq) and np.array_equal(sb_h[g].view(np.uint32), wsi.view(np.uint32))
    _check_grouped(f32(c), qa_h, sa_h, qb_h, sb_h, offs, "bf16", rows=rows)

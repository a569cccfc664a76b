"""The oracle's FP8 encoder against an independent C encoder on all 2^32 fp32
bit patterns, both formats (CPU only).

``oracle.codec.encode`` rounds on the fp32 bit pattern with integer shifts;
``oracle/codec_ref.c`` searches a table of decoded FP8 values and compares with
exact midpoints.  They share no code.  The rule both implement (OCP E4M3 /
E5M2 of "4.2 Hopper I — Transformer Engine·FP8" §4.2.3 and §4.2.8; round to
nearest even, saturation, NaN -> sign|0x7F, the sign always kept) is pinned
on its own by tests/test_oracle_codec.py; here every input is compared.
The 2^33 encodings run in worker processes, about a minute and a half on 8 cores."""

import ctypes
import multiprocessing as mp
import os

import numpy as np
import pytest

from oracle import build_ref, codec

CHUNK = 1 << 23
FORMATS = {"e4m3": 0, "e5m2": 1}


def _c_encode_range(lib, which, start, count):
    out = np.empty(count, dtype=np.uint8)
    assert lib.fp8ref_encode_range(which, start, count, out.ctypes.data_as(ctypes.c_void_p)) == 0
    return out


def _compare_chunk(args):
    fmt, start = args
    lib = build_ref.load()
    bits = np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32)
    got = codec.encode(bits.view(np.float32), fmt)
    want = _c_encode_range(lib, FORMATS[fmt], start, CHUNK)
    bad = np.flatnonzero(got != want)
    if bad.size:
        i = bad[0]
        return int(bad.size), int(bits[i]), int(got[i]), int(want[i])
    return 0, 0, 0, 0


def test_c_encoder_facts():
    """The C encoder on values fixed by the formats (so that a broken C side
    cannot pass the exhaustive comparison by agreeing with a broken oracle
    only on the patterns below)."""
    lib = build_ref.load()

    def enc(vals, fmt):
        b = np.ascontiguousarray(np.asarray(vals, dtype=np.float32)).view(np.uint32)
        out = np.empty(b.size, dtype=np.uint8)
        assert lib.fp8ref_encode_bits(FORMATS[fmt], b.ctypes.data_as(ctypes.c_void_p), b.size,
                                      out.ctypes.data_as(ctypes.c_void_p)) == 0
        return list(out)

    inf, nan = np.float32(np.inf), np.float32(np.nan)
    assert enc([448, 464, 470, 1e9, inf, -inf], "e4m3") == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert enc([17, 19, 2.0 ** -10, 3 * 2.0 ** -10, -1e-30, -0.0, 0.0], "e4m3") == \
        [0x58, 0x5A, 0x00, 0x02, 0x80, 0x80, 0x00]
    assert enc([57344, 61440, inf, 19, 1.0, 2.0 ** -16, 2.0 ** -17], "e5m2") == \
        [0x7B, 0x7B, 0x7B, 0x4D, 0x3C, 0x01, 0x00]
    assert enc([nan, -nan], "e4m3") == [0x7F, 0xFF] and enc([nan], "e5m2") == [0x7F]
    # every finite code decodes to a value that encodes back to it (-0 included)
    for fmt in FORMATS:
        f = codec.FORMATS[fmt]
        codes = np.array([c for c in range(256) if (c & 0x7F) <= f.max_code], dtype=np.uint8)
        assert enc(codec.decode(codes, fmt).astype(np.float32), fmt) == list(codes)


@pytest.mark.timeout(1800)
def test_encoder_agrees_with_c_encoder_on_every_fp32_pattern():
    jobs = [(fmt, s) for fmt in FORMATS for s in range(0, 1 << 32, CHUNK)]
    build_ref.build(force=False)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with mp.get_context("fork").Pool(workers) as pool:
        results = pool.map(_compare_chunk, jobs, chunksize=1)
    bad = [(job, r) for job, r in zip(jobs, results) if r[0]]
    assert not bad, bad[:4]
    assert len(jobs) == 2 * (1 << 32) // CHUNK

"""Host-only replay of the workgroup-to-tile maps of the GEMM kernels
(fp8_precision_numerics_amd/csrc/gemm_tile.hpp `tile_coords`, grouped_gemm.hip
`grouped_tile`): every output tile is produced by exactly one workgroup, for
the band widths the dispatch uses and for ragged and empty experts, and the
workgroups the hardware deals to one XCD (id % 8) form the compact blocks the
bands are for."""

import random

import pytest


def tile_coords(pid, tiles_m, tiles_n, group_m):
    total = tiles_m * tiles_n
    if total % 8 == 0:
        pid = (pid & 7) * (total >> 3) + (pid >> 3)
    in_group = group_m * tiles_n
    gid = pid // in_group
    first_m = gid * group_m
    gsize = min(group_m, tiles_m - first_m)
    local = pid - gid * in_group
    return first_m + local % gsize, local // gsize


@pytest.mark.parametrize("tiles_m,tiles_n", [(32, 64), (1, 1), (3, 5), (32, 16), (64, 16), (7, 9), (4, 2), (33, 65)])
@pytest.mark.parametrize("group_m", [1, 4, 16])
def test_dense_map_is_a_bijection(tiles_m, tiles_n, group_m):
    seen = set()
    for pid in range(tiles_m * tiles_n):
        tm, tn = tile_coords(pid, tiles_m, tiles_n, group_m)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n


def test_dense_fc1_xcd_blocks_are_4_by_8():
    """FC1 (8192x16384 in 256x256 tiles, one workgroup per CU): the first 32
    workgroups dealt to each XCD cover a 4 x 8 block of tiles."""
    tiles_m, tiles_n = 32, 64
    for xcd in range(8):
        first = [tile_coords(8 * j + xcd, tiles_m, tiles_n, 4) for j in range(32)]
        rows = {tm for tm, _ in first}
        cols = {tn for _, tn in first}
        assert len(rows) == 4 and len(cols) == 8


def grouped_tile(offsets, total_m, BM, tiles_n, GM, wg):
    G = len(offsets) - 1
    if GM == 0:
        return wg // tiles_n, wg % tiles_n
    real_m, prev = 0, 0
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        lo = prev if lo < prev else min(lo, total_m)
        hi = lo if hi < lo else min(hi, total_m)
        prev = hi
        real_m += (hi - lo + BM - 1) // BM
    total = real_m * tiles_n
    per_xcd = (total + 7) >> 3
    j = wg >> 3
    if j >= per_xcd:
        return None
    pid = (wg & 7) * per_xcd + j
    if pid >= total:
        return None
    in_group = GM * tiles_n
    gid = pid // in_group
    first_m = gid * GM
    gsize = min(GM, real_m - first_m)
    local = pid - gid * in_group
    return first_m + local % gsize, local // gsize


def expert_tile(offsets, total_m, BM, mt):
    """(expert, first row, end row) of M tile mt, or None (as the kernels)."""
    acc, prev = 0, 0
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        lo = prev if lo < prev else min(lo, total_m)
        hi = lo if hi < lo else min(hi, total_m)
        prev = hi
        tiles = (hi - lo + BM - 1) // BM
        if mt < acc + tiles:
            return g, lo + (mt - acc) * BM, hi
        acc += tiles
    return None


def grid(total_m, G, N, BM, BN):
    tiles_n = (N + BN - 1) // BN
    tiles_m = (total_m + BM - 1) // BM + G
    return (tiles_m * tiles_n + 7) // 8 * 8, tiles_n


CASES = [[2816, 1664, 1664, 1664, 2432, 1664, 2560, 1920], [0, 300, 0, 129, 5000, 1], [128], [0, 0, 7],
         [1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1]]


@pytest.mark.parametrize("GM", [0, 4])
@pytest.mark.parametrize("BM,BN,N", [(128, 512, 4096), (128, 128, 4096), (128, 512, 700), (128, 128, 130)])
def test_grouped_map_covers_every_row_block_once(GM, BM, BN, N):
    rng = random.Random(5)
    cases = CASES + [[rng.choice([0, rng.randint(0, 3000), 128 * rng.randint(0, 20)]) for _ in range(rng.randint(1, 9))]
                     for _ in range(20)]
    for counts in cases:
        offsets = [0]
        for c in counts:
            offsets.append(offsets[-1] + c)
        total_m = offsets[-1]
        if total_m == 0:
            continue
        n_wg, tiles_n = grid(total_m, len(counts), N, BM, BN)
        covered = {}
        for wg in range(n_wg):
            t = grouped_tile(offsets, total_m, BM, tiles_n, GM, wg)
            if t is None:
                continue
            mt, tn = t
            e = expert_tile(offsets, total_m, BM, mt)
            if e is None:
                continue
            g, row0, row_end = e
            for r in range(row0, min(row0 + BM, row_end)):
                key = (r, tn)
                assert key not in covered, (counts, wg, key)
                covered[key] = wg
        assert len(covered) == total_m * tiles_n, counts


def test_grouped_banded_map_spreads_the_padding_tiles():
    """With the real tile count, every XCD gets the same number of tiles (+-1),
    where the grid's padding (one spare M tile per expert) would otherwise all
    fall on the last XCDs."""
    counts = [2048, 1280, 3072, 768, 2560, 1536, 2816, 2304]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    n_wg, tiles_n = grid(offsets[-1], len(counts), 4096, 128, 512)
    per = [0] * 8
    for wg in range(n_wg):
        if grouped_tile(offsets, offsets[-1], 128, tiles_n, 4, wg) is not None:
            per[wg & 7] += 1
    assert max(per) - min(per) <= 1

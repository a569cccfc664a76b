"""Host-only replay of the GEMM kernels' buffer-load address arithmetic.

The operand slabs, the MXFP8 block scales and the grouped GEMM's A block
scales are fetched with buffer loads (fp8_precision_numerics_amd/csrc/
gemm_kernel.hpp, SlabLoader and MxScaleLoader; grouped_gemm.hip).  The hardware range check compares the per-lane VGPR offset
(plus the instruction offset, 0 here) with the resource's byte count; the
scalar offset is added afterwards and is not checked.  A load whose VGPR
offset passes the check therefore touches [base + voff + soff, +size): this
test replays the kernels' offsets for edge tiles of every tile shape the
dispatch uses and asserts that each such access lies inside the operand, and
that every tile row inside the operand is actually fetched (so the fix did not
turn valid rows into zeros)."""

import itertools

import pytest

KBK = 128            # K bytes per main-loop step
U32_MAX = 0xFFFFFFFF


def lds_swz(row):
    return (row & 6) | ((row >> 3) & 1)


def slab_accesses(BM, BN, NW, rows_left_a, rows_left_b, K, kt):
    """(operand, tile_row, byte_start, size, checked_offset, num_records) of every
    direct-to-LDS load of step kt, as SlabLoader::issue forms them."""
    LQA, LQB = BM // 8 // NW, BN // 8 // NW
    out = []
    k0 = kt * KBK
    for w in range(NW):
        for lane in range(64):
            lrow = w * 8 + (lane >> 3)
            voff = lrow * K + (((lane & 7) ^ lds_swz(lrow)) & 7) * 16
            for d in range(LQA + LQB):
                if d < LQA:
                    op, q, rows_left = "A", d, rows_left_a
                else:
                    op, q, rows_left = "B", d - LQA, rows_left_b
                v = voff + q * NW * 8 * K          # VGPR operand
                s = k0                             # scalar operand
                assert v < 2 ** 31, "the VGPR offset must fit a signed 32-bit register"
                nrec = min(rows_left * K, U32_MAX)
                out.append((op, lrow + q * NW * 8, v + s, 16, v, nrec))
    return out


# (BM, BN, NW): dense exact, FP8 and MXFP8 FP8-core 256x256 / 8 waves; MXFP8
# exact 256x256 / 4 waves; small problems 128x128 / 4 waves; grouped FP8
# 128x512 / 8 waves; grouped exact 128x128 / 4 waves.
SHAPES = [(256, 256, 4), (256, 256, 8), (128, 128, 4), (128, 512, 8)]


# the largest K the entry points accept: dense 2^23 (256-row slabs; the
# 128 x 128 tiles serve dense problems too), grouped 2^22 (the 128 x 512 tile's
# 512-row B slab); the last row's offsets then come within 8 MiB of 2^31
K_MAX_DENSE, K_MAX_GROUPED = 1 << 23, 1 << 22


def _k_cases(BM, BN):
    return [128, 400, 4096, K_MAX_GROUPED if (BM, BN) == (128, 512) else K_MAX_DENSE]


@pytest.mark.parametrize("BM,BN,NW", SHAPES)
@pytest.mark.parametrize("kcase", range(4))
def test_slab_loads_stay_inside_the_operand(BM, BN, NW, kcase):
    K = _k_cases(BM, BN)[kcase]
    nfull = K // KBK
    for rows_a, rows_b in [(1, BN), (BM, 1), (BM - 1, BN - 7), (9, 17), (BM // 2 + 3, BN // 2 - 5),
                           (BM, BN), (8 * NW - 1, 8 * NW + 1)]:
        for kt in sorted({0, nfull - 1}):
            fetched = {"A": set(), "B": set()}
            for op, row, start, size, chk, nrec in slab_accesses(BM, BN, NW, rows_a, rows_b, K, kt):
                rows_left = rows_a if op == "A" else rows_b
                if chk + size > nrec:           # fails the range check: reads zero, touches nothing
                    assert row >= rows_left, (op, row, rows_left)
                    continue
                assert row < rows_left, (op, row, rows_left)
                assert 0 <= start and start + size <= rows_left * K, (op, row, start, rows_left * K)
                # the access stays inside its own row and inside the step's K slice
                assert start // K == row and kt * KBK <= start % K and start % K + size <= (kt + 1) * KBK
                fetched[op].add((row, start % K))
            for op, rows_left in (("A", rows_a), ("B", rows_b)):
                want = {(r, kt * KBK + g * 16) for r in range(min(rows_left, BM if op == "A" else BN))
                        for g in range(8)}
                assert fetched[op] == want, op


def test_old_scalar_row_offset_would_have_left_the_operand():
    """The form the loads had before (row group in the unchecked scalar offset)
    reads past the end of an exactly sized operand in an edge tile; kept as a
    record of why the offset moved."""
    BM, NW, K, rows_left = 256, 4, 256, 40
    bad = 0
    for w, lane, d in itertools.product(range(NW), range(64), range(BM // 8 // NW)):
        lrow = w * 8 + (lane >> 3)
        voff = lrow * K + (((lane & 7) ^ lds_swz(lrow)) & 7) * 16
        soff = d * NW * 8 * K
        if voff + 16 <= rows_left * K and voff + soff + 16 > rows_left * K:
            bad += 1
    assert bad > 0


def mx_scale_ld(rows):
    return (rows + 63) // 64 * 64


def mx_scale_pos(r):
    return (r & ~63) | ((r & 15) << 2) | ((r >> 4) & 3)


@pytest.mark.parametrize("M,N,K", [(320, 300, 256), (64, 1000, 128), (1100, 1030, 512), (256, 256, 384)])
def test_mx_scale_loads_stay_inside_the_scale_matrices(M, N, K):
    """MxScaleLoader (256x256 tiles, 8 waves): one dword per lane per step, the
    step's block offset in the VGPR operand.  Every dword that passes the check
    lies inside its scale matrix, and every (row < M, block) byte a tile needs is
    among the bytes fetched."""
    BM = BN = 256
    NW = 8
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    ld_a, ld_b = mx_scale_ld(M), mx_scale_ld(N)
    for tm, tn in itertools.product(range(tiles_m), range(tiles_n)):
        m0, n0 = tm * BM, tn * BN
        for kt in range(K // 128):
            got_a, got_b = set(), set()
            for w, lane in itertools.product(range(NW), range(64)):
                e = w * 64 + lane
                if w < BM // 64:
                    ld, base_row, idx, rows, got = ld_a, m0, e, M, got_a
                    area = BM
                else:
                    ld, base_row, idx, rows, got = ld_b, n0, e - BM, N, got_b
                    area = BN
                voff = (idx // (area // 4)) * ld + base_row + 4 * (idx % (area // 4)) + kt * 4 * ld
                nrec = (K // 32) * ld
                assert voff < 2 ** 31
                if voff + 4 > nrec:
                    continue
                assert voff + 4 <= nrec
                for b in range(4):
                    got.add(voff + b)
            for rows, ld, r0, got in ((M, ld_a, m0, got_a), (N, ld_b, n0, got_b)):
                for r in range(r0, min(rows, r0 + BM)):
                    for blk in range(4 * kt, 4 * kt + 4):
                        assert blk * ld + mx_scale_pos(r) in got, (r, blk)


def bt_lds_offset(BN, krow, col):
    return krow * BN + ((((col >> 4) ^ (krow & 7)) << 4) | (col & 15))


def bt_accesses(BN, NW, N, K, n0, kt, ragged):
    """(krow, col, byte_start, checked_offset, lds_offset) of every direct load of
    B stored [K x N] for step kt, as SlabLoader<.., BT=true> forms them."""
    RPB = 1024 // BN
    LQB = BN // 8 // NW
    out = []
    for w in range(NW):
        for lane in range(64):
            r = w * RPB + lane // (BN // 16)
            p = lane % (BN // 16)
            q = p ^ (r & 7)
            col = n0 + 16 * q
            voff_bt = r * N + col if col < N else 0x80000000
            for d in range(LQB):
                if ragged:
                    v = voff_bt + (d * NW * RPB + kt * KBK) * N
                    s = 0
                else:
                    v = voff_bt
                    s = (d * NW * RPB + kt * KBK) * N
                assert v < 2 ** 32 and s < 2 ** 31
                krow = d * NW * RPB + r                    # K row within the step
                lds = (w + d * NW) * 1024 + lane * 16      # byte offset in the stage's B area
                out.append((krow, col, v + s, v, lds, p))
    return out


@pytest.mark.parametrize("BN,NW", [(256, 4), (256, 8), (128, 4)])
@pytest.mark.parametrize("N,K", [(1040, 400), (256, 128), (16, 16), (528, 144), (2048, 4096),
                                 (256, (1 << 23) - 128)])   # K * N at the entry point's 2^31 - 1 limit
def test_bt_slab_loads_stay_inside_b_and_land_in_the_swizzled_layout(BN, NW, N, K):
    nrec = min(K * N, U32_MAX)
    nfull = K // KBK
    for n0 in range(0, N, BN):
        steps = [(kt, False) for kt in sorted({0, nfull - 1}) if kt >= 0 and nfull > 0]
        if K % KBK:
            steps.append((nfull, True))
        for kt, ragged in steps:
            fetched = set()
            for krow, col, start, chk, lds, p in bt_accesses(BN, NW, N, K, n0, kt, ragged):
                k = kt * KBK + krow
                if chk + 16 > nrec:
                    assert col >= N or k >= K, (krow, col)
                    continue
                assert col < N and k < K, (krow, col, k)
                assert start == k * N + col and start + 16 <= K * N
                assert lds == bt_lds_offset(BN, krow, col - n0)          # swizzled home of this granule
                fetched.add((krow, col))
            want = {(kr, c) for kr in range(min(KBK, K - kt * KBK)) for c in range(n0, min(n0 + BN, N), 16)}
            assert fetched == want


@pytest.mark.parametrize("BN", [128, 256])
def test_bt_transpose_reads_are_bank_conflict_free_and_select_the_right_values(BN):
    """The fragment reads of the [K x N] B tile: within each 16-lane group the
    sixteen 8-byte pieces hit 32 distinct LDS banks, and, under the measured
    lane layout of the transpose read, every lane receives the 8 K values of its
    own column in K order."""
    def tr8(addr_of_lane, lds):
        out = {}
        for g in range(4):
            for h in range(2):
                for c in range(8):
                    lane = 16 * g + 8 * h + c
                    out[lane] = [lds[addr_of_lane[16 * g + 2 * j + h] + c] for j in range(8)]
        return out

    # LDS contents: the (k, n) coordinates of each stored byte, in the BT layout
    lds = {}
    for k in range(KBK):
        for n in range(BN):
            lds[bt_lds_offset(BN, k, n)] = (k, n)
    for col0 in range(0, BN, 16):
        for krow0 in (0, 8, 64, 120):
            addr = {}
            for lane in range(64):
                jt, ht = (lane & 15) >> 1, lane & 1
                addr[lane] = bt_lds_offset(BN, krow0 + jt, col0 + 8 * ht)
            for g in range(4):
                banks = set()
                for L in range(16):
                    a = addr[16 * g + L]
                    banks.update({(a // 4) % 64, (a // 4 + 1) % 64})
                assert len(banks) == 32
            got = tr8(addr, lds)
            for lane, vals in got.items():
                assert vals == [(krow0 + j, col0 + (lane & 15)) for j in range(8)]


# ---------------------------------------------------------------------------
# Grouped GEMM A block scales (fp8_precision_numerics_amd/csrc/grouped_gemm.hip).
# sinv_a is [total_m][nk] fp32; a tile's buffer resource starts at its first row
# and covers its rows inside the expert, so a load that passes the range check
# stays inside them and rows past the expert read as zero.  Every offset is in
# the VGPR operand (the scalar one is 0).

GROUPED_TILE_ROWS = [1, 7, 16, 17, 63, 64, 65, 100, 127, 128]
GROUPED_NK = [1, 2, 3, 7, 8, 9, 10, 16, 17, 56]


@pytest.mark.parametrize("nk", GROUPED_NK)
def test_grouped_exact_scale_chunks_reach_every_step(nk):
    """Exact kernel (BM = 128, 4 waves): chunks of 8 steps in two LDS buffers of
    [128 rows][8] fp32.  The prologue loads chunk 0 (each wave 4 loads of 8 rows);
    step kt loads rows 16p .. 16p+15 of chunk kt/8 + 1 (p = kt % 8, waves 0 and 1)
    when that chunk exists; the stage barrier publishes them.  Replays the loads
    into an LDS model and checks that each step's read of row r gives
    sinv_a[r][kt], and that every access that passes the range check lies inside
    the tile's rows."""
    BM, SCH, NW = 128, 8, 4
    for tile_rows in GROUPED_TILE_ROWS:
        nrec = min(tile_rows * nk * 4, U32_MAX)
        lds = [[None] * (BM * SCH) for _ in range(2)]

        def load(chunk, rb):
            for lane in range(64):
                sa_lane = ((lane >> 3) * nk + (lane & 7)) * 4
                voff = sa_lane + (rb * nk + chunk * SCH) * 4
                assert 0 <= voff < 2 ** 31
                pos = rb * SCH + lane                       # M0 base + lane * 4 bytes
                if voff + 4 > nrec:
                    lds[chunk & 1][pos] = 0.0               # out of range: reads zero
                    continue
                row, k = divmod(voff // 4, nk)
                assert row < tile_rows                      # inside the tile's rows
                lds[chunk & 1][pos] = (row, k)

        for w in range(NW):
            for u in range(BM // 8 // NW):
                load(0, 8 * (w + u * NW))
        for kt in range(nk):
            for r in range(BM):
                v = lds[(kt // SCH) & 1][r * SCH + kt % SCH]
                if r < tile_rows:
                    assert v == (r, kt), (tile_rows, kt, r, v)
            if (kt // SCH + 1) * SCH < nk:
                for w in range(2):
                    load(kt // SCH + 1, (kt % SCH) * 16 + 8 * w)


@pytest.mark.parametrize("nk", GROUPED_NK)
def test_grouped_fp8_staggered_scale_groups_reach_every_step(nk):
    """FP8-core kernel (BM = 128, waves of 64 rows, FM = 4 blocks of 16 rows):
    lane (rr, hh) of block i holds step s + hh for the last s <= kt with
    s % 4 == i; step kt refreshes block kt % 4 with the load issued one step
    earlier (clamped to the last step at the end) and reads block i from lane
    rr + 16 * ((kt - i) % 4).  Checks that read against sinv_a[row][kt] for
    every row inside the expert, and the bounds of every load."""
    WTM, FM = 64, 4
    for tile_rows in GROUPED_TILE_ROWS:
        for wm in range(2):
            wave_rows = max(0, min(tile_rows - wm * WTM, WTM))
            nrec = wave_rows * nk * 4

            def load(blk, first):
                vals = {}
                for lane in range(64):
                    rr, hh = lane & 15, lane >> 4
                    k = min(max(first + hh, 0), nk - 1)
                    voff = ((blk * 16 + rr) * nk + k) * 4
                    assert 0 <= voff < 2 ** 31
                    if voff + 4 > nrec:
                        vals[lane] = 0.0
                        continue
                    row, kk = divmod(voff // 4, nk)
                    assert row < wave_rows and row == blk * 16 + rr and kk == k
                    vals[lane] = (row, kk)
                return vals

            sa_q = [load(i, i - 4) for i in range(FM)]
            sa_next = load(0, 0)                            # load_scales(0) in the prologue
            for kt in range(nk):
                sa_q[kt & 3] = sa_next
                for i in range(FM):
                    for rr in range(16):
                        row = i * 16 + rr
                        got = sa_q[i][rr + 16 * ((kt - i) & 3)]
                        if row < wave_rows:
                            assert got == (row, kt), (tile_rows, wm, kt, i, rr, got)
                nxt = min(kt + 1, nk - 1)
                sa_next = load(nxt & 3, nxt)


def test_grouped_scale_offsets_at_the_largest_k():
    """K = 2^22 (nk = 32768 steps): the largest VGPR offset either grouped kernel's
    A-scale loads form (last row of the tile, last chunk or group, last lane)
    stays a non-negative 32-bit value inside a full tile's resource."""
    nk = K_MAX_GROUPED // KBK
    # exact kernel: rows rb + (lane >> 3) < 128, steps chunk * 8 + (lane & 7)
    last_chunk = (nk - 1) // 8
    voff = ((63 >> 3) * nk + (63 & 7)) * 4 + (120 * nk + last_chunk * 8) * 4
    assert voff + 4 <= 128 * nk * 4 < 2 ** 31
    # FP8-core kernel: block 3, row 15 of the wave's 64 rows, step clamped to nk - 1
    voff = ((3 * 16 + 15) * nk + (nk - 1)) * 4
    assert voff + 4 <= 64 * nk * 4 < 2 ** 31

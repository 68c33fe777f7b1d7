"""Layout maps on the CPU: the TileLayout/SwizzleLayout evaluator against the
worked tables of the TIRx "Tensor Layout" page, and the kernels' own LDS and
register placements (evaluated by the same inline functions the device code
calls) against their layout descriptions."""
import os

import pytest

import tile_scheduled_dense_amd as tg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
M, LANE, WAVE, TLANE, TCOL = tg.AXIS_M, tg.AXIS_LANE, tg.AXIS_WAVE, tg.AXIS_TLANE, tg.AXIS_TCOL


def rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def test_tensor_core_tile_case_study():
    L = tg.make_layout((8, 16), [(8, 4, LANE), (2, 1, WAVE), (4, 1, LANE), (2, 1, M)],
                       replica=[(2, 4, WAVE)], offset={WAVE: 5})
    table = rows("tirx_tensor_core_tile.txt")
    assert len(table) == 6
    for i, j, flat, c0, c1, c2, c3, lane, warps, m in table:
        coords = tg.tg_layout_eval(L, (int(i), int(j)))
        assert len(coords) == 2                                  # replicated on two warps
        assert {c[LANE] for c in coords} == {int(lane)}
        assert {c[WAVE] for c in coords} == {int(w) for w in warps.split(",")}
        assert {c[M] for c in coords} == {int(m)}
        assert int(flat) == 16 * int(i) + int(j)


def test_tensor_core_tile_closed_form_everywhere():
    L = tg.make_layout((8, 16), [(8, 4, LANE), (2, 1, WAVE), (4, 1, LANE), (2, 1, M)],
                       replica=[(2, 4, WAVE)], offset={WAVE: 5})
    for i in range(8):
        for j in range(16):
            coords = tg.tg_layout_eval(L, (i, j))
            assert sorted(c[WAVE] for c in coords) == [j // 8 + 5, j // 8 + 9]
            assert all(c[LANE] == 4 * i + (j // 2) % 4 and c[M] == j % 2 for c in coords)


def test_tensor_memory_case_study():
    L = tg.make_layout((2, 128, 112), [(2, 112, TCOL), (128, 1, TLANE), (112, 1, TCOL)])
    for a, l, c, tlane, tcol in rows("tirx_tensor_memory.txt"):
        (coord,) = tg.tg_layout_eval(L, (int(a), int(l), int(c)))
        assert coord[TLANE] == int(tlane) and coord[TCOL] == int(tcol)


def test_two_swizzles_compose_in_order():
    # Swizzle(3,3,3) then Swizzle(3,2,6) on a (64, 64) 16-bit tile: chunk j//8 is
    # XORed with row bits 0..2 and then with row bits 3..4
    L = tg.make_layout((64, 64), [(64, 64, M), (64, 1, M)], swizzle=[(3, 3, 3), (3, 2, 6)])
    for i in range(64):
        for j in range(0, 64, 5):
            (coord,) = tg.tg_layout_eval(L, (i, j))
            assert coord[M] == 64 * i + 8 * ((j // 8) ^ (i % 8) ^ ((i // 8) % 4)) + j % 8


def test_swizzle_worked_example():
    L = tg.make_layout((8, 64), [(8, 64, M), (64, 1, M)], swizzle=(3, 3, 3))
    for i, addr, bank, bank0 in rows("tirx_swizzle_worked_example.txt"):
        (coord,) = tg.tg_layout_eval(L, (int(i), 0))
        assert coord[M] == int(addr)
        assert (coord[M] * 2 // 4) % 32 == int(bank)            # bank = floor(a*b/4) mod 32, b = 2
        assert (64 * int(i) * 2 // 4) % 32 == int(bank0)
    # the page's closed form over the whole tile
    for i in range(8):
        for j in range(64):
            (coord,) = tg.tg_layout_eval(L, (i, j))
            assert coord[M] == 64 * i + 8 * ((j // 8) ^ i) + j % 8


def test_admission_and_invalid():
    L = tg.make_layout((8, 16), [(8, 4, LANE), (2, 1, WAVE), (4, 1, LANE), (2, 1, M)])
    Lbad = tg.make_layout((8, 15), [(8, 4, LANE), (2, 1, WAVE), (4, 1, LANE), (2, 1, M)])
    with pytest.raises(ValueError):
        tg.tg_layout_eval(Lbad, (0, 0))                          # size 120 != 128: not admitted
    with pytest.raises(ValueError):
        tg.tg_layout_eval(L, (8, 0))
    # any shape of the same size is admitted: (4, 32) re-derives the components
    L2 = tg.make_layout((4, 32), [(8, 4, LANE), (2, 1, WAVE), (4, 1, LANE), (2, 1, M)])
    assert tg.tg_layout_eval(L2, (1, 0)) == tg.tg_layout_eval(L, (2, 0))


# Ring (bf16/fp16) block shapes as (id for the introspection calls, block_m,
# block_n, waves, MFMA edge); the thin strip blocks of the 256 x 256
# configuration have layout-only ids.
RING = [(tg.TG_CFG_256x256, 256, 256, 4, 16), (tg.LAYOUT_CFG_STRIP_N, 256, 64, 4, 16),
        (tg.LAYOUT_CFG_STRIP_M, 64, 256, 4, 16), (tg.TG_CFG_128x128, 128, 128, 4, 32),
        (tg.TG_CFG_64x64, 64, 64, 2, 32), (tg.TG_CFG_288x160, 288, 160, 4, 16)]
BK = 32
PLANNED = [r for r in RING if r[0] < 100] + [(tg.TG_CFG_F32_64x64, 64, 64, 4, 16)]


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", PLANNED)
def test_ring_shapes_match_plans(cfg, bm, bn, waves, mt):
    dt = "f32" if cfg == tg.TG_CFG_F32_64x64 else "bf16"
    info = tg.tile_gemm_plan(1, 1024, 1024, 1024, dt, config=cfg)
    assert (info["block_m"], info["block_n"], info["waves"], info["mfma_m"]) == (bm, bn, waves, mt)


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", PLANNED + RING[1:3])
@pytest.mark.parametrize("swz", [tg.SWZ_NONE, tg.SWZ_XOR])
def test_kernel_lds_placement_matches_layout(cfg, bm, bn, waves, mt, swz):
    # the address the kernel computes (same inline function as the device code)
    # equals the TileLayout + swizzle description, and is a bijection onto the tile
    for operand, kind in [(0, tg.LAYOUT_LDS_A), (1, tg.LAYOUT_LDS_B)]:
        if cfg == tg.TG_CFG_288x160 and operand == 1 and swz == tg.SWZ_XOR:
            continue        # no TIRx description (test_320_byte_b_rows below)
        L = tg.tile_gemm_describe_layout(cfg, swz, kind)
        rows_, cols_ = L.shape[0], L.shape[1]
        seen = set()
        for r in range(rows_):
            for c in range(cols_):
                (coord,) = tg.tg_layout_eval(L, (r, c))
                off = tg.tile_gemm_lds_offset(cfg, swz, operand, r, c)
                assert off == coord[M], (operand, r, c)
                seen.add(off)
        assert seen == set(range(rows_ * cols_))


# gfx950 LDS, 64 banks x 4 bytes.  128-bit reads were measured, not modelled:
# extra cycles per ds_read_b128 (rocprofv3 SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS,
# one kernel per pattern, 64-byte A rows of four 16-byte chunks, chunk index
# XORed with mask(row)) for the two MFMA operand lane patterns: 32x32x16 (lane
# l reads row l % 32, chunk l // 32) and 16x16x32 (row l % 16, chunk l // 16).
# No simple lane-grouping model reproduces the whole table.
A_MASKS = {
    "(r>>2)&3": lambda r: (r >> 2) & 3, "r&3": lambda r: r & 3, "(r>>1)&3": lambda r: (r >> 1) & 3,
    "(r>>3)&3": lambda r: (r >> 3) & 3, "((r>>2)^(r>>4))&3": lambda r: ((r >> 2) ^ (r >> 4)) & 3,
    "((r>>1)^(r>>3))&3": lambda r: ((r >> 1) ^ (r >> 3)) & 3, "(r^(r>>2))&3": lambda r: (r ^ (r >> 2)) & 3,
    "0": lambda r: 0,
}
MEASURED_B128_EXTRA_CYCLES = {
    32: {"(r>>2)&3": 0, "r&3": 12, "(r>>1)&3": 4, "(r>>3)&3": 0, "((r>>2)^(r>>4))&3": 4,
         "((r>>1)^(r>>3))&3": 4, "(r^(r>>2))&3": 0, "0": 12},
    16: {"(r>>2)&3": 4, "r&3": 4, "(r>>1)&3": 0, "(r>>3)&3": 4, "((r>>2)^(r>>4))&3": 4,
         "((r>>1)^(r>>3))&3": 4, "(r^(r>>2))&3": 4, "0": 4},
}


def a_mask_of(cfg, swz, bm):
    """The kernel's A swizzle as a function of the row, identified among the measured candidates."""
    phys = [tg.tile_gemm_lds_offset(cfg, swz, 0, r, 0) * 2 // 16 % 4 for r in range(bm)]
    names = [n for n, f in A_MASKS.items() if all(phys[r] == f(r) for r in range(bm))]
    assert len(names) >= 1, phys[:32]
    return names[0]


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", RING)
def test_ring_a_fragment_reads_conflict_free(cfg, bm, bn, waves, mt):
    assert MEASURED_B128_EXTRA_CYCLES[mt][a_mask_of(cfg, tg.SWZ_XOR, bm)] == 0
    assert MEASURED_B128_EXTRA_CYCLES[mt][a_mask_of(cfg, tg.SWZ_NONE, bm)] > 0     # the ablation conflicts
    # a fragment read delivers the lane's own 8 consecutive k as one 16-byte chunk
    groups = 64 // mt
    for s in range(BK // (8 * groups)):
        for lane in range(64):
            row, k0 = lane % mt, 8 * (groups * s + lane // mt)
            offs = [tg.tile_gemm_lds_offset(cfg, tg.SWZ_XOR, 0, row, k0 + e) for e in range(8)]
            assert offs == list(range(offs[0], offs[0] + 8)) and offs[0] % 8 == 0


def banks_distinct(byte_offsets, width):
    banks = []
    for b in byte_offsets:
        banks += [((b + 4 * w) // 4) % 64 for w in range(width // 4)]
    return len(set(banks)) == len(banks)


def b_transpose_bytes(cfg, swz, mt, wcol, j, s, half):
    # ds_read_b64_tr_b16 for the B operand: lane L = 16 g + i of a 16-lane group
    # supplies 4 consecutive n of one k row; 32x32x16: k = 16 s + 8 (g // 2) +
    # i // 4, n = wcol + 32 j + 16 (g % 2) + 4 (i % 4); 16x16x32: k = 32 s + 8 g +
    # i // 4, n = wcol + 16 j + 4 (i % 4); +4 rows for the second read
    out = []
    for L in range(64):
        g, i = L // 16, L % 16
        if mt == 32:
            k = 16 * s + 8 * (g // 2) + i // 4 + 4 * half
            n = wcol + 32 * j + 16 * (g % 2) + 4 * (i % 4)
        else:
            k = 32 * s + 8 * g + i // 4 + 4 * half
            n = wcol + 16 * j + 4 * (i % 4)
        out.append(2 * tg.tile_gemm_lds_offset(cfg, swz, 1, k, n))
    return out


# The transposing 64-bit read serves 32 lanes per cycle from 64 banks; this
# model agrees with the measured counters for the 256 x 256 B tile under both
# MFMA shapes (zero conflicts with the XOR placement).
@pytest.mark.parametrize("cfg,bm,bn,waves,mt", RING)
def test_ring_b_transpose_reads_conflict_free(cfg, bm, bn, waves, mt):
    placements = [(tg.SWZ_XOR, True), (tg.SWZ_NONE, False)]
    if cfg in PAD_CFGS:
        placements.append((tg.SWZ_PAD, False))
    for swz, expect in placements:
        for wcol in range(0, bn, mt):
            for s in range(BK // (512 // mt)):
                for half in (0, 1):
                    offs = b_transpose_bytes(cfg, swz, mt, wcol, 0, s, half)
                    # each 64-bit read returns 4 consecutive n of one k row
                    assert all(o % 8 == 0 for o in offs)
                    free = all(banks_distinct(offs[g:g + 32], 8) for g in (0, 32))
                    assert free == expect, (swz, wcol, s, half)


# pad_stride (OCANNL Stage paragraph): the row stride is the minor dimension
# rounded up by one 16-byte unit; the extents stay as they are and the padded
# slots are never addressed.  Built for the 256 x 256 tile and its strips.
PAD_CFGS = (tg.TG_CFG_256x256, tg.LAYOUT_CFG_STRIP_N, tg.LAYOUT_CFG_STRIP_M)


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", [r for r in RING if r[0] in PAD_CFGS])
def test_pad_stride_placement(cfg, bm, bn, waves, mt):
    for operand, kind, rows_, cols_ in [(0, tg.LAYOUT_LDS_A, bm, BK), (1, tg.LAYOUT_LDS_B, BK, bn)]:
        L = tg.tile_gemm_describe_layout(cfg, tg.SWZ_PAD, kind)
        pitch = cols_ + 8
        assert (L.shape[0], L.shape[1], L.n_swizzle) == (rows_, cols_, 0)
        assert (L.shard[0].extent, L.shard[0].stride, L.shard[1].stride) == (rows_, pitch, 1)
        seen = set()
        for r in range(rows_):
            for c in range(cols_):
                (coord,) = tg.tg_layout_eval(L, (r, c))
                off = tg.tile_gemm_lds_offset(cfg, tg.SWZ_PAD, operand, r, c)
                assert off == coord[M] == r * pitch + c
                seen.add(off)
        assert len(seen) == rows_ * cols_ and all(o % pitch < cols_ for o in seen)
    # the tiles built without it refuse it
    assert tg.tile_gemm_lds_offset(tg.TG_CFG_128x128, tg.SWZ_PAD, 0, 0, 0) == -1
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_describe_layout(tg.TG_CFG_64x64, tg.SWZ_PAD, tg.LAYOUT_LDS_A)


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", [r for r in RING if r[0] in PAD_CFGS and r[2] >= 256])
def test_pad_stride_b_reads_at_most_two_way(cfg, bm, bn, waves, mt):
    # no linear pitch separates the rows k and k + 8 one transposing read pairs
    # from rows k .. k + 3 (the XOR does): under the 32-lanes-per-cycle model the
    # pad_stride pitch leaves each bank at most twice per cycle
    worst = 0
    for wcol in range(0, bn, mt):
        for half in (0, 1):
            offs = b_transpose_bytes(cfg, tg.SWZ_PAD, mt, wcol, 0, 0, half)
            for g in (0, 32):
                banks = {}
                for b in offs[g:g + 32]:
                    for w in range(2):
                        bank = (b // 4 + w) % 64
                        banks[bank] = banks.get(bank, 0) + 1
                worst = max(worst, max(banks.values()))
    assert worst == 2


def test_320_byte_b_rows():
    """The 288 x 160 tile's B rows are 320 bytes (5 units of 64): row k starts on bank 16 k, so
    rows k .. k + 3 are apart already, and the 32-byte half XOR of bit 3 of k moves k + 8 off k's
    banks.  Its placement is a bijection of the 32 x 160 tile onto 32 rows of 160 elements, and it
    is no TIRx swizzle of the linear address (the row pitch is no power of two), so it has no
    layout description."""
    cfg = tg.TG_CFG_288x160
    seen = set()
    for k in range(BK):
        for n in range(160):
            off = tg.tile_gemm_lds_offset(cfg, tg.SWZ_XOR, 1, k, n)
            assert off // 160 == k and (off % 160) // 16 == (n // 16) ^ ((k >> 3) & 1) and off % 16 == n % 16
            seen.add(off)
    assert seen == set(range(BK * 160))
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_describe_layout(cfg, tg.SWZ_XOR, tg.LAYOUT_LDS_B)


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", [r for r in RING if r[0] != tg.TG_CFG_288x160])
def test_ring_copy_ownership(cfg, bm, bn, waves, mt):
    # every physical 16-byte chunk of the A tile is filled by exactly one
    # (copy instruction, wave, lane); a copy instruction fills 1 KiB, lane l
    # writing bytes 16 l .. 16 l + 15 of it, and one wave's copies are adjacent
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_COPY_A)
    owners = {}
    for r in range(bm):
        for p in range(BK * 2 // 16):
            (coord,) = tg.tg_layout_eval(L, (r, p))
            key = (coord[M], coord[WAVE], coord[LANE])
            assert key not in owners
            owners[key] = (r, p)
            byte = (r * BK * 2) + 16 * p
            per_wave = bm * BK * 2 // 1024 // waves
            assert 0 <= coord[M] < per_wave
            assert byte == (coord[WAVE] * per_wave + coord[M]) * 1024 + 16 * coord[LANE]
    assert len(owners) == bm * BK * 2 // 16


@pytest.mark.parametrize("cfg,bm,bn,waves,mt", PLANNED + RING[1:3])
def test_accumulator_layout_matches_epilogue(cfg, bm, bn, waves, mt):
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_ACC)
    seen = set()
    step = 1 if bm * bn <= 64 * 64 else 3
    for r in range(0, bm, 1):
        for c in range(0, bn, step):
            (coord,) = tg.tg_layout_eval(L, (r, c))
            wave, lane, slot = coord[WAVE], coord[LANE], coord[M]
            assert 0 <= wave < waves and 0 <= lane < 64
            assert tg.tile_gemm_acc_coord(cfg, wave, lane, slot) == (r, c)
            seen.add((wave, lane, slot))
    if step == 1:
        assert len(seen) == bm * bn


# ---- fp32 inputs on the ring tiles (K tile 16, 16x16x4 MFMAs) --------------------------
F32_RING = [(tg.LAYOUT_CFG_F32_256, 256, 256, 4, tg.TG_CFG_256x256),
            (tg.LAYOUT_CFG_F32_128, 128, 128, 4, tg.TG_CFG_128x128),
            (tg.LAYOUT_CFG_F32_STRIP_N, 256, 64, 4, tg.LAYOUT_CFG_STRIP_N),
            (tg.LAYOUT_CFG_F32_STRIP_M, 64, 256, 4, tg.LAYOUT_CFG_STRIP_M)]
BK32 = 16


@pytest.mark.parametrize("cfg,bm,bn,waves,cfg16", F32_RING)
@pytest.mark.parametrize("swz", [tg.SWZ_NONE, tg.SWZ_XOR])
def test_f32_ring_lds_placement_matches_layout(cfg, bm, bn, waves, cfg16, swz):
    for operand, kind, rows_, cols_ in [(0, tg.LAYOUT_LDS_A, bm, BK32), (1, tg.LAYOUT_LDS_B, BK32, bn)]:
        L = tg.tile_gemm_describe_layout(cfg, swz, kind)
        assert (L.shape[0], L.shape[1]) == (rows_, cols_)
        seen = set()
        for r in range(rows_):
            for c in range(cols_):
                (coord,) = tg.tg_layout_eval(L, (r, c))
                off = tg.tile_gemm_lds_offset(cfg, swz, operand, r, c)
                assert off == coord[M], (operand, r, c)
                seen.add(off)
        assert seen == set(range(rows_ * cols_))
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_describe_layout(cfg, tg.SWZ_PAD, tg.LAYOUT_LDS_A)


@pytest.mark.parametrize("cfg,bm,bn,waves,cfg16", F32_RING)
def test_f32_ring_a_tile_is_the_16bit_a_tile(cfg, bm, bn, waves, cfg16):
    # 64-byte rows either way: fp32 element (r, k) sits at the bytes of 16-bit element
    # (r, 2k) of the 16x16x32 tile, so the same ds_read_b128 lane pattern (row l % 16,
    # chunk l // 16) reads it, with the same measured conflict-free XOR; a lane's chunk
    # holds its 4 consecutive k
    for swz in (tg.SWZ_NONE, tg.SWZ_XOR):
        for r in range(bm):
            for k in range(BK32):
                byte = 4 * tg.tile_gemm_lds_offset(cfg, swz, 0, r, k)
                mask = ((r >> 1) & 3) if swz == tg.SWZ_XOR else 0
                assert byte == 64 * r + 16 * ((k // 4) ^ mask) + 4 * (k % 4)
                if cfg16 != tg.TG_CFG_128x128:     # (the 16-bit 128 x 128 tile takes 32x32x16 MFMAs)
                    assert byte == 2 * tg.tile_gemm_lds_offset(cfg16, swz, 0, r, 2 * k)
    assert MEASURED_B128_EXTRA_CYCLES[16]["(r>>1)&3"] == 0
    assert MEASURED_B128_EXTRA_CYCLES[16]["0"] > 0
    for lane in range(64):
        row, k0 = lane % 16, 4 * (lane // 16)
        offs = [tg.tile_gemm_lds_offset(cfg, tg.SWZ_XOR, 0, row, k0 + e) for e in range(4)]
        assert offs == list(range(offs[0], offs[0] + 4)) and offs[0] % 4 == 0


@pytest.mark.parametrize("cfg,bm,bn,waves,cfg16", F32_RING)
def test_f32_ring_b_reads_conflict_free(cfg, bm, bn, waves, cfg16):
    # MFMA step e's B operand: lane L = 16 g + i reads the 4 bytes of B[4 g + e][n0 + i]
    # (ds_read_b32, 64 lanes over the 64 banks at once).  The XOR of the 64-byte unit
    # with (k >> 2) & 3 = g sends the four lane groups to four distinct bank quarters;
    # row-major, all four land on the same 16 banks (four-way conflicts)
    for swz, expect in [(tg.SWZ_XOR, True), (tg.SWZ_NONE, False)]:
        for n0 in range(0, bn, 16):
            for e in range(4):
                offs = [4 * tg.tile_gemm_lds_offset(cfg, swz, 1, 4 * (L // 16) + e, n0 + L % 16) for L in range(64)]
                assert banks_distinct(offs, 4) == expect, (swz, n0, e)


@pytest.mark.parametrize("cfg,bm,bn,waves,cfg16", F32_RING)
def test_f32_ring_copies_and_accumulators(cfg, bm, bn, waves, cfg16):
    # the A copies own each 16-byte chunk once, as for the 16-bit tile; the accumulator
    # layout (16x16 MFMA output) is the epilogue's
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_COPY_A)
    owners = set()
    per_wave = bm * 64 // 1024 // waves
    for r in range(bm):
        for p in range(4):
            (coord,) = tg.tg_layout_eval(L, (r, p))
            assert (r * 64) + 16 * p == (coord[WAVE] * per_wave + coord[M]) * 1024 + 16 * coord[LANE]
            owners.add((coord[M], coord[WAVE], coord[LANE]))
    assert len(owners) == bm * 4
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_ACC)
    for r in range(0, bm, 3):
        for c in range(0, bn, 5):
            (coord,) = tg.tg_layout_eval(L, (r, c))
            assert tg.tile_gemm_acc_coord(cfg, coord[WAVE], coord[LANE], coord[M]) == (r, c)

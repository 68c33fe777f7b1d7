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


CONFIGS = [(tg.TG_CFG_256x256, "bf16"), (tg.TG_CFG_128x128, "bf16"), (tg.TG_CFG_64x64, "bf16"),
           (tg.TG_CFG_F32_64x64, "f32")]
RING = CONFIGS[:3]          # bf16/fp16 configurations: the direct-copy K ring


def dims(cfg, dt):
    info = tg.tile_gemm_plan(1, 1024, 1024, 1024, dt, config=cfg)
    return info["block_m"], info["block_n"], info["block_k"], info["waves"]


@pytest.mark.parametrize("cfg,dt", CONFIGS)
@pytest.mark.parametrize("swz", [tg.SWZ_NONE, tg.SWZ_XOR])
def test_kernel_lds_placement_matches_layout(cfg, dt, swz):
    # the address the kernel computes (same inline function as the device code)
    # equals the TileLayout + swizzle description, and is a bijection onto the tile
    for operand, kind in [(0, tg.LAYOUT_LDS_A), (1, tg.LAYOUT_LDS_B)]:
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


# gfx950 LDS, measured: 64 banks x 4 bytes; a 128-bit read serves 16 lanes per
# cycle, a 64-bit read 32 lanes, a 128-bit write 8 lanes.
def banks_distinct(byte_offsets, width):
    banks = []
    for b in byte_offsets:
        banks += [((b + 4 * w) // 4) % 64 for w in range(width // 4)]
    return len(set(banks)) == len(banks)


def a_fragment_bytes(cfg, swz, base, s):
    # 32x32x16 MFMA A operand: lane l holds row base + l % 32, k = 16 s + 8 (l // 32) .. + 7
    return [2 * tg.tile_gemm_lds_offset(cfg, swz, 0, base + l % 32, 16 * s + 8 * (l // 32)) for l in range(64)]


def b_transpose_bytes(cfg, swz, wcol, j, s, half):
    # ds_read_b64_tr_b16 for the B operand: lane L = 16 g + i supplies row
    # k = 16 s + 8 (g // 2) + i // 4 (+4 for the second read), columns
    # n = wcol + 32 j + 16 (g % 2) + 4 (i % 4) .. + 3
    out = []
    for L in range(64):
        g, i = L // 16, L % 16
        k = 16 * s + 8 * (g // 2) + i // 4 + 4 * half
        n = wcol + 32 * j + 16 * (g % 2) + 4 * (i % 4)
        out.append(2 * tg.tile_gemm_lds_offset(cfg, swz, 1, k, n))
    return out


@pytest.mark.parametrize("cfg,dt", RING)
def test_ring_a_fragment_reads_conflict_free(cfg, dt):
    bm, bn, bk, _ = dims(cfg, dt)
    for swz, expect in [(tg.SWZ_XOR, True), (tg.SWZ_NONE, False)]:
        for base in range(0, bm, 32):
            for s in range(bk // 16):
                offs = a_fragment_bytes(cfg, swz, base, s)
                free = all(banks_distinct(offs[g:g + 16], 16) for g in range(0, 64, 16))
                assert free == expect, (swz, base, s)


@pytest.mark.parametrize("cfg,dt", RING)
def test_ring_b_transpose_reads_conflict_free(cfg, dt):
    bm, bn, bk, waves = dims(cfg, dt)
    for swz, expect in [(tg.SWZ_XOR, True), (tg.SWZ_NONE, False)]:
        for wcol in range(0, bn, 32):
            for s in range(bk // 16):
                for half in (0, 1):
                    offs = b_transpose_bytes(cfg, swz, wcol, 0, s, half)
                    # each 64-bit read returns 4 consecutive n of one k row
                    assert all(o % 8 == 0 for o in offs)
                    free = all(banks_distinct(offs[g:g + 32], 8) for g in (0, 32))
                    assert free == expect, (swz, wcol, s, half)


@pytest.mark.parametrize("cfg,dt", RING)
def test_ring_copy_ownership(cfg, dt):
    # every physical 16-byte chunk of the A tile is filled by exactly one
    # (copy instruction, wave, lane); a copy instruction fills 1 KiB, lane l
    # writing bytes 16 l .. 16 l + 15 of it, and one wave's copies are adjacent
    bm, bn, bk, waves = dims(cfg, dt)
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_COPY_A)
    owners = {}
    for r in range(bm):
        for p in range(bk * 2 // 16):
            (coord,) = tg.tg_layout_eval(L, (r, p))
            key = (coord[M], coord[WAVE], coord[LANE])
            assert key not in owners
            owners[key] = (r, p)
            byte = (r * bk * 2) + 16 * p
            per_wave = bm * bk * 2 // 1024 // waves
            assert 0 <= coord[M] < per_wave
            assert byte == (coord[WAVE] * per_wave + coord[M]) * 1024 + 16 * coord[LANE]
    assert len(owners) == bm * bk * 2 // 16


@pytest.mark.parametrize("cfg,dt", CONFIGS)
def test_accumulator_layout_matches_epilogue(cfg, dt):
    bm, bn, bk, waves = dims(cfg, dt)
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

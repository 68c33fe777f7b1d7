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


def dims(cfg, dt):
    info = tg.tile_gemm_plan(1, 1024, 1024, 1024, dt, config=cfg)
    return info["block_m"], info["block_n"], info["block_k"], info["waves"]


@pytest.mark.parametrize("cfg,dt", CONFIGS)
@pytest.mark.parametrize("swz", [tg.SWZ_NONE, tg.SWZ_XOR])
def test_kernel_lds_placement_matches_layout(cfg, dt, swz):
    bm, bn, bk, _ = dims(cfg, dt)
    for operand, kind, rows_ in [(0, tg.LAYOUT_LDS_A, bm), (1, tg.LAYOUT_LDS_B, bn)]:
        L = tg.tile_gemm_describe_layout(cfg, swz, kind)
        seen = set()
        for r in range(rows_):
            for k in range(bk):
                (coord,) = tg.tg_layout_eval(L, (r, k))
                off = tg.tile_gemm_lds_offset(cfg, swz, operand, r, k)
                assert off == coord[M], (operand, r, k)
                seen.add(off)
        assert seen == set(range(rows_ * bk))                    # a bijection onto the tile


# Two LDS bank models for 16-byte accesses:
#  * the layout page's: 32 banks x 4 bytes, one 128-byte line per cycle, so the
#    8 lanes served together must use 8 distinct 16-byte bank groups;
#  * gfx950's 128-bit reads: 64 banks x 4 bytes, 16 lanes per cycle, so 16
#    consecutive lanes must use 16 distinct groups of a 256-byte line.
MODELS = {"32x4B/8 lanes": (8, 8), "64x4B/16 lanes": (16, 16)}


def conflict_free(byte_offsets, lanes_per_cycle, groups):
    for g in range(0, len(byte_offsets), lanes_per_cycle):
        units = [(b // 16) % groups for b in byte_offsets[g:g + lanes_per_cycle]]
        if len(set(units)) != len(units):
            return False
    return True


@pytest.mark.parametrize("cfg,dt", CONFIGS[:3])
@pytest.mark.parametrize("model", sorted(MODELS))
def test_fragment_reads_conflict_free_under_swizzle(cfg, dt, model):
    # 32x32x16 MFMA: lane l reads row (l % 32), chunk 2s + l // 32 of the A (or
    # transposed B) tile, for rows starting at any multiple of 32.
    lanes_per_cycle, groups = MODELS[model]
    bm, bn, bk, _ = dims(cfg, dt)
    for swz, expect_free in [(tg.SWZ_XOR, True), (tg.SWZ_NONE, False)]:
        for base in range(0, bm, 32):
            for s in range(4):
                offs = [2 * tg.tile_gemm_lds_offset(cfg, swz, 0, base + l % 32, 8 * (2 * s + l // 32))
                        for l in range(64)]
                assert conflict_free(offs, lanes_per_cycle, groups) == expect_free, (swz, base, s)


@pytest.mark.parametrize("cfg,dt", CONFIGS[:3])
@pytest.mark.parametrize("model", sorted(MODELS))
def test_a_copy_writes_conflict_free(cfg, dt, model):
    # 128-bit LDS writes are served 8 lanes (128 bytes) per cycle in both models
    groups = MODELS[model][1]
    L = tg.tile_gemm_describe_layout(cfg, 0, tg.LAYOUT_COPY_A)
    bm, bn, bk, waves = dims(cfg, dt)
    owner = {}
    for r in range(bm):
        for ch in range(8):
            (coord,) = tg.tg_layout_eval(L, (r, ch))
            owner[(coord[WAVE], coord[LANE], coord[M])] = (r, ch)
    assert len(owner) == bm * 8                                   # each chunk copied by one thread slot
    for (w, lane, q), (r, ch) in owner.items():
        if lane % 8:
            continue
        group = [owner[(w, lane + d, q)] for d in range(8)]
        offs = [2 * tg.tile_gemm_lds_offset(cfg, tg.SWZ_XOR, 0, rr, 8 * cc) for rr, cc in group]
        assert conflict_free(offs, 8, groups)


@pytest.mark.parametrize("cfg,dt", CONFIGS[:3])
@pytest.mark.parametrize("model", sorted(MODELS))
def test_b_copy_writes_conflict_free(cfg, dt, model):
    # loader lanes 8g..8g+7 take the squares kb = 0..7 of one column block nb and
    # write, for each column c of it, chunk kb of transposed-tile row nb*8 + c
    groups = MODELS[model][1]
    bm, bn, bk, waves = dims(cfg, dt)
    for nb in range(bn // 8):
        for c in range(8):
            offs = [2 * tg.tile_gemm_lds_offset(cfg, tg.SWZ_XOR, 1, nb * 8 + c, 8 * kb) for kb in range(8)]
            assert conflict_free(offs, 8, groups)


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

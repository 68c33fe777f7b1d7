"""The C ABI on the CPU: the library loads, exports what the header declares,
validates arguments before any device work and plans blocks as documented.
No kernel is launched here (there is no GPU in this container)."""
import ctypes
import os
import re

import pytest

import tile_scheduled_dense_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tile_gemm.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(tg.library_path())
    declared = header_functions()
    assert set(declared) == set(tg.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert tg.abi_version() == tg.ABI_VERSION == 11
    for s in range(6):
        assert tg.STATUS_NAMES[s] in tg.status_string(s)


FAKE = 0x10000  # never dereferenced: every case below fails validation or has no GPU


def call(batch=1, M=64, N=64, K=64, dtype=tg.TG_BF16, A=FAKE, lda=None, sA=0, B=FAKE * 64, ldb=None, sB=0,
         C=FAKE * 4096, ldc=None, sC=0, alpha=1.0, beta=0.0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tg.tile_gemm_status("tile_gemm_strided_batched", batch, M, N, K, dtype, A, lda, sA, B, ldb, sB,
                               C, ldc, sC, alpha, beta, 0)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-2), dict(K=-3), dict(batch=-1),
    dict(lda=63), dict(ldb=10), dict(ldc=63), dict(dtype=7),
    dict(A=0), dict(B=0), dict(C=0),
    dict(A=FAKE + 1), dict(C=FAKE * 4096 + 2),
    dict(sA=-1), dict(batch=2, sC=64 * 63),            # batch entries of C overlap
    dict(C=FAKE),                                      # C overlaps A
    dict(C=FAKE * 64 + 64),                            # C overlaps B
])
def test_invalid_arguments_rejected_without_device(kw):
    assert call(**kw) == tg.TG_ERR_INVALID_ARG


def test_empty_problems_are_ok_without_device():
    assert call(M=0) == tg.TG_OK
    assert call(N=0, ldb=1, ldc=1) == tg.TG_OK
    assert call(batch=0) == tg.TG_OK
    assert call(M=0, A=0, B=0, C=0) == tg.TG_OK


def test_no_gpu_is_unsupported():
    # valid arguments: the only failure left is the missing gfx950 device
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert call() == tg.TG_ERR_UNSUPPORTED
    assert call(K=0, lda=1) == tg.TG_ERR_UNSUPPORTED     # K == 0 still launches (C = beta*C)


def test_options_validation():
    info = tg.PlanInfo()
    lib = tg._lib()
    # shorter than the version-1 layout: rejected
    opt = tg.Options(tg.OPTIONS_V1_SIZE - 4, 0, 0, 0, 0)
    assert lib.tile_gemm_plan(1, 8, 8, 8, tg.TG_BF16, ctypes.byref(opt), ctypes.byref(info)) == tg.TG_ERR_INVALID_ARG
    # a version-1 sized struct: the split-K fields beyond it are not read
    opt = tg.Options(tg.OPTIONS_V1_SIZE, 0, 0, 0, 0, 4, None, 0)
    assert lib.tile_gemm_plan(1, 64, 64, 8192, tg.TG_BF16, ctypes.byref(opt), ctypes.byref(info)) == tg.TG_OK
    assert info.split_k == 1
    opt.struct_size = ctypes.sizeof(tg.Options)
    assert lib.tile_gemm_plan(1, 64, 64, 8192, tg.TG_BF16, ctypes.byref(opt), ctypes.byref(info)) == tg.TG_OK
    assert info.split_k == 4
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8, 8, 8, "bf16", pipeline_depth=3)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8, 8, 8, "f32", config=tg.TG_CFG_64x64)     # the 16-bit 64 x 64 ring tile
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8, 8, 8, "f32", config=tg.TG_CFG_288x160)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8, 8, 8, "bf16", config=tg.TG_CFG_F32_64x64)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8, 8, 8, "bf16", swizzle=5)


# Block classes of the five measured problems (pad-to-tile + partition).
@pytest.mark.parametrize("args,expect", [
    ((1, 67, 45, 53, "f32"), dict(config=tg.TG_CFG_F32_64x64, tiles_m=2, tiles_n=1, interior_blocks=0,
                                  fringe_blocks=2, k_tiles=2, k_tail=21, mfma_m=16, mfma_k=4)),
    ((1, 8192, 8192, 8192, "bf16"), dict(config=tg.TG_CFG_256x256, tiles_m=32, tiles_n=32, grid=1024, persistent=0,
                                         interior_blocks=1024, fringe_blocks=0, k_tiles=256, k_tail=0,
                                         lds_bytes=4 * 32768, pipeline_depth=4, strip_blocks=0,
                                         mfma_m=16, mfma_n=16, mfma_k=32)),
    # N = 32 * 256 + 1: the one-column tail goes to 32 strip blocks of 256 x 64
    ((1, 8191, 8193, 8190, "bf16"), dict(config=tg.TG_CFG_256x256, tiles_m=32, tiles_n=32, grid=1024 + 32,
                                         interior_blocks=31 * 32, fringe_blocks=32, strip_blocks=32,
                                         tail_n_splits=0, tail_m_splits=0, k_tiles=256, k_tail=30)),
    ((512, 257, 129, 1000, "f16"), dict(tiles_m=5, tiles_n=3, interior_blocks=8, fringe_blocks=7,
                                        grid=15 * 512, k_tiles=32, k_tail=8, lds_bytes=4 * 8192,
                                        mfma_m=32, mfma_k=16, strip_blocks=0)),
    ((1, 512, 512, 131072, "bf16"), dict(k_tiles=4096, k_tail=0, fringe_blocks=0)),
])
def test_plan_block_classes(args, expect):
    kw = {}
    if args[1] == 257:
        kw["config"] = tg.TG_CFG_64x64
    info = tg.tile_gemm_plan(*args, **kw)
    for k, v in expect.items():
        assert info[k] == v, (k, info)


def test_plan_depth_changes_lds_and_residency_only():
    plans = {d: tg.tile_gemm_plan(1, 1000, 1000, 1000, "bf16", config=tg.TG_CFG_128x128, pipeline_depth=d)
             for d in (1, 2, 4)}
    stage = 128 * 32 * 2 * 2
    # three workgroups per CU by registers; at depth 4 the LDS holds two
    assert {d: info["per_cu"] for d, info in plans.items()} == {1: 3, 2: 3, 4: 2}
    for d, info in plans.items():
        assert info["lds_bytes"] == d * stage
        assert {k: v for k, v in info.items() if k not in ("lds_bytes", "pipeline_depth", "per_cu")} == \
               {k: v for k, v in plans[1].items() if k not in ("lds_bytes", "pipeline_depth", "per_cu")}
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 64, "bf16", pipeline_depth=3)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 64, "bf16", pipeline_depth=2, swizzle=tg.SWZ_NONE)
    assert tg.tile_gemm_plan(1, 64, 64, 64, "f32")["pipeline_depth"] == 2


def test_split_k_plans():
    # forced: at most S slices of a multiple of block_k, the last one shorter
    info = tg.tile_gemm_plan(1, 512, 512, 131072, "bf16", config=tg.TG_CFG_128x128, split_k=16)
    assert (info["split_k"], info["k_slice"], info["grid"]) == (16, 8192, 16 * 16)
    assert info["workspace_bytes"] == 16 * 512 * 512 * 4
    info = tg.tile_gemm_plan(3, 100, 70, 1000, "f16", config=tg.TG_CFG_64x64, split_k=3)
    assert (info["split_k"], info["k_slice"]) == (3, 352)
    assert info["grid"] == 2 * 2 * 3 * 3 and info["workspace_bytes"] == 3 * 3 * 100 * 70 * 4
    info = tg.tile_gemm_plan(1, 64, 64, 40, "bf16", config=tg.TG_CFG_64x64, split_k=8)
    assert (info["split_k"], info["k_slice"]) == (2, 32)       # K = 40 has two K tiles
    assert tg.tile_gemm_plan(1, 64, 64, 32, "bf16", split_k=8)["split_k"] == 1
    assert tg.tile_gemm_plan(1, 64, 64, 0, "bf16", split_k=8)["split_k"] == 1
    assert tg.tile_gemm_plan(1, 64, 64, 8192, "bf16", split_k=1000)["split_k"] == 64
    # automatic: only for too few tiles, deep K, and with the workspace it asks for
    assert tg.tile_gemm_workspace_size(1, 8192, 8192, 8192, "bf16") == 0
    need = tg.tile_gemm_workspace_size(1, 512, 512, 131072, "bf16")
    assert need > 0
    assert tg.tile_gemm_plan(1, 512, 512, 131072, "bf16")["split_k"] == 1
    assert tg.tile_gemm_plan(1, 512, 512, 131072, "bf16", workspace=FAKE, workspace_bytes=need)["split_k"] > 1
    assert tg.tile_gemm_workspace_size(1, 512, 512, 131072, "bf16", split_k=1) == 0
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 8192, "f32", split_k=4)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 8192, "bf16", split_k=-2)
    # a forced split with no workspace is rejected before any device work
    st = tg.tile_gemm_status("tile_gemm_ex", 1, 64, 64, 8192, tg.TG_BF16, FAKE, 8192, 0, FAKE * 64, 64, 0,
                             FAKE * 4096, 64, 0, 1.0, 0.0, 0,
                             ctypes.byref(tg.Options(ctypes.sizeof(tg.Options), 0, 0, 0, 0, 4, None, 0)))
    assert st in (tg.TG_ERR_INVALID_ARG, tg.TG_ERR_UNSUPPORTED)


def test_lds_budget():
    # every configuration's two pipeline copies fit the 160 KiB LDS of a gfx950 CU
    for cfg, dt in [(1, "bf16"), (2, "bf16"), (3, "bf16"), (4, "f32")]:
        info = tg.tile_gemm_plan(1, 4096, 4096, 4096, dt, config=cfg)
        assert info["lds_bytes"] <= 160 * 1024


@pytest.mark.parametrize("M,N,strips", [
    (1000, 1000, dict(tiles_m=4, tiles_n=4, strip_blocks=0)),        # tails of 232: whole tiles
    (1000, 1025, dict(tiles_m=4, tiles_n=4, strip_blocks=4)),        # N tail of 1: one strip per tile row
    (1025, 1000, dict(tiles_m=4, tiles_n=4, strip_blocks=4)),        # M tail of 1: one strip per tile column
    (1025, 1025, dict(tiles_m=4, tiles_n=4, strip_blocks=4 + 5)),    # both, the corner in the M strip
    (1088, 1088, dict(tiles_m=4, tiles_n=4, strip_blocks=9)),        # tails of exactly 64
    (1089, 1089, dict(tiles_m=5, tiles_n=5, strip_blocks=0)),        # tails of 65: whole tiles
    (300, 200, dict(tiles_m=1, tiles_n=1, strip_blocks=1)),          # M tail of 44 beside one tile, N < 256
    (257, 129, dict(tiles_m=1, tiles_n=1, strip_blocks=1)),          # M strip beside a 256-row tile, N < 256
    (129, 257, dict(tiles_m=1, tiles_n=1, strip_blocks=1)),          # N strip beside a 256-column tile
    (200, 200, dict(tiles_m=1, tiles_n=1, strip_blocks=0)),          # no main tile to put a strip beside
])
def test_plan_thin_strips(M, N, strips):
    info = tg.tile_gemm_plan(3, M, N, 512, "bf16", config=tg.TG_CFG_256x256)
    for k, v in strips.items():
        assert info[k] == v, (k, info)
    assert info["grid"] == 3 * (info["tiles_m"] * info["tiles_n"] + info["strip_blocks"])
    # other configurations have no strips
    assert tg.tile_gemm_plan(1, M, N, 512, "bf16", config=tg.TG_CFG_128x128)["strip_blocks"] == 0


def test_plan_pack_a():
    # the remainder column of this shape is kept in the grid here (tail_gemm=1): the
    # A copy alone; test_plan_tail_gemm covers the two together
    big = dict(workspace=1 << 40, workspace_bytes=1 << 40, tail_gemm=1)
    args = (1, 8191, 8193, 8190, "bf16")
    ldp_bytes = -(-8191 * 8192 * 2 // 256) * 256
    # misaligned rows, many tile columns, workspace: repack
    p = tg.tile_gemm_plan(*args, plan_lda=8193, **big)
    assert p["pack_a"] == 1 and p["workspace_bytes"] == ldp_bytes and p["split_k"] == 1
    assert tg.tile_gemm_workspace_size(*args, plan_lda=8193, tail_gemm=1) == ldp_bytes
    # aligned rows (lda a multiple of 8, or unknown): no repack, no workspace wanted
    assert tg.tile_gemm_plan(*args, plan_lda=8192, **big)["pack_a"] == 0
    assert tg.tile_gemm_workspace_size(*args, plan_lda=8192, tail_gemm=1) == 0
    assert tg.tile_gemm_workspace_size(*args, tail_gemm=1) == 0
    # too small a workspace: the plain plan, but the size it wants is reported
    p = tg.tile_gemm_plan(*args, plan_lda=8193, workspace=1 << 20, workspace_bytes=ldp_bytes - 256, tail_gemm=1)
    assert p["pack_a"] == 0
    # never, and few tile columns (each A panel read by few workgroups)
    assert tg.tile_gemm_plan(*args, plan_lda=8193, pack_a=1, **big)["pack_a"] == 0
    assert tg.tile_gemm_plan(1, 8191, 1000, 8190, "bf16", plan_lda=8193, **big)["pack_a"] == 0
    # forced: only for the 16-bit 256 x 256 configuration without a split
    assert tg.tile_gemm_plan(1, 100, 100, 100, "bf16", config=tg.TG_CFG_256x256, pack_a=2)["pack_a"] == 1
    # with the tile left to the library, a forced repack takes that tile unsplit, whatever the shape
    # and workspace would choose otherwise
    for shape in [(1, 1024, 1024, 4096), (1, 2048, 2048, 8192), (1, 8192, 64, 8192), (3, 257, 129, 1000)]:
        p = tg.tile_gemm_plan(*shape, "bf16", pack_a=2, workspace=1 << 40, workspace_bytes=1 << 40)
        assert (p["config"], p["split_k"], p["pack_a"]) == (tg.TG_CFG_256x256, 1, 1), shape
    for kw in (dict(config=tg.TG_CFG_128x128), dict(config=tg.TG_CFG_256x256, split_k=4), dict(split_k=4)):
        with pytest.raises(tg.TileGemmError):
            tg.tile_gemm_plan(1, 512, 512, 4096, "bf16", pack_a=2, **kw)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 64, "f32", pack_a=2)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(*args, pack_a=3)


def test_plan_tail_gemm():
    """A thin remainder as a GEMM of its own, on request (tail_gemm=2)."""
    args = (1, 8191, 8193, 8190, "bf16")
    big = dict(workspace=1 << 40, workspace_bytes=1 << 40)
    tail_bytes = 8 * 8191 * 1 * 4 + 32            # 8 K slices of an 8191 x 1 partial, rounded to 256
    # never split (1): 32 strip blocks after the 1024 main tiles, no workspace
    p = tg.tile_gemm_plan(*args, tail_gemm=1, **big)
    assert (p["strip_blocks"], p["tail_n_splits"], p["tail_m_splits"], p["grid"]) == (32, 0, 0, 1056)
    assert tg.tile_gemm_workspace_size(*args, tail_gemm=1) == 0
    # split strips (3, and by default (0) here: the 1024 main tiles fill the GPU): 8 K slices of
    # each of the 32 strip blocks, partials 8 x 8191 x 1; whole strips without the workspace
    for t in (0, 3):
        p = tg.tile_gemm_plan(*args, tail_gemm=t, **big)
        assert (p["strip_blocks"], p["strip_splits"], p["grid"]) == (32, 8, 1024 + 8 * 32)
        assert tg.tile_gemm_workspace_size(*args, tail_gemm=t) == tail_bytes
        p = tg.tile_gemm_plan(*args, tail_gemm=t)
        assert (p["strip_blocks"], p["strip_splits"], p["grid"]) == (32, 1, 1056)
    # forced: 8 K slices of the one-column GEMM (about 1024 workgroups of 64 x 64)
    p = tg.tile_gemm_plan(*args, tail_gemm=2, **big)
    assert (p["strip_blocks"], p["tail_n_splits"], p["tail_m_splits"], p["grid"]) == (0, 8, 0, 1024)
    assert p["workspace_bytes"] == tail_bytes
    assert tg.tile_gemm_workspace_size(*args, tail_gemm=2) == tail_bytes
    # with the A copy: the copy first, the partials after it
    ldp_bytes = -(-8191 * 8192 * 2 // 256) * 256
    p = tg.tile_gemm_plan(*args, plan_lda=8193, tail_gemm=2, **big)
    assert p["pack_a"] == 1 and p["tail_n_splits"] == 8 and p["workspace_bytes"] == ldp_bytes + tail_bytes
    assert tg.tile_gemm_workspace_size(*args, plan_lda=8193, tail_gemm=2) == ldp_bytes + tail_bytes
    # no workspace for the partials: the remainder GEMM is not split
    p = tg.tile_gemm_plan(*args, tail_gemm=2)
    assert (p["strip_blocks"], p["tail_n_splits"], p["workspace_bytes"]) == (0, 1, 0)
    # both remainders, short K (no split), batches
    p = tg.tile_gemm_plan(2, 300, 257, 100, "bf16", config=tg.TG_CFG_256x256, tail_gemm=2)
    assert (p["strip_blocks"], p["tail_n_splits"], p["tail_m_splits"], p["grid"]) == (0, 1, 1, 2)
    # an M remainder (8193 rows), K deep enough for 8 slices of 1024
    p = tg.tile_gemm_plan(1, 8193, 8192, 8192, "bf16", tail_gemm=2, **big)
    assert (p["strip_blocks"], p["tail_n_splits"], p["tail_m_splits"]) == (0, 0, 8)
    # no thin remainder: nothing to do
    p = tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", tail_gemm=2, **big)
    assert (p["strip_blocks"], p["tail_n_splits"], p["tail_m_splits"]) == (0, 0, 0)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(*args, tail_gemm=4)


def test_plan_persistent():
    """Persistent workgroups, on request: a whole grid of interior 256 x 256 tiles of one problem."""
    on = dict(persistent=2)
    p = tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", **on)
    assert (p["persistent"], p["grid"], p["tiles_m"] * p["tiles_n"]) == (1, 256, 1024)
    p = tg.tile_gemm_plan(1, 6144, 6144, 384, "f16", **on)    # 576 tiles: two or three per workgroup
    assert (p["persistent"], p["grid"]) == (1, 256)
    # not by default; and each condition broken in turn
    for t in (0, 1):
        assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", persistent=t)["persistent"] == 0
    for args, kw in [((1, 8192, 8192, 8160, "bf16"), {}),       # K not a multiple of 128
                     ((1, 8192, 8192, 128, "bf16"), {}),        # fewer than 8 K tiles
                     ((1, 8192, 8200, 8192, "bf16"), {}),       # N not a multiple of 256 (strips)
                     ((1, 8191, 8192, 8192, "bf16"), {}),       # a fringe row
                     ((2, 4096, 4096, 4096, "bf16"), {}),       # a batch
                     ((1, 4096, 4096, 4096, "bf16"), {}),       # 256 tiles: one per workgroup
                     ((1, 8192, 8192, 8192, "bf16"), dict(pipeline_depth=2)),
                     ((1, 8192, 8192, 8192, "bf16"), dict(block_order=1)),
                     ((1, 8192, 8192, 8192, "bf16"), dict(config=tg.TG_CFG_128x128)),
                     ((1, 8192, 8192, 8192, "f32"), {})]:
        p = tg.tile_gemm_plan(*args, **kw, **on)
        assert p["persistent"] == 0, (args, kw)
    big = dict(workspace=1 << 40, workspace_bytes=1 << 40)
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", plan_lda=8193, **big, **on)["persistent"] == 0   # repack
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", persistent=3)


def _plan_status(*args, **kw):
    try:
        tg.tile_gemm_plan(*args, **kw)
        return tg.TG_OK
    except tg.TileGemmError as e:
        return e.status


def test_plan_fused_tail():
    """The tail leaves the plan as it is without it (but for persistent workgroups); the options it
    is not built for are refused; a plan query takes the modes without a bias pointer."""
    for shape in [(1, 8192, 8192, 8192, "bf16"), (1, 8191, 8193, 8190, "bf16"), (512, 257, 129, 1000, "f16"),
                  (1, 512, 512, 131072, "bf16"), (1, 67, 45, 53, "f32"), (1, 300, 2100, 1100, "bf16")]:
        for extra in ({}, dict(workspace=1 << 40, workspace_bytes=1 << 40), dict(tail_gemm=2),
                      dict(tail_gemm=2, workspace=1 << 40, workspace_bytes=1 << 40)):
            base = tg.tile_gemm_plan(*shape, plan_lda=shape[3] + 3, **extra)
            for kw in (dict(bias_mode=1), dict(bias_mode=2), dict(activation=1), dict(bias_mode=1, activation=2)):
                assert tg.tile_gemm_plan(*shape, plan_lda=shape[3] + 3, **extra, **kw) == base, (shape, extra, kw)
                assert tg.tile_gemm_workspace_size(*shape, plan_lda=shape[3] + 3, **kw,
                                                   tail_gemm=extra.get("tail_gemm", 0)) == \
                    tg.tile_gemm_workspace_size(*shape, plan_lda=shape[3] + 3, tail_gemm=extra.get("tail_gemm", 0))
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", config=tg.TG_CFG_256x256, split_k=1,
                             activation=2)["config"] == tg.TG_CFG_256x256
    # persistent workgroups are not built with the tail
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", persistent=2)["persistent"] == 1
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", persistent=2, bias_mode=1)["persistent"] == 0
    shape = (1, 1024, 1024, 1024, "bf16")
    assert _plan_status(*shape, pipeline_depth=2, activation=1) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(*shape, pipeline_depth=5, config=tg.TG_CFG_128x128, bias_mode=1) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(*shape, swizzle=1, activation=2) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(*shape, pipeline_depth=2, split_k=2, activation=1) == tg.TG_OK     # applied by the combine
    assert _plan_status(1, 64, 64, 32, "bf16", config=tg.TG_CFG_256x256, split_k=2, activation=1) == tg.TG_OK
    assert _plan_status(*shape, bias_mode=3) == tg.TG_ERR_INVALID_ARG
    assert _plan_status(*shape, activation=-1) == tg.TG_ERR_INVALID_ARG
    assert _plan_status(*shape, bias_mode=1, bias_stride=-1) == tg.TG_ERR_INVALID_ARG


def test_packed_b_ld_and_size():
    """Packed rows are a multiple of 16 bytes; the size is batch x K rows of them."""
    assert tg.tile_gemm_packed_b_ld(8193, "bf16") == 8200
    assert tg.tile_gemm_packed_b_ld(8192, "f16") == 8192
    assert tg.tile_gemm_packed_b_ld(45, "f32") == 48
    assert tg.tile_gemm_packed_b_ld(0, "bf16") == 8 and tg.tile_gemm_packed_b_ld(0, "f32") == 4
    assert tg.tile_gemm_packed_b_size(3, 100, 129, "f16") == 3 * 100 * 136 * 2
    assert tg.tile_gemm_packed_b_size(2, 53, 45, "f32") == 2 * 53 * 48 * 4
    assert tg.tile_gemm_packed_b_size(0, 53, 45, "f32") == 0
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_packed_b_ld(-1, "bf16")
    for args in [(-1, 4, 4, "bf16"), (1, -4, 4, "bf16"), (1, 4, -4, "bf16"), (1, 4, 4, 7)]:
        with pytest.raises(tg.TileGemmError):
            tg.tile_gemm_packed_b_size(*args)


def test_pack_b_argument_errors():
    """Rejected before any device work (placeholder addresses are never dereferenced)."""
    B, P = 0x10000000, 0x20000000
    K, N = 64, 100
    need = tg.tile_gemm_packed_b_size(1, K, N, "bf16")

    def st(batch=1, k=K, n=N, dt=tg.TG_BF16, b=B, ldb=N, sb=0, tr=0, p=P, pb=need):
        return tg.tile_gemm_status("tile_gemm_pack_b", batch, k, n, dt, b, ldb, sb, tr, p, pb, None)
    bad = tg.TG_ERR_INVALID_ARG
    assert st(b=None) == bad
    assert st(p=None) == bad
    assert st(p=P + 128) == bad                   # not 256-byte aligned
    assert st(pb=need - 1) == bad
    assert st(ldb=N - 1) == bad
    assert st(tr=1, ldb=K - 1) == bad             # the transposed source's rows hold K elements
    assert st(tr=2) == bad
    assert st(sb=-1) == bad
    assert st(batch=-1) == bad and st(k=-1) == bad and st(n=-1) == bad
    assert st(dt=9) == bad
    assert st(b=P + 256) == bad                   # B inside the packed buffer
    assert st(batch=0) == tg.TG_OK and st(k=0) == tg.TG_OK and st(n=0) == tg.TG_OK
    # valid arguments reach the device check; only where no GPU is visible (the placeholder
    # addresses must never reach a kernel)
    import torch
    if torch.cuda.device_count() == 0:
        assert st() == tg.TG_ERR_UNSUPPORTED


def test_plan_automatic_split_across_tiles():
    """Without a forced tile, each tile size is weighed with its own automatic split and the best
    fill of the 256 CUs wins (ties: the larger tile); the workloads keep their plans."""
    big = dict(workspace=1 << 40, workspace_bytes=1 << 40)
    cases = [((1, 1024, 1024, 4096, "bf16"), (tg.TG_CFG_128x128, 4, 256)),   # not 256x256 split 4 (64 blocks)
             ((1, 512, 2048, 2048, "bf16"), (tg.TG_CFG_64x64, 1, 256)),      # not 256x256 split 2 (32 blocks)
             ((1, 512, 512, 131072, "bf16"), (tg.TG_CFG_256x256, 64, 256)),  # a tie at 256: the larger tile
             ((1, 8192, 8192, 8192, "bf16"), (tg.TG_CFG_256x256, 1, 1024)),
             ((512, 257, 129, 1000, "f16"), (tg.TG_CFG_288x160, 1, 256)),   # two problems per workgroup
             ((1, 1000, 1000, 1000, "bf16"), (tg.TG_CFG_64x64, 1, 256)),
             ((1, 384, 4096, 4096, "bf16"), (tg.TG_CFG_128x128, 4, 384)),     # 512 slots for the smaller tiles
             ((1, 256, 256, 65536, "bf16"), (tg.TG_CFG_64x64, 32, 512)),
             # skinny: the 256 x 256 tile's padding would be mostly zeros
             ((1, 8192, 64, 8192, "bf16"), (tg.TG_CFG_64x64, 4, 512)),
             ((1, 64, 8192, 8192, "bf16"), (tg.TG_CFG_64x64, 4, 512)),
             ((1, 16384, 96, 4096, "bf16"), (tg.TG_CFG_128x128, 4, 512))]
    for shape, want in cases:
        p = tg.tile_gemm_plan(*shape, **big)
        assert (p["config"], p["split_k"], p["grid"]) == want, (shape, p)
    # a forced tile keeps its own split; without a workspace there is no split at all
    p = tg.tile_gemm_plan(1, 1024, 1024, 4096, "bf16", config=tg.TG_CFG_256x256, **big)
    assert (p["config"], p["split_k"]) == (tg.TG_CFG_256x256, 4)
    assert tg.tile_gemm_plan(1, 1024, 1024, 4096, "bf16")["split_k"] == 1
    assert tg.tile_gemm_workspace_size(1, 1024, 1024, 4096, "bf16") == 4 * 1024 * 1024 * 4
    assert tg.tile_gemm_workspace_size(1, 512, 2048, 2048, "bf16") == 0


def test_plan_single_round_of_256():
    """256 x 256 when its tiles fill at least half the CUs and 128 x 128 would need a second round."""
    for shape in [(1, 3000, 3000, 3000, "bf16"), (1, 3072, 3072, 3072, "bf16"), (1, 4096, 2560, 2048, "bf16"),
                  (1, 3840, 3840, 1024, "bf16"), (4, 1536, 1536, 1024, "bf16")]:
        assert tg.tile_gemm_plan(*shape)["config"] == tg.TG_CFG_256x256, shape
    for shape in [(1, 2048, 2048, 2048, "bf16"), (1, 4096, 2048, 2048, "bf16")]:    # one round of 128 x 128
        assert tg.tile_gemm_plan(*shape)["config"] == tg.TG_CFG_128x128, shape


def test_plan_placements():
    """swizzle codes: 0 default (XOR), 1 none, 2 pad_stride, 3 XOR; pad_stride only on the 256 x 256
    tile at depth 4, whose LDS copies then hold the padded rows (A 256 x 80 bytes = 20 KiB, B 32 x
    528 bytes in 17 KiB)."""
    base = tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16")
    assert base["swizzle"] == tg.SWZ_XOR == 3
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", swizzle=tg.SWZ_XOR) == base
    pad = tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16", swizzle=tg.SWZ_PAD)
    assert pad["swizzle"] == tg.SWZ_PAD and pad["lds_bytes"] == 4 * (20 + 17) * 1024
    assert {k: v for k, v in pad.items() if k not in ("swizzle", "lds_bytes")} == \
           {k: v for k, v in base.items() if k not in ("swizzle", "lds_bytes")}
    for kw in (dict(config=tg.TG_CFG_128x128), dict(pipeline_depth=2), dict(config=tg.TG_CFG_64x64)):
        assert _plan_status(1, 1024, 1024, 1024, "bf16", swizzle=tg.SWZ_PAD, **kw) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(1, 64, 64, 64, "f32", swizzle=tg.SWZ_PAD) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(1, 64, 64, 64, "bf16", swizzle=4) == tg.TG_ERR_INVALID_ARG


def noalloc(batch=1, M=512, N=512, K=8192, opt=None, A=FAKE, B=FAKE * 4096, C=FAKE * 65536 * 64):
    return tg.tile_gemm_status("tile_gemm_ex_noalloc", batch, M, N, K, tg.TG_BF16, A, K, M * K, B, N, K * N,
                               C, N, M * N, 1.0, 0.0, 0, ctypes.byref(opt) if opt is not None else None)


def test_noalloc_limits_checked_before_any_device():
    """tile_gemm_ex_noalloc refuses, with no device work, a call whose scratch need exceeds the
    library's array, and a caller workspace; a call that fits only lacks the GPU here."""
    assert tg.NOALLOC_SCRATCH_BYTES == 64 << 20
    # 32 planes of 1024 x 1024 fp32 = 128 MiB of split partials
    assert noalloc(M=1024, N=1024, opt=tg._options(split_k=32)) == tg.TG_ERR_SCRATCH_LIMIT
    # 64 planes of 512 x 512 = 64 MiB: fits
    import torch
    fits = tg.TG_OK if torch.cuda.is_available() else tg.TG_ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        assert noalloc(opt=tg._options(split_k=64)) == fits
        assert noalloc() == fits
    # a forced repack of a 16384 x 4099 A (134 MB) does not fit
    assert noalloc(M=16384, N=256, K=4099, opt=tg._options(pack_a=2)) == tg.TG_ERR_SCRATCH_LIMIT
    # a caller workspace, and argument errors, as tile_gemm_ex would report them
    assert noalloc(opt=tg._options(workspace=FAKE * 65536 * 1024, workspace_bytes=1 << 20)) == \
        tg.TG_ERR_INVALID_ARG
    assert noalloc(M=-1) == tg.TG_ERR_INVALID_ARG
    assert noalloc(M=0) == tg.TG_OK


def test_plan_one_block_per_small_problem():
    """Batched problems that fit one 288 x 160 tile, at least half of it output, take one block
    per problem; the batched workload 512 x (257 x 129 x 1000) is one such."""
    p = tg.tile_gemm_plan(512, 257, 129, 1000, "f16", persistent=1)
    assert (p["config"], p["block_m"], p["block_n"], p["tiles_m"], p["tiles_n"], p["grid"]) == \
           (tg.TG_CFG_288x160, 288, 160, 1, 1, 512)
    assert (p["interior_blocks"], p["fringe_blocks"], p["strip_blocks"], p["lds_bytes"], p["per_cu"]) == \
           (0, 1, 0, 4 * (18 + 10) * 1024, 1)
    assert (p["mfma_m"], p["mfma_k"], p["k_tiles"], p["k_tail"]) == (16, 32, 32, 8)
    # too few problems, too small a share of the tile, or too large: another tile
    assert tg.tile_gemm_plan(64, 257, 129, 1000, "f16")["config"] != tg.TG_CFG_288x160
    assert tg.tile_gemm_plan(512, 100, 100, 1000, "f16")["config"] != tg.TG_CFG_288x160
    assert tg.tile_gemm_plan(512, 300, 129, 1000, "f16")["config"] != tg.TG_CFG_288x160
    # depths 2 and 4 are built, and the none placement at depth 4
    for d in (2, 4):
        assert tg.tile_gemm_plan(8, 257, 129, 100, "bf16", config=tg.TG_CFG_288x160, pipeline_depth=d)["grid"] == 8
    assert _plan_status(8, 257, 129, 100, "bf16", config=tg.TG_CFG_288x160, pipeline_depth=1) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(8, 257, 129, 100, "bf16", config=tg.TG_CFG_288x160, swizzle=tg.SWZ_PAD) == \
        tg.TG_ERR_UNSUPPORTED
    assert _plan_status(8, 257, 129, 100, "f32", config=tg.TG_CFG_288x160) == tg.TG_ERR_UNSUPPORTED


def test_plan_two_problems_per_workgroup():
    """Single-block problems on the 288 x 160 tile in more than one round and at most two run two
    per workgroup (256 workgroups), unless persistent = 1 asks for the plain grid; the plan is
    otherwise the plain grid's."""
    c4 = (512, 257, 129, 1000, "f16")
    chained, plain = tg.tile_gemm_plan(*c4), tg.tile_gemm_plan(*c4, persistent=1)
    assert (chained["config"], chained["persistent"], chained["grid"]) == (tg.TG_CFG_288x160, 1, 256)
    assert (plain["persistent"], plain["grid"]) == (0, 512)
    assert {k: v for k, v in chained.items() if k not in ("persistent", "grid")} == \
           {k: v for k, v in plain.items() if k not in ("persistent", "grid")}
    assert tg.tile_gemm_plan(*c4, persistent=2)["persistent"] == 1
    assert tg.tile_gemm_plan(*c4, bias_mode=1, activation=2)["persistent"] == 1      # with the fused tail too
    assert tg.tile_gemm_plan(257, 257, 129, 1000, "bf16")["grid"] == 256
    # one round, more than two, fewer than four K tiles, another depth or placement: the plain grid
    for args, kw in [((256, 257, 129, 1000, "f16"), {}), ((513, 257, 129, 1000, "f16"), {}),
                     ((512, 257, 129, 96, "f16"), {}), (c4, dict(pipeline_depth=2)), (c4, dict(swizzle=tg.SWZ_NONE))]:
        p = tg.tile_gemm_plan(*args, **kw)
        assert p["config"] == tg.TG_CFG_288x160 and p["persistent"] == 0 and p["grid"] == args[0], (args, kw, p)


def test_plan_b_repack_and_split_strips():
    """The repack of B takes rows that are only 2-byte aligned (odd ldb) on plans with at least
    8 tile rows; the ragged workload's ldb = N + 5 (rows 4-byte aligned) is left in place.  Its
    32 strip blocks split into 8 K slices by default when the workspace holds them (the 1024 main
    tiles fill the GPU), and on request (tail_gemm = 3)."""
    args = (1, 8191, 8193, 8190, "bf16")
    a_bytes = -(-8191 * 8192 * 2 // 256) * 256
    b_bytes = -(-8190 * 8200 * 2 // 256) * 256
    s_bytes = -(-8 * 8191 * 1 * 4 // 256) * 256
    kw = dict(plan_lda=8193, plan_ldb=8198)
    assert tg.tile_gemm_workspace_size(*args, tail_gemm=1, **kw) == a_bytes
    assert tg.tile_gemm_workspace_size(*args, **kw) == a_bytes + s_bytes
    p = tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=1 << 40, tail_gemm=1, **kw)
    assert (p["pack_a"], p["pack_b"], p["strip_splits"], p["grid"]) == (1, 0, 1, 1024 + 32)
    p = tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=1 << 40, **kw)
    assert (p["pack_a"], p["pack_b"], p["strip_splits"], p["grid"]) == (1, 0, 8, 1024 + 8 * 32)
    # the A copy fits but not the strip partials after it: the strips stay whole
    p = tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=a_bytes, **kw)
    assert (p["pack_a"], p["strip_splits"], p["workspace_bytes"]) == (1, 1, a_bytes)
    # an odd ldb: B repacked after the A copy
    kw = dict(plan_lda=8193, plan_ldb=8197)
    n = tg.tile_gemm_workspace_size(*args, tail_gemm=1, **kw)
    assert n == a_bytes + b_bytes
    p = tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=n, tail_gemm=1, **kw)
    assert (p["pack_a"], p["pack_b"], p["workspace_bytes"]) == (1, 1, n)
    # forced (2) also for 4-byte aligned rows; never (1)
    assert tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=1 << 40, pack_b=2, plan_ldb=8198)["pack_b"] == 1
    assert tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=1 << 40, pack_b=1, plan_ldb=8197)["pack_b"] == 0
    # split strips on request, after both copies
    n = tg.tile_gemm_workspace_size(*args, tail_gemm=3, **kw)
    assert n == a_bytes + b_bytes + s_bytes
    p = tg.tile_gemm_plan(*args, workspace=1 << 40, workspace_bytes=n, tail_gemm=3, **kw)
    assert (p["pack_a"], p["pack_b"], p["strip_blocks"], p["strip_splits"], p["grid"]) == (1, 1, 32, 8, 1024 + 8 * 32)
    # few tile rows: no B copy
    assert tg.tile_gemm_plan(1, 1000, 8193, 8190, "bf16", workspace=1 << 40, workspace_bytes=1 << 40,
                             plan_ldb=8197)["pack_b"] == 0
    assert _plan_status(*args, pack_b=3) == tg.TG_ERR_INVALID_ARG
    assert _plan_status(*args, pack_b=2, config=tg.TG_CFG_128x128) == tg.TG_ERR_UNSUPPORTED
    assert _plan_status(*args, tail_gemm=4) == tg.TG_ERR_INVALID_ARG


def test_plan_strips_split_automatically_after_a_full_round():
    # tail_gemm 0 splits the thin strips along K when the main tiles fill a round of the GPU
    # (256 workgroups) and the workspace holds the partials; 1 keeps them whole; 3 always asks
    big_ws = dict(workspace=1 << 40, workspace_bytes=1 << 40)
    c3 = dict(plan_lda=8190 + 3, plan_ldb=8193 + 5)
    info = tg.tile_gemm_plan(1, 8191, 8193, 8190, "bf16", **c3, **big_ws)
    assert (info["strip_blocks"], info["strip_splits"]) == (32, 8), info
    assert tg.tile_gemm_plan(1, 8191, 8193, 8190, "bf16", tail_gemm=1, **c3, **big_ws)["strip_splits"] == 1
    assert tg.tile_gemm_plan(1, 8191, 8193, 8190, "bf16", **c3)["strip_splits"] == 1        # no workspace
    n0 = tg.tile_gemm_workspace_size(1, 8191, 8193, 8190, "bf16", tail_gemm=1, **c3)
    n1 = tg.tile_gemm_workspace_size(1, 8191, 8193, 8190, "bf16", **c3)
    assert n1 > n0                                                  # it asks for the partials too
    # strips beside a part-filled last round stay whole unless asked: 144 main tiles and 25
    # strips (3073^2), 576 main tiles (64 in the last round) and 49 strips (6145^2); 256 main
    # tiles (4097^2, a whole round): split
    for n in (3073, 6145):
        assert tg.tile_gemm_plan(1, n, n, 2048, "bf16", **big_ws)["strip_splits"] == 1, n
        assert tg.tile_gemm_plan(1, n, n, 2048, "bf16", tail_gemm=3, **big_ws)["strip_splits"] > 1, n
    assert tg.tile_gemm_plan(1, 4097, 4097, 2048, "bf16", **big_ws)["strip_splits"] > 1
    # 240 main tiles and 32 strips (3841 x 4097): more strips than free slots, split
    assert tg.tile_gemm_plan(1, 3841, 4097, 2048, "bf16", **big_ws)["strip_splits"] > 1


def test_plan_fp32_ring_tiles():
    # fp32 inputs on the LDS ring: 256 x 256 and 128 x 128 block tiles with 16x16x4 MFMAs and a
    # K tile of 16 (64-byte A rows), chosen by the 16-bit rule except that a part-filled round of
    # 256 x 256 tiles needs three quarters of the CUs (192 tiles, not 128); the register-staged
    # 64 x 64 tile for problems that fill the GPU with neither
    info = tg.tile_gemm_plan(1, 8192, 8192, 8192, "f32")
    assert (info["config"], info["block_m"], info["block_n"], info["block_k"]) == (tg.TG_CFG_256x256, 256, 256, 16)
    assert (info["mfma_m"], info["mfma_k"], info["grid"], info["k_tiles"]) == (16, 4, 1024, 512)
    assert (info["pipeline_depth"], info["lds_bytes"], info["per_cu"]) == (4, 4 * (16384 + 16384), 1)
    info = tg.tile_gemm_plan(1, 2048, 2048, 2048, "f32")
    assert (info["config"], info["block_k"], info["lds_bytes"], info["per_cu"]) == (tg.TG_CFG_128x128, 16,
                                                                                      4 * (8192 + 8192), 2)
    assert tg.tile_gemm_plan(1, 67, 45, 53, "f32")["config"] == tg.TG_CFG_F32_64x64
    # with a workspace, fp32 ring tiles split by the busiest CU's share of slices:
    # 576 tiles of 128 x 128 are 3 per CU, split 2 makes 2.5 and split 4 2.25
    big_ws = dict(workspace=1 << 40, workspace_bytes=1 << 40)
    for (M, N, K), split in [((3072, 3072, 3072), 4), ((3072, 3072, 1024), 2), ((3072, 3072, 800), 1),
                             ((2048, 2048, 2048), 1), ((2560, 2560, 2560), 1), ((8192, 8192, 8192), 1)]:
        info = tg.tile_gemm_plan(1, M, N, K, "f32", **big_ws)
        assert info["split_k"] == split, (M, N, K, info["config"], info["split_k"])
        assert tg.tile_gemm_plan(1, M, N, K, "f32")["split_k"] == 1
    assert tg.tile_gemm_plan(1, 3072, 3072, 3072, "bf16", **big_ws)["split_k"] == 1   # 16-bit: unchanged
    # 144, 169, 196 and 225 tiles of 256 x 256 in one part-filled round
    for n, cfg in [(3072, tg.TG_CFG_128x128), (3328, tg.TG_CFG_128x128), (3584, tg.TG_CFG_256x256),
                   (3840, tg.TG_CFG_256x256)]:
        assert tg.tile_gemm_plan(1, n, n, n, "f32")["config"] == cfg, n
        assert tg.tile_gemm_plan(1, n, n, n, "bf16")["config"] == tg.TG_CFG_256x256, n
    # ragged: thin strips beside the 256 x 256 tiles, as for 16-bit inputs
    info = tg.tile_gemm_plan(1, 8191, 8193, 8190, "f32")
    assert (info["config"], info["strip_blocks"], info["k_tail"]) == (tg.TG_CFG_256x256, 32, 8190 % 16)
    # depths: 2 or 4 on the 256 x 256 tile, 1, 2, 4 or 5 on the 128 x 128 tile
    for d in (2, 4):
        assert tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", config=tg.TG_CFG_256x256, pipeline_depth=d)["lds_bytes"] \
            == d * 32768
    for d in (1, 3, 5):
        with pytest.raises(tg.TileGemmError):
            tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", config=tg.TG_CFG_256x256, pipeline_depth=d)
    for d in (1, 2, 4, 5):
        assert tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", config=tg.TG_CFG_128x128,
                                 pipeline_depth=d)["lds_bytes"] == d * 16384
    # placements: XOR and none; pad_stride is a 16-bit ablation only
    assert tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", config=tg.TG_CFG_256x256, swizzle=tg.SWZ_NONE)["swizzle"] \
        == tg.SWZ_NONE
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", config=tg.TG_CFG_256x256, swizzle=tg.SWZ_PAD)
    # split-K on the ring tiles, forced and automatic (with the workspace it asks for)
    info = tg.tile_gemm_plan(1, 512, 512, 131072, "f32", config=tg.TG_CFG_256x256, split_k=64)
    assert (info["split_k"], info["k_slice"], info["grid"]) == (64, 2048, 4 * 64)
    need = tg.tile_gemm_workspace_size(1, 512, 512, 131072, "f32")
    assert need > 0
    info = tg.tile_gemm_plan(1, 512, 512, 131072, "f32", workspace=FAKE, workspace_bytes=need)
    assert info["split_k"] > 1 and info["config"] in (tg.TG_CFG_256x256, tg.TG_CFG_128x128)
    # the register-staged tile still has no split; the remainder GEMMs are 16-bit only;
    # the repacks and the persistent grid stay 16-bit
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 64, 64, 8192, "f32", config=tg.TG_CFG_F32_64x64, split_k=4)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 8191, 8193, 8190, "f32", tail_gemm=2)
    with pytest.raises(tg.TileGemmError):
        tg.tile_gemm_plan(1, 4096, 4096, 4096, "f32", pack_a=2)
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "f32", persistent=2)["persistent"] == 0

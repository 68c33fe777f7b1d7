"""fp32 inputs on the LDS ring (TG_CFG_256x256 and TG_CFG_128x128 with fp32 A and B).

The K tile is 16 (64-byte A rows, the 16-bit kernel's A tile byte for byte); a lane's
16-byte A chunk holds 4 consecutive k and element e feeds 16x16x4 MFMA step e, whose B
operand is one 4-byte read of row 4 g + e.  Checked against the fp64 oracle at the fp32
tolerance (1e-5 of sum |a||b|), bit for bit on integer inputs, and bitwise across the
schedule knobs and the pad-to-tile embedding.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, need_gpu, oracle_full, result_points
from tests.test_gpu_invariants import padded

pytestmark = pytest.mark.gpu

RING = [tg.TG_CFG_256x256, tg.TG_CFG_128x128]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(p, workspace=None, **opts):
    gp = GpuProblem(p)
    gp.reset_c()
    if workspace is not None:
        opts["workspace"] = workspace
    gp.run(**opts)
    out = gp.result()
    gp.check_guards()
    return out


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def workspace_for(p, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, **opts)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")


# shapes over every block kind of the two tiles: one element, a tile with a ragged K,
# interior and fringe tiles, the 256 x 256 tile's N and M strips (and their corner),
# K of one, two and many K tiles of 16
SHAPES = [(1, 1, 1), (17, 15, 16), (67, 45, 53), (256, 256, 64), (300, 520, 200), (513, 257, 130),
          (257, 129, 1000), (1000, 1025, 333), (1025, 1000, 17)]


@pytest.mark.parametrize("cfg", RING)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity_f32_ring(cfg, shape):
    M, N, K = shape
    p = workloads.custom("f32", M, N, K, lda_pad=1, ldb_pad=3, ldc_pad=2, alpha=1.5, beta=0.5, seed=M + N + K)
    info = tg.tile_gemm_plan(1, M, N, K, "f32", config=cfg)
    assert info["block_k"] == 16 and info["mfma_k"] == 4
    check_parity(p, run(p, config=cfg))


@pytest.mark.parametrize("cfg", RING)
@pytest.mark.parametrize("shape", [(67, 45, 53, 0, 0), (300, 520, 200, 3, 5), (513, 1031, 777, 1, 7)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f32_ring_integer_inputs_bit_exact(cfg, shape):
    M, N, K, pa, pb = shape
    p = workloads.custom("f32", M, N, K, lda_pad=pa, ldb_pad=pb, alpha=1.5, beta=0.5, dist="int", seed=M + K)
    assert 4 * K * 1.5 + 0.5 * p.c0_ilim < 2 ** 23
    ref, _ = oracle_full(p)
    assert np.array_equal(run(p, config=cfg), ref)


@pytest.mark.parametrize("cfg,variants", [
    (tg.TG_CFG_256x256, [dict(pipeline_depth=2), dict(swizzle=tg.SWZ_NONE), dict(block_order=1)]),
    (tg.TG_CFG_128x128, [dict(pipeline_depth=1), dict(pipeline_depth=2), dict(pipeline_depth=5),
                         dict(swizzle=tg.SWZ_NONE), dict(block_order=1)]),
])
def test_f32_ring_depth_swizzle_order_bitwise_invisible(cfg, variants):
    p = workloads.custom("f32", 531, 389, 333, lda_pad=1, ldb_pad=2, alpha=0.75, beta=-1.25, seed=3)
    ref = run(p, config=cfg)
    for opts in variants:
        assert np.array_equal(bits(run(p, config=cfg, **opts)), bits(ref)), opts


@pytest.mark.parametrize("cfg,tile", [(tg.TG_CFG_256x256, (256, 256, 16)), (tg.TG_CFG_128x128, (128, 128, 16))])
@pytest.mark.parametrize("shape", [(300, 333, 130), (67, 45, 53), (257, 129, 1000)], ids=str)
def test_f32_ring_ragged_equals_cropped_padded(cfg, tile, shape):
    M, N, K = shape
    p = workloads.custom("f32", M, N, K, batch=2, lda_pad=3, ldb_pad=1, ldc_pad=5, alpha=1.5, beta=0.5, seed=K)
    base = run(p, config=cfg)
    up = lambda x, t: -(-x // t) * t
    for Mp, Np, Kp in [(up(M, tile[0]), up(N, tile[1]), up(K, tile[2])),
                       (up(M, tile[0]) + tile[0], up(N, tile[1]), up(K, tile[2]) + 2 * tile[2])]:
        q = padded(p, Mp, Np, Kp)
        got = run(q, config=cfg)[:, :M, :N]
        assert np.array_equal(bits(got), bits(base)), (Mp, Np, Kp)


@pytest.mark.parametrize("cfg,M,N,K,S", [(tg.TG_CFG_256x256, 512, 300, 4100, 8),
                                         (tg.TG_CFG_128x128, 200, 150, 2600, 6)])
def test_f32_ring_split_equals_slices_folded_in_tree_order(cfg, M, N, K, S):
    alpha = 1.5
    p = workloads.custom("f32", M, N, K, lda_pad=3, ldb_pad=5, alpha=alpha, beta=0.0, name="split_tree_f32")
    plan = tg.tile_gemm_plan(1, M, N, K, "f32", config=cfg, split_k=S)
    S_eff, ks = plan["split_k"], plan["k_slice"]
    assert S_eff > 1 and ks % 16 == 0
    got = run(p, workspace=workspace_for(p, config=cfg, split_k=S), config=cfg, split_k=S)
    check_parity(p, got)
    gp = GpuProblem(p)
    parts = []
    for s in range(S_eff):
        k0, kl = s * ks, min(ks, K - s * ks)
        out = torch.zeros(M * N, dtype=torch.float32, device="cuda")
        tg.tile_gemm_ex(1, M, N, kl, "f32", gp.A.data_ptr() + 4 * k0, p.lda, 0,
                        gp.B.data_ptr() + 4 * k0 * p.ldb, p.ldb, 0, out, N, 0, 1.0, 0.0, None,
                        config=cfg, split_k=1)
        torch.cuda.synchronize()
        parts.append(out.cpu().numpy().astype(np.float32))
    v, w = list(parts), 1
    while w < S_eff:
        for i in range(0, S_eff, 2 * w):
            if i + w < S_eff:
                v[i] = (v[i] + v[i + w]).astype(np.float32)
        w *= 2
    ref = (np.float32(alpha) * v[0]).astype(np.float32).reshape(M, N)
    assert np.array_equal(bits(got[0].astype(np.float32)), bits(ref))


def test_f32_ring_split_strips():
    # the 256 x 256 tile's thin strips split along K (tail_gemm = 3), against the oracle
    M, N, K = 520, 513, 2100
    p = workloads.custom("f32", M, N, K, lda_pad=1, ldb_pad=3, alpha=1.25, beta=0.5, seed=11)
    ws = workspace_for(p, config=tg.TG_CFG_256x256, tail_gemm=3)
    got = run(p, workspace=ws, config=tg.TG_CFG_256x256, tail_gemm=3)
    check_parity(p, got)
    assert tg.tile_gemm_plan(1, M, N, K, "f32", config=tg.TG_CFG_256x256)["strip_blocks"] > 0
    # integer inputs: the split strips are exact too
    q = workloads.custom("f32", M, N, K, alpha=1.0, beta=1.0, dist="int", seed=5)
    ref, _ = oracle_full(q)
    assert np.array_equal(run(q, workspace=workspace_for(q, config=tg.TG_CFG_256x256, tail_gemm=3),
                              config=tg.TG_CFG_256x256, tail_gemm=3), ref)


def test_f32_ring_full_size_sampled():
    # 8192^3 fp32 on the default plan (the 256 x 256 ring tile): the whole last row and
    # column and 3000 random points against the oracle, each a K = 8192 dot product
    p = workloads.custom("f32", 8192, 8192, 8192, dist="uniform", seed=7, name="f32_8192")
    assert tg.tile_gemm_plan(1, 8192, 8192, 8192, "f32")["config"] == tg.TG_CFG_256x256
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run()
    pts = workloads.sample_points(p, 3000)
    got = np.zeros((1, p.M, p.N))
    vals = result_points(gp, pts)
    got[pts[:, 0], pts[:, 1], pts[:, 2]] = vals
    check_parity(p, got, points=pts)

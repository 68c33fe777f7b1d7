"""The in-call repack of B and thin strips split along K, on the GPU through the C ABI.

* repack of B (ldb not a multiple of 8): the same values in aligned rows, the same MFMA
  sequence, so C is bitwise the call without it (pack_b = 1), alone and with the A repack;
* strips split along K (tail_gemm = 3 with a workspace, or tail_gemm = 0 where the whole strips
  would run as a round of their own after the main tiles): the main tiles are bitwise those of
  the unsplit plan (tail_gemm = 1); the strip region is a regrouped k sum, within the stated
  tolerance of the oracle, and bit-exact on integer-valued inputs (every partial sum exact);
  thin N tails, thin M tails with the corner, batches, beta != 0 and the fused tail.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, need_gpu, oracle_points

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def run(p, bias=None, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, plan_ldb=p.ldb, **opts)
    ws = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, plan_ldb=p.ldb, workspace=ws,
                             **opts)
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, plan_lda=p.lda, plan_ldb=p.ldb, bias=bias, **opts)
    out = gp.result()
    gp.check_guards()
    return out, plan


@pytest.mark.parametrize("dt,M,N,K,batch,lda_pad,ldb_pad", [
    ("bf16", 2100, 1030, 700, 1, 0, 5), ("f16", 2100, 1030, 700, 2, 3, 1), ("bf16", 2048, 2048, 64, 1, 1, 3)])
def test_b_repack_is_bitwise_invisible(dt, M, N, K, batch, lda_pad, ldb_pad):
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=lda_pad, ldb_pad=ldb_pad, alpha=1.5, beta=0.5, seed=K)
    big = dict(config=tg.TG_CFG_256x256, tail_gemm=1)      # the repacks belong to the 256 x 256 tile
    got, plan = run(p, **big)
    assert plan["pack_b"] == 1 and plan["pack_a"] == (1 if lda_pad and plan["tiles_n"] >= 8 else 0)
    ref, ref_plan = run(p, pack_b=1, **big)
    assert ref_plan["pack_b"] == 0
    assert np.array_equal(bits(got), bits(ref))
    forced, fp = run(p, pack_b=2, pack_a=1, **big)
    assert fp["pack_b"] == 1 and fp["pack_a"] == 0
    assert np.array_equal(bits(forced), bits(ref))
    if M * N * K * batch <= 2e9:
        check_parity(p, got)


# Thin N tails, thin M tails (corner included), both, a batch.
STRIP_SHAPES = [(4096, 4097, 2048, 1), (4097, 4096, 2048, 1), (4097, 4097, 2048, 1), (2048, 2049, 2048, 4),
                (4097, 4097, 1100, 1)]


def strip_points(p):
    """Every output of the strip regions (the last row and column of each batch entry, for these
    one-wide tails) and random points elsewhere."""
    return workloads.sample_points(p, 500, seed=3)


@pytest.mark.parametrize("M,N,K,batch", STRIP_SHAPES, ids=str)
def test_split_strips(M, N, K, batch):
    p = workloads.custom("bf16", M, N, K, batch=batch, lda_pad=2, ldb_pad=1, alpha=1.5, beta=0.5, seed=M + K)
    got, plan = run(p, tail_gemm=3)
    assert plan["strip_blocks"] > 0 and plan["strip_splits"] > 1, plan
    ref, ref_plan = run(p, tail_gemm=1)
    assert ref_plan["strip_splits"] == 1
    m_main = plan["tiles_m"] * 256 if M % 256 <= 64 else M
    n_main = plan["tiles_n"] * 256 if N % 256 <= 64 else N
    assert np.array_equal(bits(got[:, :m_main, :n_main]), bits(ref[:, :m_main, :n_main]))   # main tiles untouched
    pts = strip_points(p)
    check_parity(p, got, points=pts)


@pytest.mark.parametrize("M,N,K", [(4097, 4097, 2048), (4096, 4097, 4096)], ids=str)
def test_automatic_strip_split(M, N, K):
    """tail_gemm 0 with the workspace it asks for: the strips after a whole round of 256 main
    tiles are split along K by themselves; the main tiles are bitwise the whole-strip plan's."""
    p = workloads.custom("bf16", M, N, K, lda_pad=2, ldb_pad=1, alpha=1.5, beta=0.5, seed=M + K)
    got, plan = run(p)
    assert plan["strip_blocks"] > 0 and plan["strip_splits"] > 1, plan
    ref, ref_plan = run(p, tail_gemm=1)
    assert ref_plan["strip_splits"] == 1
    n_main = plan["tiles_n"] * 256
    m_main = plan["tiles_m"] * 256 if M % 256 else M
    assert np.array_equal(bits(got[:, :m_main, :n_main]), bits(ref[:, :m_main, :n_main]))
    check_parity(p, got, points=strip_points(p))


@pytest.mark.parametrize("M,N,K,batch", STRIP_SHAPES[:4], ids=str)
def test_split_strips_integer_exact(M, N, K, batch):
    p = workloads.custom("bf16", M, N, K, batch=batch, lda_pad=2, ldb_pad=1, alpha=1.5, beta=0.5, dist="int",
                         seed=M + K)
    got, plan = run(p, tail_gemm=3)
    assert plan["strip_splits"] > 1
    pts = strip_points(p)
    ref, _ = oracle_points(p, pts)
    assert np.array_equal(got[pts[:, 0], pts[:, 1], pts[:, 2]], ref)


@pytest.mark.parametrize("mode,act", [(1, 2), (2, 1)])
def test_split_strips_fused_tail(mode, act):
    import oracle
    p = workloads.custom("f16", 4097, 4097, 1200, lda_pad=0, ldb_pad=3, alpha=1.0, beta=0.5, seed=5)
    length = p.N if mode == 1 else p.M
    bias_np = (np.random.default_rng(3).standard_normal(length) * 10).astype(np.float32)
    bias = torch.from_numpy(bias_np).cuda()
    got, plan = run(p, bias=bias, bias_mode=mode, activation=act, tail_gemm=3)
    assert plan["strip_splits"] > 1
    pts = strip_points(p)
    ref, den = oracle.gemm_points(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, pts, C0=p.C0, ldc=p.ldc,
                                  alpha=p.alpha, beta=p.beta, bias=bias_np, bias_stride=0, bias_mode=mode,
                                  activation=act)
    c0 = p.C0[pts[:, 1] * p.ldc + pts[:, 2]].astype(np.float64)
    bv = bias_np[pts[:, 2]] if mode == 1 else bias_np[pts[:, 1]]
    den = den + np.abs(p.beta * c0) + np.abs(bv.astype(np.float64))
    g = got[pts[:, 0], pts[:, 1], pts[:, 2]]
    err = float(np.max(np.abs(g - ref) / (den + 1e-30)))
    assert err <= 4e-3, err

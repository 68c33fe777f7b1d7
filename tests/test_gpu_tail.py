"""Thin remainders computed by a GEMM of their own (tile_gemm.h, tail_gemm), on the GPU.

* forced (tail_gemm=2) on problems with an N remainder, an M remainder or both,
  split along K or not, on the repacked A, batched: parity with the fp64
  oracle over the whole output, and no write outside C;
* the main tiles are the same launch either way: outside the remainder rows and
  columns the result equals the strip plan's (tail_gemm=1) bit for bit;
* full size: 8193 x 8192 x 8192 (a one-row M remainder after 1024 main
  tiles), sampled inside and outside the remainder.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import (GpuProblem, check_parity, need_gpu, oracle_points, parity_error,
                            parity_error_rounded, result_points)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(p, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, **opts)
    ws = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, plan_lda=p.lda, **opts)
    out = gp.result()
    gp.check_guards()
    return out


TAIL_CASES = [
    # dtype, M, N, K, batch, lda_pad, ldb_pad, alpha, beta, expected (tail_n_splits, tail_m_splits, pack_a)
    ("bf16", 300, 257, 100, 1, 0, 3, 1.0, 0.0, (1, 1, 0)),        # both remainders, short K
    ("bf16", 520, 300, 2100, 1, 0, 5, 1.5, 0.5, (4, 4, 0)),       # both, split along K
    ("f16", 257, 1000, 1300, 1, 0, 0, -0.75, 1.0, (0, 2, 0)),     # one-row M remainder, split
    ("bf16", 300, 2100, 1100, 1, 3, 2, 1.0, 0.5, (2, 2, 1)),      # on the repacked A
    ("f16", 290, 260, 64, 2, 0, 1, 1.0, 0.0, (1, 1, 0)),          # batched
]


@pytest.mark.parametrize("dt,M,N,K,batch,lpad,bpad,alpha,beta,expect", TAIL_CASES,
                         ids=lambda v: str(v) if not isinstance(v, tuple) else "x".join(map(str, v)))
def test_tail_gemm_parity(dt, M, N, K, batch, lpad, bpad, alpha, beta, expect):
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=lpad, ldb_pad=bpad, alpha=alpha, beta=beta,
                         seed=M + N + K, name="tail")
    cfg = dict(config=tg.TG_CFG_256x256, split_k=1)   # the main problem unsplit
    plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, tail_gemm=2, workspace=1 << 40,
                             workspace_bytes=1 << 40, **cfg)
    assert (plan["tail_n_splits"], plan["tail_m_splits"], plan["pack_a"]) == expect, plan
    assert plan["strip_blocks"] == 0
    tail = run(p, tail_gemm=2, **cfg)
    check_parity(p, tail)
    strips = run(p, tail_gemm=1, **cfg)
    check_parity(p, strips)
    # the main tiles: the same kernel, the same MFMA sequence
    m_main = M // 256 * 256 if expect[1] else M
    n_main = N // 256 * 256 if expect[0] else N
    a = tail[:, :m_main, :n_main].astype(np.float32).view(np.uint32)
    b = strips[:, :m_main, :n_main].astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(a, b)


def test_full_size_m_remainder_sampled():
    # 8193 x 8192 x 8192: 1024 main tiles, the last row a GEMM of its own in 8 K slices
    p = workloads.custom("bf16", 8193, 8192, 8192, alpha=1.5, beta=0.5, seed=7, name="mtail")
    plan = tg.tile_gemm_plan(1, p.M, p.N, p.K, p.dtype, workspace=1 << 40, workspace_bytes=1 << 40, tail_gemm=2)
    assert (plan["strip_blocks"], plan["tail_n_splits"], plan["tail_m_splits"], plan["grid"]) == (0, 0, 8, 1024)
    n = tg.tile_gemm_workspace_size(1, p.M, p.N, p.K, p.dtype, tail_gemm=2)
    ws = torch.empty(n // 4 + 4, dtype=torch.float32, device="cuda")
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, tail_gemm=2)
    rng = np.random.default_rng(3)
    tail_pts = np.stack([np.zeros(64, np.int64), np.full(64, 8192), rng.integers(0, 8192, 64)], axis=1)
    pts = np.concatenate([tail_pts, workloads.sample_points(p, 200)])
    got = result_points(gp, pts)
    ref, den = oracle_points(p, pts)
    c0 = p.C0[pts[:, 1] * p.ldc + pts[:, 2]].astype(np.float64)
    err = parity_error_rounded(got, ref, den, p.beta, c0)
    print(f"8193 x 8192 x 8192: sampled parity error {err:.3e} over {len(pts)} outputs")
    assert err <= 4e-3
    gp.check_guards()

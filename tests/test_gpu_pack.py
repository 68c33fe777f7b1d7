"""Repack of A into aligned rows (tile_gemm.h, pack_a), on the GPU through the C ABI.

* a repacked call equals the plain call on the same problem bit for bit: the
  copy holds the same values and the GEMM runs the same MFMA sequence;
* parity with the fp64 oracle (ragged, batched, beta != 0), and on the full
  8191 x 8193 x 8190 workload with its automatic repack, at sampled outputs;
* the workspace contract: a forced repack without enough workspace, an
  overlapping workspace, and repacks of other configurations are rejected.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import (GpuProblem, c0_at, check_parity, need_gpu, oracle_points, parity_error,
                            parity_error_rounded, result_points)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def workspace_for(p, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, **opts)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda"), n


def run(p, ws=None, **opts):
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, **opts)
    out = gp.result()
    gp.check_guards()
    return out


PACK_CASES = [
    # dtype, M, N, K, batch, lda_pad, alpha, beta: lda = K + lda_pad is not a multiple of 8
    ("bf16", 300, 2100, 700, 1, 3, 1.0, 0.0),
    ("f16", 513, 2049, 129, 2, 1, 1.5, 0.5),
    ("bf16", 257, 2304, 1000, 1, 5, -0.75, 1.0),
    ("bf16", 40, 2090, 33, 3, 6, 1.0, 0.5),
]


@pytest.mark.parametrize("dt,M,N,K,batch,pad,alpha,beta", PACK_CASES)
def test_pack_bitwise_and_parity(dt, M, N, K, batch, pad, alpha, beta):
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=pad, ldb_pad=2, alpha=alpha, beta=beta,
                         seed=M + K, name="pack")
    opts = dict(config=tg.TG_CFG_256x256)
    plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, workspace=1 << 40,
                             workspace_bytes=1 << 40, **opts)
    assert plan["pack_a"] == 1 and plan["tiles_n"] >= 8
    ws, n = workspace_for(p, **opts)
    assert n == -(-p.batch * p.M * (-(-p.K // 8) * 8) * 2 // 256) * 256
    packed = run(p, ws, **opts)
    plain = run(p, None, pack_a=1, **opts)
    np.testing.assert_array_equal(packed.astype(np.float32).view(np.uint32), plain.astype(np.float32).view(np.uint32))
    check_parity(p, packed)


def test_full_size_ragged_sampled():
    # 8191 x 8193 x 8190, lda = K + 3: the automatic repack with the workspace the library asks for
    p = workloads.config("c3_bf16_ragged")
    ws, n = workspace_for(p)
    assert n > 0
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, plan_lda=p.lda)
    pts = workloads.sample_points(p, 300)
    got = result_points(gp, pts)
    ref, den = oracle_points(p, pts)
    err = parity_error_rounded(got, ref, den, p.beta, c0_at(p, pts))
    print(f"c3 repacked: sampled parity error {err:.3e} over {len(pts)} outputs")
    assert err <= 4e-3
    gp.check_guards()


def test_pack_workspace_errors():
    p = workloads.custom("bf16", 64, 2100, 100, lda_pad=3, name="pack_err")
    gp = GpuProblem(p)
    args = (1, p.M, p.N, p.K, "bf16", gp.A, p.lda, 0, gp.B, p.ldb, 0, gp.C, p.ldc, 0)
    need = tg.tile_gemm_workspace_size(1, p.M, p.N, p.K, "bf16", config=tg.TG_CFG_256x256, pack_a=2)
    assert need == p.M * 104 * 2 // 256 * 256 + (256 if p.M * 104 * 2 % 256 else 0)
    ws = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")

    def status(**kw):
        try:
            tg.tile_gemm_ex(*args, **kw)
            return tg.TG_OK
        except tg.TileGemmError as e:
            return e.status
    cfg = dict(config=tg.TG_CFG_256x256)
    assert status(pack_a=2, **cfg) == tg.TG_ERR_INVALID_ARG                                 # no workspace
    assert status(pack_a=2, workspace=ws, workspace_bytes=need - 4, **cfg) == tg.TG_ERR_INVALID_ARG
    assert status(pack_a=2, workspace=gp.C, workspace_bytes=need, **cfg) == tg.TG_ERR_INVALID_ARG  # overlaps C
    assert status(pack_a=2, workspace=ws, config=tg.TG_CFG_128x128) == tg.TG_ERR_UNSUPPORTED
    assert status(pack_a=3, workspace=ws, **cfg) == tg.TG_ERR_INVALID_ARG
    assert status(pack_a=2, workspace=ws, **cfg) == tg.TG_OK
    torch.cuda.synchronize()

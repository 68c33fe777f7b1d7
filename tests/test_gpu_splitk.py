"""Split-K: the deterministic two-pass split reduction (OCANNL "Module
Ir.Schedule" page, paragraph of that name), on the GPU through the C ABI.

* parity with the fp64 oracle within the stated tolerance, ragged K, batches,
  beta != 0, and bitwise on integer-valued inputs (exact in any order);
* the partials and the combine: split(S) equals, bit for bit, S unsplit calls
  on the K slices (same config) folded on the host in the fixed balanced-tree
  order, then scaled by alpha;
* bitwise reproducible run to run; split_k = 1 is the unsplit kernel;
* the workspace contract: a forced split without enough workspace, a
  misaligned or overlapping workspace and fp32 split requests are rejected.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import (GpuProblem, check_parity, need_gpu, oracle_full, oracle_points, parity_error,
                            result_points)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def workspace_for(p, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, **opts)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda"), n


def run_split(p, **opts):
    ws, _ = workspace_for(p, **opts)
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, **opts)
    out = gp.result()
    gp.check_guards()
    return out


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


SPLIT_CASES = [
    # dtype, M, N, K, batch, config, split_k, alpha, beta
    ("bf16", 130, 97, 5000, 1, tg.TG_CFG_64x64, 4, 1.0, 0.0),
    ("f16", 257, 129, 1000, 3, tg.TG_CFG_64x64, 3, 1.5, 0.5),
    ("bf16", 300, 260, 4099, 1, tg.TG_CFG_128x128, 8, -0.75, 1.0),
    ("bf16", 512, 512, 16384, 1, tg.TG_CFG_256x256, 16, 1.0, 0.0),
    ("f16", 64, 64, 70, 2, tg.TG_CFG_64x64, 64, 1.0, 0.5),       # more slices requested than K tiles
]


@pytest.mark.parametrize("dt,M,N,K,batch,cfg,S,alpha,beta", SPLIT_CASES)
def test_split_parity(dt, M, N, K, batch, cfg, S, alpha, beta):
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=3, ldb_pad=5, alpha=alpha, beta=beta,
                         name=f"split_{dt}_{M}x{N}x{K}")
    plan = tg.tile_gemm_plan(batch, M, N, K, dt, config=cfg, split_k=S)
    assert plan["split_k"] > 1 and plan["split_k"] <= S
    assert plan["k_slice"] % plan["block_k"] == 0
    assert (plan["split_k"] - 1) * plan["k_slice"] < K <= plan["split_k"] * plan["k_slice"]
    got = run_split(p, config=cfg, split_k=S)
    check_parity(p, got, points=None if M * N * K * batch <= 2e9 else workloads.sample_points(p, 400))


@pytest.mark.parametrize("dt,M,N,K,batch,cfg,S", [("bf16", 200, 136, 3000, 2, tg.TG_CFG_64x64, 5),
                                                  ("f16", 257, 129, 1000, 1, tg.TG_CFG_128x128, 4)])
def test_split_integer_exact(dt, M, N, K, batch, cfg, S):
    # integer entries in {-2..2}: every partial and the combine are exact, so the
    # split result equals the oracle bit for bit
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=1, ldb_pad=2, alpha=1.5, beta=0.5, dist="int",
                         name="split_int")
    got = run_split(p, config=cfg, split_k=S)
    ref, _ = oracle_full(p)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K,S", [(200, 150, 2600, 6), (101, 99, 2600, 5), (64, 64, 4096, 7),
                                     (96, 80, 4096, 13), (33, 65, 2048, 3), (64, 32, 8192, 64)])
def test_split_equals_slices_folded_in_tree_order(M, N, K, S):
    # M x N a multiple of 4 takes the combine's 16-byte loads, otherwise one element a thread
    dt, cfg, alpha = "bf16", tg.TG_CFG_64x64, 1.5
    p = workloads.custom(dt, M, N, K, lda_pad=3, ldb_pad=5, alpha=alpha, beta=0.0, name="split_tree")
    plan = tg.tile_gemm_plan(1, M, N, K, dt, config=cfg, split_k=S)
    S_eff, ks = plan["split_k"], plan["k_slice"]
    got = run_split(p, config=cfg, split_k=S)
    gp = GpuProblem(p)
    parts = []
    for s in range(S_eff):
        k0, kl = s * ks, min(ks, K - s * ks)
        out = torch.zeros(M * N, dtype=torch.float32, device="cuda")
        # the slice as its own problem: A shifted by k0 columns, B by k0 rows
        tg.tile_gemm_ex(1, M, N, kl, dt, gp.A.data_ptr() + 2 * k0, p.lda, 0,
                        gp.B.data_ptr() + 2 * k0 * p.ldb, p.ldb, 0, out, N, 0, 1.0, 0.0, None,
                        config=cfg, split_k=1)
        torch.cuda.synchronize()
        parts.append(out.cpu().numpy().astype(np.float32))
    # the fixed balanced tree: level w adds slice i + w into slice i, i = 0, 2w, ...
    v = list(parts)
    w = 1
    while w < S_eff:
        for i in range(0, S_eff, 2 * w):
            if i + w < S_eff:
                v[i] = (v[i] + v[i + w]).astype(np.float32)
        w *= 2
    ref = (np.float32(alpha) * v[0]).astype(np.float32).reshape(M, N)
    assert np.array_equal(bits(got[0].astype(np.float32)), bits(ref))


def test_split_deterministic_and_unsplit_identity():
    p = workloads.custom("bf16", 256, 192, 8192, alpha=1.0, beta=0.0, name="split_det")
    outs = [run_split(p, config=tg.TG_CFG_128x128, split_k=8) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(bits(o.astype(np.float32)), bits(outs[0].astype(np.float32)))
    # split_k = 1 is the plain kernel, bit for bit
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(config=tg.TG_CFG_128x128)
    plain = gp.result()
    one = run_split(p, config=tg.TG_CFG_128x128, split_k=1)
    assert np.array_equal(bits(plain.astype(np.float32)), bits(one.astype(np.float32)))
    # and split differs from unsplit only within the tolerance
    check_parity(p, outs[0])


def test_auto_split_needs_workspace():
    # 512 x 512 x 131072 has too few tiles to fill the GPU: the automatic choice
    # splits only when given the workspace it asks for
    M = N = 512
    K = 131072
    plain = tg.tile_gemm_plan(1, M, N, K, "bf16")
    assert plain["split_k"] == 1
    need = tg.tile_gemm_workspace_size(1, M, N, K, "bf16")
    assert need > 0
    with_ws = tg.tile_gemm_plan(1, M, N, K, "bf16", workspace=1 << 20, workspace_bytes=need)
    assert with_ws["split_k"] > 1 and with_ws["workspace_bytes"] == need
    assert with_ws["grid"] == with_ws["tiles_m"] * with_ws["tiles_n"] * with_ws["split_k"]
    short = tg.tile_gemm_plan(1, M, N, K, "bf16", workspace=1 << 20, workspace_bytes=need - 4)
    assert short["split_k"] == 1


def test_full_size_deep_k_sampled():
    # the 512 x 512 x 131072 bf16 workload with its automatic split, sampled outputs
    p = workloads.config("c5_bf16_deepk")
    ws, n = workspace_for(p)
    assert n > 0
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws)
    pts = workloads.sample_points(p, 300)
    got = result_points(gp, pts)
    ref, den = oracle_points(p, pts)
    err = parity_error(got, ref, den)
    print(f"c5 split: sampled parity error {err:.3e} over {len(pts)} outputs")
    assert err <= 4e-3
    gp.check_guards()


def test_workspace_errors():
    p = workloads.custom("bf16", 64, 64, 4096, name="split_err")
    gp = GpuProblem(p)
    args = (1, p.M, p.N, p.K, "bf16", gp.A, p.lda, 0, gp.B, p.ldb, 0, gp.C, p.ldc, 0)
    need = tg.tile_gemm_workspace_size(1, p.M, p.N, p.K, "bf16", split_k=4)
    assert need == 4 * p.M * p.N * 4
    ws = torch.empty(need // 4 + 64, dtype=torch.float32, device="cuda")
    def status(**kw):
        try:
            tg.tile_gemm_ex(*args, **kw)
            return tg.TG_OK
        except tg.TileGemmError as e:
            return e.status
    assert status(split_k=4) == tg.TG_ERR_INVALID_ARG                                  # no workspace
    assert status(split_k=4, workspace=ws, workspace_bytes=need - 4) == tg.TG_ERR_INVALID_ARG
    assert status(split_k=4, workspace=ws.data_ptr() + 4, workspace_bytes=need) == tg.TG_ERR_INVALID_ARG
    assert status(split_k=4, workspace=gp.C, workspace_bytes=need) == tg.TG_ERR_INVALID_ARG   # overlaps C
    assert status(split_k=-1, workspace=ws) == tg.TG_ERR_INVALID_ARG
    assert status(split_k=4, workspace=ws) == tg.TG_OK
    torch.cuda.synchronize()
    q = workloads.custom("f32", 64, 64, 4096, name="split_f32")
    gq = GpuProblem(q)
    try:
        tg.tile_gemm_ex(1, q.M, q.N, q.K, "f32", gq.A, q.lda, 0, gq.B, q.ldb, 0, gq.C, q.ldc, 0, split_k=4,
                        workspace=ws)
        raise AssertionError("fp32 split accepted")
    except tg.TileGemmError as e:
        assert e.status == tg.TG_ERR_UNSUPPORTED


@pytest.mark.parametrize("dt,M,N,K,cfg", [("bf16", 2048, 64, 8192, tg.TG_CFG_64x64),
                                          ("bf16", 64, 2048, 8192, tg.TG_CFG_64x64),
                                          ("bf16", 1024, 96, 4096, tg.TG_CFG_64x64),
                                          ("bf16", 256, 256, 16384, tg.TG_CFG_64x64),
                                          ("bf16", 1024, 1024, 4096, tg.TG_CFG_128x128),
                                          ("f32", 512, 512, 65536, tg.TG_CFG_256x256),
                                          ("f32", 3072, 3072, 1024, tg.TG_CFG_128x128)])
def test_automatic_split_on_skinny_and_deep(dt, M, N, K, cfg):
    """The automatic choice with a workspace (tile and split weighed together) against the oracle."""
    p = workloads.custom(dt, M, N, K, ldb_pad=3, alpha=1.5, beta=0.5, seed=M + N, name="auto_split")
    plan = tg.tile_gemm_plan(1, M, N, K, dt, workspace=1 << 40, workspace_bytes=1 << 40)
    assert plan["split_k"] > 1 and plan["config"] == cfg, plan
    got = run_split(p)
    check_parity(p, got)

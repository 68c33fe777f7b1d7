"""Persistent workgroups (tile_gemm.h, persistent = 2) and two batch entries per
workgroup (the 288 x 160 tile's automatic plan), on the GPU through the C ABI.

Each tile runs the same MFMA sequence in the persistent grid as in the plain
one, so the two results must be equal bit for bit; the persistent result is
also compared with the fp64 oracle at sampled outputs.  The shapes give every
workgroup two tiles, two or three (576 tiles over 256 workgroups), and four.
"""
import numpy as np
import pytest

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, need_gpu, oracle_points, parity_error, result_points

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = [
    ("bf16", 4096, 8192, 256, 1.0, 0.0),
    ("f16", 6144, 6144, 384, 1.5, 0.5),
    ("bf16", 8192, 8192, 1024, -0.75, 1.0),
]


@pytest.mark.parametrize("dt,M,N,K,alpha,beta", CASES, ids=lambda v: str(v))
def test_persistent_bitwise_and_parity(dt, M, N, K, alpha, beta):
    p = workloads.custom(dt, M, N, K, alpha=alpha, beta=beta, seed=M + K, name="persistent")
    assert tg.tile_gemm_plan(1, M, N, K, dt, persistent=2)["persistent"] == 1
    gp = GpuProblem(p)
    out = {}
    for persistent in (2, 0):
        gp.reset_c()
        gp.run(persistent=persistent)
        out[persistent] = gp.c_view().clone()
        gp.check_guards()
    a = out[2].cpu().numpy().view(np.uint32)
    b = out[0].cpu().numpy().view(np.uint32)
    assert np.array_equal(a, b), f"{int((a != b).sum())} outputs differ between the persistent and plain grids"
    pts = workloads.sample_points(p, 200)
    gp.reset_c()
    gp.run(persistent=2)
    got = result_points(gp, pts)
    ref, den = oracle_points(p, pts)
    c0 = p.C0[pts[:, 1] * p.ldc + pts[:, 2]].astype(np.float64) if beta != 0 else 0.0
    err = parity_error(got, ref, abs(alpha) * den + abs(beta) * np.abs(c0))
    assert err <= 4e-3, err


# Two batch entries per workgroup (the automatic plan for single-block problems on the
# 288 x 160 tile in more than one round and at most two): each entry runs the plain ring's
# MFMA sequence, so the result equals the plain grid's (persistent = 1) bit for bit.
# (dtype, M, N, K, batch, alpha, beta, bias mode, activation)
CHAIN_CASES = [
    ("f16", 257, 129, 1000, 512, 1.0, 0.0, 0, 0),      # the batched workload: every workgroup two entries
    ("bf16", 200, 150, 333, 300, 1.5, 0.5, 0, 0),      # 44 workgroups with two, the rest one
    ("f16", 288, 160, 128, 257, -1.0, 1.0, 0, 0),      # whole tiles, the fewest K tiles the chain takes
    ("bf16", 160, 100, 1024, 400, 1.0, 0.0, 1, 2),     # fused tail, a bias vector per entry
]


@pytest.mark.parametrize("dt,M,N,K,B,alpha,beta,mode,act", CHAIN_CASES, ids=lambda v: str(v))
def test_two_entries_per_workgroup_bitwise_and_parity(dt, M, N, K, B, alpha, beta, mode, act):
    import torch
    p = workloads.custom(dt, M, N, K, batch=B, alpha=alpha, beta=beta, seed=B + K, name="chain")
    opts = dict(config=tg.TG_CFG_288x160)
    if mode:
        bias = np.random.default_rng(B).standard_normal(B * N).astype(np.float32)
        opts.update(bias=torch.from_numpy(bias).to("cuda"), bias_stride=N, bias_mode=mode, activation=act)
    plan_kw = {k: v for k, v in opts.items() if k not in ("bias", "bias_stride")}
    plan = tg.tile_gemm_plan(B, M, N, K, dt, **plan_kw)
    assert (plan["persistent"], plan["grid"]) == (1, 256)
    assert tg.tile_gemm_plan(B, M, N, K, dt, persistent=1, **plan_kw)["grid"] == B
    gp = GpuProblem(p)
    out = {}
    for persistent in (0, 1):
        gp.reset_c()
        gp.run(persistent=persistent, **opts)
        out[persistent] = gp.c_view().clone()
        gp.check_guards()
    a = out[0].cpu().numpy().view(np.uint32)
    b = out[1].cpu().numpy().view(np.uint32)
    assert np.array_equal(a, b), f"{int((a != b).sum())} outputs differ between two entries per workgroup and one"
    if mode:
        return      # the fused tail's parity is the plain grid's (test_gpu_fused_tail.py)
    check_parity(p, out[0].cpu().numpy().astype(np.float64), points=workloads.sample_points(p, 400))

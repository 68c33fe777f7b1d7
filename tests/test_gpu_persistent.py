"""Persistent workgroups (tile_gemm.h, persistent = 2), on the GPU through the C ABI.

Each tile runs the same MFMA sequence in the persistent grid as in the plain
one, so the two results must be equal bit for bit; the persistent result is
also compared with the fp64 oracle at sampled outputs.  The shapes give every
workgroup two tiles, two or three (576 tiles over 256 workgroups), and four.
"""
import numpy as np
import pytest

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, need_gpu, oracle_points, parity_error, result_points

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

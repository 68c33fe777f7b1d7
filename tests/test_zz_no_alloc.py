"""tile_gemm_ex_noalloc: the call that works in the library's own scratch.

Through the C ABI: its C equals, bit for bit, tile_gemm_ex's C for the same
arguments and a caller workspace of the scratch's size (the same plan, the
same kernels), over two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents, which the second must not depend on);
forced splits and repacks that need more than the scratch holds are refused
before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def run_both(p, **opts):
    """(noalloc C, tile_gemm_ex C with a workspace of the scratch's size)."""
    gp = GpuProblem(p)
    gp.reset_c()
    tg.tile_gemm_ex_noalloc(p.batch, p.M, p.N, p.K, p.dtype, gp.A, p.lda, p.strideA, gp.B, p.ldb, p.strideB,
                            gp.C, p.ldc, p.strideC, p.alpha, p.beta, None, **opts)
    got = gp.result()
    gp.check_guards()
    ws = torch.empty(tg.NOALLOC_SCRATCH_BYTES // 4, dtype=torch.float32, device="cuda")
    ref_gp = GpuProblem(p)
    ref_gp.reset_c()
    ref_gp.run(workspace=ws, **opts)
    ref = ref_gp.result()
    return got, ref


# (first call, second smaller call): each a problem and its options
PAIRS = [
    # split-K into the scratch: 16 partial planes of 1 MiB, then 4 of 300 x 260
    (dict(dt="bf16", M=512, N=512, K=16384, batch=1, alpha=1.0, beta=0.0, opts=dict(split_k=16)),
     dict(dt="bf16", M=300, N=260, K=4000, batch=1, alpha=1.5, beta=0.5, opts=dict(split_k=4))),
    # the automatic choice: the deep-K workload's split (64 planes, all 64 MiB), then a batch
    (dict(dt="bf16", M=512, N=512, K=131072, batch=1, alpha=1.0, beta=0.0, opts={}),
     dict(dt="f16", M=130, N=97, K=5000, batch=2, alpha=1.0, beta=0.5, opts={})),
    # two batch entries per workgroup on the 288 x 160 tile (no scratch), then a split into it
    (dict(dt="bf16", M=150, N=100, K=200, batch=260, alpha=1.5, beta=0.5, opts=dict(config=tg.TG_CFG_288x160)),
     dict(dt="bf16", M=300, N=260, K=4000, batch=1, alpha=1.0, beta=0.0, opts=dict(split_k=4))),
    # the aligned copy of A (lda = K + 3) in the scratch, then a split call of another config
    (dict(dt="bf16", M=2048, N=2300, K=1000, batch=1, alpha=1.5, beta=0.5, lda_pad=3, opts=dict(pack_a=2)),
     dict(dt="f16", M=257, N=129, K=1000, batch=3, alpha=1.0, beta=0.0, opts=dict(config=tg.TG_CFG_64x64,
                                                                                  split_k=3))),
]


def problem(c):
    return workloads.custom(c["dt"], c["M"], c["N"], c["K"], batch=c["batch"], lda_pad=c.get("lda_pad", 0),
                            ldb_pad=1, alpha=c["alpha"], beta=c["beta"], seed=c["K"] % 97)


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_workspace_call_twice(first, second):
    for c in (first, second):
        p = problem(c)
        plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, workspace=1 << 8,
                                 workspace_bytes=tg.NOALLOC_SCRATCH_BYTES, **c["opts"])
        assert plan["workspace_bytes"] <= tg.NOALLOC_SCRATCH_BYTES
        got, ref = run_both(p, **c["opts"])
        assert np.array_equal(bits(got), bits(ref)), c
        if p.M * p.N * p.K * p.batch <= (1 << 31):
            check_parity(p, got)


def test_noalloc_refuses_what_does_not_fit():
    # a forced split whose partials exceed 64 MiB: 32 planes of 1024 x 1024 fp32 (128 MiB)
    p = workloads.custom("bf16", 1024, 1024, 8192, seed=1)
    gp = GpuProblem(p)
    gp.reset_c()
    opt = tg._options(split_k=32, workspace=None, workspace_bytes=0)
    args = (1, p.M, p.N, p.K, tg.TG_BF16, gp.A.data_ptr(), p.lda, 0, gp.B.data_ptr(), p.ldb, 0,
            gp.C.data_ptr(), p.ldc, 0, 1.0, 0.0, 0)
    assert tg.tile_gemm_status("tile_gemm_ex_noalloc", *args, ctypes.byref(opt)) == tg.TG_ERR_SCRATCH_LIMIT
    # a caller workspace is refused: the call owns its scratch
    opt = tg._options(workspace=gp.C.data_ptr(), workspace_bytes=1024)
    assert tg.tile_gemm_status("tile_gemm_ex_noalloc", *args, ctypes.byref(opt)) == tg.TG_ERR_INVALID_ARG
    # nothing was launched: C still holds what reset_c wrote (NaN, beta == 0)
    assert np.isnan(gp.result()).all()

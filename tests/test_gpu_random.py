"""Seeded random sweep of the call's options against the fp64 oracle, on the GPU.

Each case draws, from its own fixed seed, a dtype, ragged extents (1 to 600), a batch of 1 to 3,
leading-dimension padding, alpha and beta, a tile configuration, a split-K count, the repacks of
A and B, remainder GEMMs or split strips and a fused tail (bias per column or per row with a batch stride, ReLU or
GELU).  A combination the plan refuses (TG_ERR_UNSUPPORTED) is skipped; every other case must
match the oracle over the whole output and write nothing outside C.  The seeds are fixed, so
the sweep is the same on every run.
"""
import numpy as np
import pytest
import torch

import oracle
import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import TOL, GpuProblem, c0_at, need_gpu, parity_error, parity_error_rounded

pytestmark = pytest.mark.gpu

N_CASES = 48


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    dt = ["f32", "bf16", "f16"][r.integers(0, 3)]
    ext = lambda: int(r.choice([r.integers(1, 70), r.integers(60, 300), r.integers(250, 601)]))
    M, N, K = ext(), ext(), int(r.choice([r.integers(0, 40), r.integers(30, 600)]))
    batch = int(r.integers(1, 4))
    pads = [int(r.integers(0, 8)) for _ in range(3)]
    alpha = float(r.choice([1.0, -0.5, 1.5, 2.0]))
    beta = float(r.choice([0.0, 0.0, 1.0, 0.5, -1.0]))
    opts = {}
    if dt == "f32":
        opts["config"] = int(r.choice([0, tg.TG_CFG_F32_64x64]))
    else:
        opts["config"] = int(r.choice([0, tg.TG_CFG_256x256, tg.TG_CFG_128x128, tg.TG_CFG_64x64]))
        opts["split_k"] = int(r.choice([0, 1, 1, 2, 3, 5]))
        opts["pack_a"] = int(r.choice([0, 0, 1, 2]))
        opts["tail_gemm"] = int(r.choice([0, 0, 2]))
    mode = int(r.choice([0, 0, 1, 2]))
    act = int(r.choice([0, 0, 1, 2]))
    if dt != "f32" and r.integers(0, 6) == 0:      # drawn last, so the draws above stay as they were
        opts["config"] = tg.TG_CFG_288x160
    if dt != "f32":
        opts["pack_b"] = int(r.choice([0, 0, 1, 2]))
        if opts["pack_b"] == 2 and opts["config"] not in (0, tg.TG_CFG_256x256):
            opts["pack_b"] = 0                      # built for the 256 x 256 tile only
        if r.integers(0, 5) == 0:
            opts["tail_gemm"] = 3
    if dt == "f32" and r.integers(0, 2) == 0:       # the fp32 ring tiles, with a split or split strips
        opts["config"] = int(r.choice([tg.TG_CFG_256x256, tg.TG_CFG_128x128]))
        opts["split_k"] = int(r.choice([0, 1, 2, 3, 5]))
        opts["tail_gemm"] = int(r.choice([0, 0, 3]))
    return dt, M, N, K, batch, pads, alpha, beta, opts, mode, act


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    dt, M, N, K, batch, pads, alpha, beta, opts, mode, act = draw(seed)
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=pads[0], ldb_pad=pads[1], ldc_pad=pads[2],
                         alpha=alpha, beta=beta, seed=seed, name="rand")
    length = N if mode == 1 else M
    stride = (length + 3) if (mode and batch > 1) else 0
    bias = None
    if mode:
        bias = (np.random.default_rng(seed).standard_normal((batch - 1) * stride + length)
                * max(K, 1) ** 0.5 / 3).astype(np.float32)
    tail = dict(bias_mode=mode, activation=act)
    try:
        tg.tile_gemm_plan(batch, M, N, K, dt, plan_lda=p.lda, plan_ldb=p.ldb, workspace=1 << 40,
                          workspace_bytes=1 << 40, **opts, **tail)
    except tg.TileGemmError as e:
        if e.status == tg.TG_ERR_UNSUPPORTED:
            pytest.skip(f"combination not built: {opts} {tail}")
        raise
    n = tg.tile_gemm_workspace_size(batch, M, N, K, dt, plan_lda=p.lda, plan_ldb=p.ldb, **opts, **tail)
    ws = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    gp = GpuProblem(p)
    gp.reset_c()
    try:
        gp.run(workspace=ws, plan_lda=p.lda, plan_ldb=p.ldb, bias=torch.from_numpy(bias).cuda() if bias is not None else None,
               bias_stride=stride, **opts, **tail)
    except tg.TileGemmError as e:
        if e.status == tg.TG_ERR_UNSUPPORTED:
            pytest.skip(f"combination not built for this call: {opts} {tail}")
        raise
    got = gp.result()
    ref, den = oracle.gemm(M, N, K, dt, p.A, p.lda, p.B, p.ldb, C0=p.C0, ldc=p.ldc, alpha=alpha, beta=beta,
                           batch=batch, strideA=p.strideA, strideB=p.strideB, strideC=p.strideC, with_absden=True,
                           bias=bias, bias_stride=stride, bias_mode=mode, activation=act)
    if mode or act:
        # the tail's activation acts on alpha * A.B + bias: its input's magnitude is the scale
        den = abs(alpha) * den + abs(beta) * np.abs(c0_at(p))
        if mode:
            for b in range(batch):
                v = np.abs(bias[b * stride: b * stride + length].astype(np.float64))
                den[b] += v[None, :] if mode == 1 else v[:, None]
        err = parity_error(got, ref, den)
    else:
        err = parity_error_rounded(got, ref, den, beta, c0_at(p))
    assert err <= TOL[dt], f"seed {seed}: {dt} {batch}x{M}x{N}x{K} {opts} {tail}: parity error {err:.3e}"
    gp.check_guards()

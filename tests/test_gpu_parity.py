"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerance (from the problem statement): max |C_gpu - C_ref| / (sum_k |A_ik||B_kj| + 1e-30)
<= 1e-5 for fp32 inputs and <= 4e-3 for bf16/fp16 inputs.  Integer-valued inputs,
whose every fp32 partial sum is exact, must match the oracle bit for bit.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import (GpuProblem, check_parity, need_gpu, oracle_full, oracle_points, parity_error,
                            result_points)

pytestmark = pytest.mark.gpu

CFG16 = [tg.TG_CFG_256x256, tg.TG_CFG_128x128, tg.TG_CFG_64x64, tg.TG_CFG_288x160]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_full(p, **opts):
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(**opts)
    out = gp.result()
    gp.check_guards()
    return out


# ---- small and medium shapes: several tiles plus ragged tails, full oracle -----------

SHAPES16 = [(1, 1, 1), (17, 15, 16), (64, 64, 64), (65, 63, 65), (300, 520, 200), (513, 257, 130),
            (256, 256, 512), (100, 700, 1000)]


@pytest.mark.parametrize("cfg", CFG16)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES16, ids=lambda s: "x".join(map(str, s)))
def test_parity_16bit(cfg, dtype, shape):
    M, N, K = shape
    p = workloads.custom(dtype, M, N, K, lda_pad=3, ldb_pad=5, ldc_pad=2, alpha=1.5, beta=0.5, seed=M + N + K)
    check_parity(p, run_full(p, config=cfg))


@pytest.mark.parametrize("shape", [(1, 1, 1), (67, 45, 53), (64, 64, 32), (130, 70, 97), (200, 300, 257)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ab", [(1.0, 0.0), (1.5, 0.5), (-0.75, 2.0)])
def test_parity_f32(shape, ab):
    M, N, K = shape
    p = workloads.custom("f32", M, N, K, lda_pad=1, ldb_pad=3, alpha=ab[0], beta=ab[1], seed=M * N + K)
    check_parity(p, run_full(p))


# ---- integer-valued inputs: every partial sum exact, so the result is bit-exact ------

INT_SHAPES = [("bf16", 67, 45, 53, 0, 0), ("bf16", 300, 520, 200, 3, 5), ("f16", 257, 129, 1000, 0, 0),
              ("bf16", 513, 1031, 777, 1, 7), ("f32", 67, 45, 53, 0, 0), ("f32", 131, 77, 150, 2, 1)]


@pytest.mark.parametrize("case", INT_SHAPES, ids=lambda c: "_".join(map(str, c)))
@pytest.mark.parametrize("ab", [(1.0, 0.0), (1.5, 0.5), (1.0, 1.0)])
def test_integer_inputs_bit_exact(case, ab):
    dt, M, N, K, pa, pb = case
    p = workloads.custom(dt, M, N, K, lda_pad=pa, ldb_pad=pb, alpha=ab[0], beta=ab[1], dist="int",
                         seed=M + K)
    assert 4 * K * abs(ab[0]) + abs(ab[1]) * p.c0_ilim < 2 ** 23
    cfgs = [0] if dt == "f32" else CFG16
    ref, den = oracle_full(p)
    for cfg in cfgs:
        got = run_full(p, config=cfg)
        assert np.array_equal(got, ref), f"config {cfg}: not bit-exact"


# ---- the five measured problems ------------------------------------------------------

def config_problem(name, dist=None):
    p = workloads.CONFIGS[name]
    if dist:
        p = replace(p, dist=dist)
    return workloads.materialize(p)


def test_config1_f32_full():
    p = config_problem("c1_f32_67x45x53")
    err = check_parity(p, run_full(p), stated=True)
    print(f"c1 parity error {err:.3e}")


@pytest.mark.parametrize("name", ["c2_bf16_8192", "c3_bf16_ragged", "c4_f16_batched", "c5_bf16_deepk"])
def test_config_full_size_sampled(name):
    p = config_problem(name)
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run()
    pts = workloads.sample_points(p, 3000, seed=5)
    got = result_points(gp, pts)
    ref, den = oracle_points(p, pts)
    err = parity_error(got, ref, den)
    print(f"{name}: sampled parity error {err:.3e} over {len(pts)} outputs")
    assert err <= 4e-3
    if name == "c3_bf16_ragged":
        gp.check_guards()


@pytest.mark.parametrize("name", ["c2_bf16_8192", "c3_bf16_ragged", "c4_f16_batched", "c5_bf16_deepk"])
def test_config_full_size_integer_bit_exact(name):
    p = config_problem(name, dist="int")
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run()
    pts = workloads.sample_points(p, 2000, seed=9)
    got = result_points(gp, pts)
    ref, _ = oracle_points(p, pts)
    assert np.array_equal(got, ref)


def test_config4_whole_batches():
    p = config_problem("c4_f16_batched")
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run()
    out = gp.result()
    for b in (0, 1, 255, 511):
        q = workloads.Problem("c4_one", "f16", p.M, p.N, p.K, lda=p.lda, ldb=p.ldb, ldc=p.ldc)
        q.A = np.ascontiguousarray(p.A[b * p.strideA:(b + 1) * p.strideA])
        q.B = np.ascontiguousarray(p.B[b * p.strideB:(b + 1) * p.strideB])
        check_parity(q, out[b:b + 1], stated=True)

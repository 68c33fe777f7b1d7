"""Hoisted pre-pack of B (tile_gemm.h, tile_gemm_pack_b), on the GPU.

* the packed layout, byte for byte against the same layout built on the host,
  for fp32 / bf16 / fp16, B as stored or transposed, ragged K and N, ldb
  padding and a strided batch; every packed element is written (padding zero);
* a GEMM on the packed copy equals the GEMM on the original B bit for bit (the
  same values in the same MFMA sequence) on every tile configuration, split
  along K and at full size 8191 x 8193 x 8190 (ldb = N + 5), and matches the
  fp64 oracle; a transposed source gives the same C as its transpose.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, device_tensor, need_gpu, oracle_points, parity_error, \
    parity_error_rounded, result_points

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def dense_storage(p):
    """B of each batch entry as a (K, N) array of its storage type (uint16 or float32)."""
    return np.stack([p.B[b * p.strideB: b * p.strideB + p.K * p.ldb].reshape(p.K, p.ldb)[:, :p.N]
                     for b in range(p.batch)])


def expected_packed(p, ld):
    Bd = dense_storage(p)
    out = np.zeros((p.batch, p.K, ld), dtype=Bd.dtype)
    out[:, :, :p.N] = Bd
    return out


def packed_buffer(p):
    n = tg.tile_gemm_packed_b_size(p.batch, p.K, p.N, p.dtype)
    itemsize = 4 if p.dtype == "f32" else 2
    # a sentinel in every byte, so an unwritten element shows
    t = torch.full((max(n, 256) // 4 + 64,), -1, dtype=torch.int32, device="cuda")
    return t, n, itemsize


def transposed_source(p, pad):
    """B of each batch entry stored transposed: N rows of K (+ pad) elements, batch-strided."""
    Bd = dense_storage(p)
    ldt = p.K + pad
    st = p.N * ldt + 7
    src = np.zeros(p.batch * st, dtype=Bd.dtype)
    for b in range(p.batch):
        m = np.zeros((p.N, ldt), dtype=Bd.dtype)
        m[:, :p.K] = Bd[b].T
        src[b * st: b * st + p.N * ldt] = m.reshape(-1)
    return src, ldt, st


LAYOUT_CASES = [
    # dtype, K, N, batch, ldb_pad
    ("bf16", 100, 257, 1, 3),
    ("f16", 65, 64, 3, 0),
    ("f32", 53, 45, 2, 1),
    ("bf16", 1, 1, 1, 0),
    ("f32", 300, 1000, 1, 5),
]


@pytest.mark.parametrize("transposed", [0, 1])
@pytest.mark.parametrize("dt,K,N,batch,pad", LAYOUT_CASES, ids=lambda v: str(v))
def test_packed_layout(dt, K, N, batch, pad, transposed):
    p = workloads.custom(dt, 8, N, K, batch=batch, ldb_pad=pad, seed=K + N, name="pk")
    ld = tg.tile_gemm_packed_b_ld(N, dt)
    assert ld % (8 if dt != "f32" else 4) == 0 and N <= ld < N + (8 if dt != "f32" else 4) + (N == 0)
    buf, n, itemsize = packed_buffer(p)
    if transposed:
        src, ldt, st = transposed_source(p, pad)
        tg.tile_gemm_pack_b(batch, K, N, dt, device_tensor(src), ldt, st, buf, n, transposed=1)
    else:
        tg.tile_gemm_pack_b(batch, K, N, dt, device_tensor(p.B), p.ldb, p.strideB, buf, n)
    torch.cuda.synchronize()
    raw = buf.cpu().numpy().view(np.uint8)
    want = expected_packed(p, ld)
    got = raw[:want.nbytes].view(want.dtype).reshape(want.shape)
    np.testing.assert_array_equal(got.view(np.uint8), want.view(np.uint8))
    assert np.all(raw[want.nbytes:] == 0xFF), "a write past the packed size"


GEMM_CASES = [
    # dtype, M, N, K, batch, ldb_pad, config, split_k, alpha, beta
    ("bf16", 300, 257, 100, 1, 3, 0, 0, 1.0, 0.0),
    ("bf16", 520, 600, 700, 2, 5, tg.TG_CFG_256x256, 1, 1.5, 0.5),
    ("f16", 257, 129, 1000, 3, 1, 0, 0, 1.0, 0.0),
    ("bf16", 200, 300, 2100, 1, 5, tg.TG_CFG_128x128, 3, 1.0, -1.0),
    ("f16", 97, 65, 40, 1, 0, tg.TG_CFG_64x64, 1, 1.0, 0.0),
    ("f32", 67, 45, 53, 1, 1, 0, 0, 1.0, 0.0),
]


def run_gemm(p, B_dev, ldb, strideB, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, **opts)
    ws = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    gp = GpuProblem(p)
    gp.reset_c()
    tg.tile_gemm_ex(p.batch, p.M, p.N, p.K, p.dtype, gp.A, p.lda, p.strideA, B_dev, ldb, strideB, gp.C, p.ldc,
                    p.strideC, p.alpha, p.beta, None, workspace=ws, plan_lda=p.lda, **opts)
    return gp


@pytest.mark.parametrize("transposed", [0, 1])
@pytest.mark.parametrize("dt,M,N,K,batch,pad,cfg,split,alpha,beta", GEMM_CASES, ids=lambda v: str(v))
def test_gemm_on_packed_b(dt, M, N, K, batch, pad, cfg, split, alpha, beta, transposed):
    p = workloads.custom(dt, M, N, K, batch=batch, ldb_pad=pad, alpha=alpha, beta=beta, seed=M + K, name="pkg")
    opts = dict(config=cfg, split_k=split)
    ref = run_gemm(p, device_tensor(p.B), p.ldb, p.strideB, **opts)
    buf, n, _ = packed_buffer(p)
    if transposed:
        src, ldt, st = transposed_source(p, pad)
        tg.tile_gemm_pack_b(batch, K, N, dt, device_tensor(src), ldt, st, buf, n, transposed=1)
    else:
        tg.tile_gemm_pack_b(batch, K, N, dt, device_tensor(p.B), p.ldb, p.strideB, buf, n)
    ld = tg.tile_gemm_packed_b_ld(N, dt)
    got = run_gemm(p, buf, ld, K * ld, **opts)
    a, b = got.result(), ref.result()
    np.testing.assert_array_equal(a.astype(np.float32).view(np.uint32), b.astype(np.float32).view(np.uint32))
    check_parity(p, a)
    got.check_guards()


def test_full_size_ragged_packed_b():
    # 8191 x 8193 x 8190, lda = K + 3, ldb = N + 5: B packed once, then the call on the packed copy
    p = workloads.custom("bf16", 8191, 8193, 8190, lda_pad=3, ldb_pad=5, alpha=1.5, beta=0.5, seed=11, name="pkf")
    ref = run_gemm(p, device_tensor(p.B), p.ldb, p.strideB)
    buf, n, _ = packed_buffer(p)
    tg.tile_gemm_pack_b(1, p.K, p.N, "bf16", device_tensor(p.B), p.ldb, 0, buf, n)
    ld = tg.tile_gemm_packed_b_ld(p.N, "bf16")
    got = run_gemm(p, buf, ld, 0)
    torch.cuda.synchronize()
    assert torch.equal(got.c_view().contiguous().view(torch.int32), ref.c_view().contiguous().view(torch.int32))
    pts = workloads.sample_points(p, 200)
    vals = result_points(got, pts)
    o, den = oracle_points(p, pts)
    c0 = p.C0[pts[:, 1] * p.ldc + pts[:, 2]].astype(np.float64)
    assert parity_error_rounded(vals, o, den, p.beta, c0) <= 4e-3
    got.check_guards()

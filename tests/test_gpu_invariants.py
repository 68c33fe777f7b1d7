"""GPU-vs-GPU invariants of the schedule (bitwise), plus edge cases.

* pad-to-tile: a ragged problem equals, bit for bit, the crop of the same
  problem zero-padded to tile multiples (OCANNL Pad paragraph: pad iterations
  are no-ops; staged fringes are zero-filled);
* window-2 pipeline == depth 1, bitwise (OCANNL pipeline_depth paragraph);
* the placement (none, pad_stride, XOR swizzle) and the block order change
  where values sit only, bitwise (OCANNL Stage paragraph, swizzle and
  pad_stride: semantics unchanged);
* fused alpha/beta epilogue == a separate elementwise pass (OCANNL epilogue
  fusion: bitwise equal to the two-kernel form);
* NaN in the lda/ldb padding never reaches C; C outside M x N is never written;
  beta == 0 never reads C; repeated runs are bitwise identical.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import GpuProblem, check_parity, need_gpu

pytestmark = pytest.mark.gpu

CFG16 = [tg.TG_CFG_256x256, tg.TG_CFG_128x128, tg.TG_CFG_64x64, tg.TG_CFG_288x160]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(p, **opts):
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(**opts)
    out = gp.result()
    gp.check_guards()
    return out


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def padded(p, Mp, Np, Kp):
    """The problem embedded in zeros at (Mp, Np, Kp), contiguous strides, NaN beyond."""
    q = workloads.Problem(p.name + "_pad", p.dtype, Mp, Np, Kp, batch=p.batch, lda=Kp + 8, ldb=Np + 8,
                          ldc=Np, alpha=p.alpha, beta=p.beta)
    nan = {"bf16": 0x7FC0, "f16": 0x7E00}
    def embed(buf, rows, cols, ld, stride, R, Cc, ldn, stride_n, f32=False):
        dt = np.float32 if f32 else np.uint16
        out = np.zeros((q.batch, R, ldn), dtype=dt)
        out[:, :, Cc:] = np.nan if f32 else nan[p.dtype]
        for b in range(p.batch):
            src = buf[b * stride: b * stride + rows * ld].reshape(rows, ld)[:, :cols]
            out[b, :rows, :cols] = src
        return out.reshape(-1)
    f32 = p.dtype == "f32"
    q.A = embed(p.A, p.M, p.K, p.lda, p.strideA, Mp, Kp, q.lda, q.strideA, f32)
    q.B = embed(p.B, p.K, p.N, p.ldb, p.strideB, Kp, Np, q.ldb, q.strideB, f32)
    if p.beta != 0:
        c = np.zeros((q.batch, Mp, Np), dtype=np.float32)
        for b in range(p.batch):
            c[b, :p.M, :p.N] = p.C0[b * p.strideC: b * p.strideC + p.M * p.ldc].reshape(p.M, p.ldc)[:, :p.N]
        q.C0 = c.reshape(-1)
    return q


@pytest.mark.parametrize("cfg,dt,tile", [(tg.TG_CFG_256x256, "bf16", (256, 256, 32)),
                                         (tg.TG_CFG_128x128, "f16", (128, 128, 32)),
                                         (tg.TG_CFG_64x64, "bf16", (64, 64, 32)),
                                         (tg.TG_CFG_288x160, "f16", (288, 160, 32)),
                                         (0, "f32", (64, 64, 32))])
# (300, 328, 130): an N edge on a 16-byte chunk (the fringe blocks copy like interior ones);
# N = 333, 45, 129: an N edge inside a chunk (per-copy resources)
@pytest.mark.parametrize("shape", [(300, 333, 130), (67, 45, 53), (257, 129, 1000), (300, 328, 130)], ids=str)
def test_ragged_equals_cropped_padded(cfg, dt, tile, shape):
    M, N, K = shape
    p = workloads.custom(dt, M, N, K, batch=2, lda_pad=3, ldb_pad=1, ldc_pad=5, alpha=1.5, beta=0.5, seed=K)
    base = run(p, config=cfg)
    up = lambda x, t: -(-x // t) * t
    for Mp, Np, Kp in [(up(M, tile[0]), up(N, tile[1]), up(K, tile[2])),
                       (up(M, tile[0]) + tile[0], up(N, tile[1]), up(K, tile[2]) + 2 * tile[2])]:
        q = padded(p, Mp, Np, Kp)
        got = run(q, config=cfg)[:, :M, :N]
        assert np.array_equal(bits(got), bits(base)), (Mp, Np, Kp)


@pytest.mark.parametrize("cfg,dt", [(c, "bf16") for c in CFG16] + [(tg.TG_CFG_128x128, "f16"), (0, "f32")])
def test_depth_swizzle_order_are_bitwise_invisible(cfg, dt):
    p = workloads.custom(dt, 531, 389, 333, lda_pad=1, ldb_pad=2, alpha=0.75, beta=-1.25, seed=3)
    ref = run(p, config=cfg)
    variants = [dict(pipeline_depth=1), dict(pipeline_depth=2), dict(swizzle=tg.SWZ_NONE), dict(block_order=1)]
    if cfg == tg.TG_CFG_288x160:           # built at depths 2 and 4
        variants = variants[1:]
    if dt == "f32":
        variants.append(dict(pipeline_depth=1, swizzle=tg.SWZ_NONE, block_order=1))
    if cfg == tg.TG_CFG_256x256:
        variants.append(dict(swizzle=tg.SWZ_PAD))
    for opts in variants:
        got = run(p, config=cfg, **opts)
        assert np.array_equal(bits(got), bits(ref)), opts


# The three placements of the 256 x 256 kernel at its default depth, over shapes
# whose plans use every block kind: interior and fringe tiles, 256 x 64 N strips
# and 64 x 256 M strips (with their corner), a ragged last K tile, a batch.
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(531, 389, 333, 1), (300, 520, 100, 2), (770, 1030, 1024, 1),
                                   (256, 256, 32, 1), (257, 129, 1000, 3)], ids=str)
def test_none_pad_xor_placements_are_bitwise_equal(dt, shape):
    M, N, K, batch = shape
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=5, ldb_pad=3, ldc_pad=1, alpha=1.5, beta=0.5,
                         seed=M + K)
    out = {swz: run(p, config=tg.TG_CFG_256x256, swizzle=swz) for swz in (tg.SWZ_NONE, tg.SWZ_PAD, tg.SWZ_XOR)}
    assert np.array_equal(bits(out[tg.SWZ_PAD]), bits(out[tg.SWZ_XOR]))
    assert np.array_equal(bits(out[tg.SWZ_NONE]), bits(out[tg.SWZ_XOR]))
    check_parity(p, out[tg.SWZ_PAD])


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("ab", [(1.0, 0.5), (2.0, -1.5), (0.5, 1.0)])
def test_fused_epilogue_equals_separate_pass(dt, ab):
    # alpha is a power of two, so alpha*acc is exact and the fused fma(alpha, acc, beta*c0)
    # equals the unfused two-kernel tail: acc first (alpha=1, beta=0), then alpha*acc + beta*c0.
    alpha, beta = ab
    p = workloads.custom(dt, 333, 271, 190, ldc_pad=3, alpha=alpha, beta=beta, seed=7)
    fused = run(p)
    p0 = workloads.custom(dt, 333, 271, 190, ldc_pad=3, alpha=1.0, beta=0.0, seed=7)
    p0.A, p0.B = p.A, p.B
    acc = torch.from_numpy(run(p0).astype(np.float32)).cuda()
    c0 = torch.from_numpy(p.C0.reshape(p.M, p.ldc)[:, :p.N].copy()).cuda()
    tail = (alpha * acc) + (beta * c0)          # elementwise pass on the GPU, fp32
    assert np.array_equal(bits(fused), bits(tail.cpu().numpy()))


def test_deterministic_runs():
    p = workloads.custom("bf16", 1000, 1100, 900, lda_pad=3, alpha=1.5, beta=0.5, seed=2)
    gp = GpuProblem(p)
    outs = []
    for _ in range(10):
        gp.reset_c()
        gp.run()
        outs.append(bits(gp.result()))
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 300, 7), (300, 1, 7), (15, 16, 17), (63, 65, 64),
                                   (129, 64, 1), (64, 129, 200), (16, 16, 0)], ids=str)
def test_edge_extents(dt, shape):
    M, N, K = shape
    for ab in [(1.0, 0.0), (1.0, 1.0), (-2.0, 0.5)]:
        p = workloads.custom(dt, M, N, K, lda_pad=2, ldb_pad=1, alpha=ab[0], beta=ab[1], seed=M + N + K)
        check_parity(p, run(p))


@pytest.mark.parametrize("N", [300, 296])   # an N edge inside a 16-byte chunk, and on one
def test_beta_zero_never_reads_c_and_nan_padding_never_leaks(N):
    p = workloads.custom("bf16", 200, N, 100, lda_pad=7, ldb_pad=9, ldc_pad=4, alpha=1.0, beta=0.0, seed=4)
    gp = GpuProblem(p)
    gp.reset_c()            # C = NaN inside the window (beta == 0 must not read it)
    gp.run()
    out = gp.result()
    gp.check_guards()
    assert not np.isnan(out).any()
    check_parity(p, out)


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_c_row_stride_at_the_tile_offset_limit(beta):
    """A block's tile of C spans at most 2^31 - 4097 bytes (a fringe block stores C through a
    buffer resource with 32-bit byte offsets): with 256 x 256 blocks the largest row stride
    allowed computes (fringe rows and columns, its last row 8 MB from its first), the next
    is refused before any device work and C is left as it was."""
    lim = 2**31 - 1 - 4096
    ldc_max = ((lim - 1) // 4 - 256) // 256
    assert (256 * ldc_max + 256) * 4 < lim <= (256 * (ldc_max + 1) + 256) * 4
    p = workloads.custom("bf16", 3, 40, 64, ldc_pad=ldc_max - 40, alpha=1.5, beta=beta, seed=11)
    check_parity(p, run(p, config=tg.TG_CFG_256x256))
    q = workloads.custom("bf16", 3, 40, 64, ldc_pad=ldc_max + 1 - 40, alpha=1.5, beta=beta, seed=11)
    gq = GpuProblem(q)
    gq.reset_c()
    before = gq.cbuf.cpu().numpy().copy()
    with pytest.raises(tg.TileGemmError) as e:
        gq.run(config=tg.TG_CFG_256x256)
    assert e.value.status == tg.TG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.array_equal(gq.cbuf.cpu().numpy().view(np.uint32), before.view(np.uint32))


def test_shared_operand_batch_stride_zero():
    p = workloads.custom("f16", 70, 90, 110, batch=3, alpha=1.0, beta=0.0, seed=6)
    p.strideB = 0
    p.B = p.B[: p.K * p.ldb].copy()
    check_parity(p, run(p))


def test_stream_argument_is_used():
    p = workloads.custom("bf16", 512, 512, 512, seed=8)
    gp = GpuProblem(p)
    gp.reset_c()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gp.run(stream=s)
    s.synchronize()
    check_parity(p, gp.c_view().cpu().numpy().astype(np.float64))


def test_negative_status_on_device_for_bad_args():
    # argument errors are caught before any device work, also with a GPU present
    assert tg.tile_gemm_status("tile_gemm", 4, 4, 4, 1, 0, 4, 0, 4, 0, 3, 1.0, 0.0, 0) == tg.TG_ERR_INVALID_ARG

"""The fused elementwise tail C <- act(alpha A.B + bias) + beta C0 (tile_gemm.h), on the GPU.

* every tile configuration (256 x 256 with its thin strips, 128 x 128, 64 x 64,
  288 x 160, the fp32 tiles), ragged across several tiles, with a per-column bias, a
  per-row bias or none, and ReLU, GELU or no activation, beta zero or not:
  parity with the fp64 oracle over the whole output and no write outside C;
* split along K, where the combine pass applies the tail; thin remainders as
  GEMMs of their own (their slice of the bias); the repacked A; batched with a
  bias stride (0: one vector shared);
* the plan is the one taken without the tail; the argument errors (NULL,
  misaligned or overlapping bias, unknown modes, options the tail is not built
  for);
* ReLU passes a NaN through; full size 8191 x 8193 x 8190 (lda = K + 3,
  ldb = N + 5), sampled.

The parity denominator is everything summed into an output:
|alpha| sum_k |a||b| + |bias| + |beta| |C0|; both activations are 1-Lipschitz
to within 13 %, so an error before the activation stays that size after it.
"""
import numpy as np
import pytest
import torch

import oracle
import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import TOL, GpuProblem, c0_at, need_gpu, parity_error, result_points

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def make_bias(p, mode, stride, seed):
    """Normal bias about the size of alpha * A.B, so ReLU and GELU see both signs."""
    if mode == 0:
        return None
    length = p.N if mode == 1 else p.M
    n = (p.batch - 1) * stride + length
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(max(n, 1)) * abs(p.alpha) * max(p.K, 1) ** 0.5 / 3).astype(np.float32)


def oracle_tail(p, bias, stride, mode, act, pts=None):
    kw = dict(C0=p.C0, ldc=p.ldc, alpha=p.alpha, beta=p.beta, batch=p.batch, strideA=p.strideA,
              strideB=p.strideB, strideC=p.strideC, bias=bias, bias_stride=stride, bias_mode=mode, activation=act)
    if pts is None:
        ref, den = oracle.gemm(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, with_absden=True, **kw)
    else:
        ref, den = oracle.gemm_points(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, pts, **kw)
    return ref, den


def bias_at(p, bias, stride, mode, pts=None):
    """|bias| broadcast to (batch, M, N), or at the points."""
    if mode == 0:
        return 0.0
    if pts is not None:
        idx = pts[:, 0] * stride + (pts[:, 2] if mode == 1 else pts[:, 1])
        return np.abs(bias[idx].astype(np.float64))
    out = np.zeros((p.batch, p.M, p.N))
    for b in range(p.batch):
        v = np.abs(bias[b * stride: b * stride + (p.N if mode == 1 else p.M)].astype(np.float64))
        out[b] = v[None, :] if mode == 1 else v[:, None]
    return out


def run(p, bias_t, stride, mode, act, **opts):
    n = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, bias_mode=mode,
                                    activation=act, **{k: v for k, v in opts.items() if k != "workspace"})
    ws = torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    gp = GpuProblem(p)
    gp.reset_c()
    gp.run(workspace=ws, plan_lda=p.lda, bias=bias_t, bias_stride=stride, bias_mode=mode, activation=act, **opts)
    return gp


def check(p, got, bias, stride, mode, act, pts=None):
    ref, den = oracle_tail(p, bias, stride, mode, act, pts)
    c0 = c0_at(p, pts)
    den = abs(p.alpha) * den + bias_at(p, bias, stride, mode, pts) + abs(p.beta) * np.abs(c0)
    err = parity_error(got, ref, den)
    assert err <= TOL[p.dtype], f"parity error {err:.3e} > {TOL[p.dtype]:.0e}"
    return err


CASES = [
    # dtype, M, N, K, batch, config, split_k, alpha, beta, bias_mode, activation
    ("bf16", 300, 257, 100, 1, tg.TG_CFG_256x256, 1, 1.0, 0.0, 1, 1),     # an N strip and an M strip
    ("bf16", 300, 257, 300, 1, tg.TG_CFG_256x256, 1, 1.5, 0.5, 2, 2),
    ("f16", 520, 600, 700, 1, tg.TG_CFG_256x256, 1, -0.5, 1.0, 1, 2),     # whole fringe tiles
    ("bf16", 256, 512, 64, 1, tg.TG_CFG_256x256, 1, 1.0, 0.0, 0, 1),      # interior only, one K tile
    ("bf16", 300, 257, 100, 1, tg.TG_CFG_128x128, 1, 1.0, 0.0, 1, 1),
    ("bf16", 300, 257, 100, 1, tg.TG_CFG_128x128, 1, 1.5, 0.5, 2, 2),
    ("bf16", 131, 200, 37, 1, tg.TG_CFG_128x128, 1, -1.0, 1.0, 0, 2),
    ("f16", 200, 131, 300, 1, tg.TG_CFG_64x64, 1, 0.75, 0.0, 2, 1),
    ("f16", 257, 129, 1000, 1, tg.TG_CFG_64x64, 1, 1.0, -0.5, 1, 0),
    ("bf16", 97, 65, 40, 1, tg.TG_CFG_64x64, 1, 1.0, 0.0, 0, 1),
    ("f32", 67, 45, 53, 1, tg.TG_CFG_F32_64x64, 1, 1.0, 0.0, 1, 2),
    ("f32", 130, 70, 200, 1, tg.TG_CFG_F32_64x64, 1, 1.5, 0.5, 2, 1),
    ("f32", 300, 257, 100, 1, tg.TG_CFG_256x256, 1, 1.0, 0.5, 1, 2),     # fp32 ring tile with its strips
    ("f32", 131, 200, 37, 1, tg.TG_CFG_128x128, 1, -1.0, 1.0, 2, 1),
    ("f32", 300, 260, 2100, 1, tg.TG_CFG_256x256, 3, 1.0, 0.5, 1, 2),     # fp32 split: the combine applies it
    ("bf16", 300, 260, 2100, 1, tg.TG_CFG_256x256, 3, 1.0, 0.5, 1, 2),     # combine pass applies it
    ("f16", 257, 300, 1300, 1, tg.TG_CFG_128x128, 2, 1.0, 0.0, 2, 1),
    ("f16", 257, 129, 1000, 4, tg.TG_CFG_288x160, 1, 1.0, -0.5, 1, 2),   # one block per problem
    ("bf16", 200, 100, 77, 3, tg.TG_CFG_288x160, 1, 1.5, 0.0, 2, 1),
    ("bf16", 300, 170, 90, 1, tg.TG_CFG_288x160, 1, -1.0, 1.0, 0, 2),    # fringe blocks across both axes
]


@pytest.mark.parametrize("dt,M,N,K,batch,cfg,split,alpha,beta,mode,act", CASES,
                         ids=lambda v: str(v))
def test_fused_tail_parity(dt, M, N, K, batch, cfg, split, alpha, beta, mode, act):
    p = workloads.custom(dt, M, N, K, batch=batch, ldb_pad=3, ldc_pad=2, alpha=alpha, beta=beta,
                         seed=M * 7 + N + K, name="fused")
    bias = make_bias(p, mode, 0, seed=K)
    bias_t = torch.from_numpy(bias).to("cuda") if bias is not None else None
    plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, config=cfg, split_k=split, bias_mode=mode,
                             activation=act, workspace=1 << 40, workspace_bytes=1 << 40)
    assert (plan["config"], plan["split_k"]) == (cfg, split), plan
    gp = run(p, bias_t, 0, mode, act, config=cfg, split_k=split)
    err = check(p, gp.result(), bias, 0, mode, act)
    print(f"{dt} {M}x{N}x{K} cfg {cfg} split {split} bias {mode} act {act}: parity error {err:.3e}")
    gp.check_guards()


@pytest.mark.parametrize("mode,stride", [(1, 0), (1, 300), (2, 0), (2, 250)])
@pytest.mark.parametrize("cfg,split", [(tg.TG_CFG_128x128, 1), (tg.TG_CFG_64x64, 1), (tg.TG_CFG_128x128, 2),
                                       (tg.TG_CFG_F32_64x64, 1), (tg.TG_CFG_288x160, 1)])
def test_fused_tail_batched(mode, stride, cfg, split):
    dt = "f32" if cfg == tg.TG_CFG_F32_64x64 else "bf16"
    p = workloads.custom(dt, 200, 260, 600, batch=3, ldb_pad=1, alpha=1.25, beta=0.5, seed=31, name="fb")
    bias = make_bias(p, mode, stride, seed=stride + mode)
    bias_t = torch.from_numpy(bias).to("cuda")
    gp = run(p, bias_t, stride, mode, 2, config=cfg, split_k=split)
    check(p, gp.result(), bias, stride, mode, 2)
    gp.check_guards()


def test_automatic_plan_256():
    # 4096 x 4096 x 512 takes the 256 x 256 tile, with the tail as without it
    base = tg.tile_gemm_plan(1, 4096, 4096, 512, "bf16")
    assert base["config"] == tg.TG_CFG_256x256
    assert tg.tile_gemm_plan(1, 4096, 4096, 512, "bf16", bias_mode=1) == base
    p = workloads.custom("bf16", 4096, 4096, 512, alpha=1.0, beta=0.0, seed=4, name="auto")
    bias = make_bias(p, 1, 0, seed=4)
    gp = run(p, torch.from_numpy(bias).to("cuda"), 0, 1, 1)
    pts = workloads.sample_points(p, 400)
    check(p, result_points(gp, pts), bias, 0, 1, 1, pts)


def test_relu_passes_nan():
    p = workloads.custom("bf16", 64, 80, 32, seed=9, name="nan")
    bias = make_bias(p, 1, 0, seed=9)
    bias[17] = np.nan
    gp = run(p, torch.from_numpy(bias).to("cuda"), 0, 1, 1, config=tg.TG_CFG_64x64)
    got = gp.result()[0]
    assert np.isnan(got[:, 17]).all()
    keep = np.ones(p.N, bool)
    keep[17] = False
    ref, _ = oracle_tail(p, bias, 0, 1, 1)
    assert not np.isnan(got[:, keep]).any()
    assert np.max(np.abs(got[:, keep] - ref[0][:, keep])) <= 4e-3 * (np.abs(ref[0][:, keep]).max() + 1)


REMAINDER_CASES = [
    # M, N, K, lda_pad, tail_gemm, pack_a, bias_mode, activation, expected (tail_n_splits, tail_m_splits, pack_a)
    (520, 300, 2100, 0, 2, 0, 1, 2, (4, 4, 0)),      # both remainders as GEMMs, split along K
    (520, 300, 2100, 0, 2, 0, 2, 1, (4, 4, 0)),
    (300, 2100, 1100, 3, 2, 0, 1, 1, (2, 2, 1)),     # on the repacked A
    (300, 2100, 1100, 3, 1, 2, 2, 2, (0, 0, 1)),     # strips, repacked A
]


@pytest.mark.parametrize("M,N,K,lpad,tail_gemm,pack,mode,act,expect", REMAINDER_CASES, ids=lambda v: str(v))
def test_fused_tail_remainders_and_repack(M, N, K, lpad, tail_gemm, pack, mode, act, expect):
    p = workloads.custom("bf16", M, N, K, lda_pad=lpad, ldb_pad=2, alpha=1.25, beta=0.5, seed=M + N, name="rem")
    opts = dict(config=tg.TG_CFG_256x256, split_k=1, tail_gemm=tail_gemm, pack_a=pack)
    plan = tg.tile_gemm_plan(1, M, N, K, "bf16", plan_lda=p.lda, bias_mode=mode, activation=act,
                             workspace=1 << 40, workspace_bytes=1 << 40, **opts)
    assert (plan["tail_n_splits"], plan["tail_m_splits"], plan["pack_a"]) == expect, plan
    bias = make_bias(p, mode, 0, seed=K + mode)
    gp = run(p, torch.from_numpy(bias).to("cuda"), 0, mode, act, **opts)
    check(p, gp.result(), bias, 0, mode, act)
    gp.check_guards()


def _status(fn):
    try:
        fn()
        return tg.TG_OK
    except tg.TileGemmError as e:
        return e.status


def test_fused_tail_argument_errors():
    p = workloads.custom("bf16", 64, 64, 256, seed=3, name="err")
    gp = GpuProblem(p)
    bias = torch.zeros(64, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.float32, device="cuda")

    def call(**kw):
        return _status(lambda: gp.run(workspace=ws, **kw))
    assert call(bias_mode=1, bias=None) == tg.TG_ERR_INVALID_ARG             # NULL with a mode
    assert call(bias_mode=0, bias=bias) == tg.TG_ERR_INVALID_ARG             # a bias without a mode
    assert call(bias_mode=3, bias=bias) == tg.TG_ERR_INVALID_ARG
    assert call(activation=3) == tg.TG_ERR_INVALID_ARG
    assert call(bias_mode=1, bias=bias, bias_stride=-1) == tg.TG_ERR_INVALID_ARG
    assert call(bias_mode=1, bias=bias.data_ptr() + 2) == tg.TG_ERR_INVALID_ARG   # misaligned
    assert call(bias_mode=1, bias=gp.C.data_ptr()) == tg.TG_ERR_INVALID_ARG       # overlaps C
    assert call(activation=1, config=tg.TG_CFG_256x256, split_k=1) == tg.TG_OK
    assert call(activation=1, pipeline_depth=2) == tg.TG_ERR_UNSUPPORTED
    assert call(activation=1, swizzle=1) == tg.TG_ERR_UNSUPPORTED
    assert call(activation=1, config=tg.TG_CFG_256x256, split_k=2) == tg.TG_OK              # K in two slices
    assert call(activation=1, config=tg.TG_CFG_256x256, split_k=8) == tg.TG_OK
    torch.cuda.synchronize()
    gp.check_guards()


def test_full_size_ragged_sampled():
    # 8191 x 8193 x 8190, lda = K + 3, ldb = N + 5, alpha 1.5, beta 0.5, per-column bias, GELU
    p = workloads.custom("bf16", 8191, 8193, 8190, lda_pad=3, ldb_pad=5, alpha=1.5, beta=0.5, seed=11,
                         name="fused_full")
    bias = make_bias(p, 1, 0, seed=11)
    plan = tg.tile_gemm_plan(1, p.M, p.N, p.K, p.dtype, plan_lda=p.lda, bias_mode=1, activation=2,
                             workspace=1 << 40, workspace_bytes=1 << 40)
    assert (plan["config"], plan["split_k"], plan["pack_a"]) == (tg.TG_CFG_256x256, 1, 1), plan
    gp = run(p, torch.from_numpy(bias).to("cuda"), 0, 1, 2)
    pts = workloads.sample_points(p, 300)
    err = check(p, result_points(gp, pts), bias, 0, 1, 2, pts)
    print(f"8191 x 8193 x 8190 bias+GELU: sampled parity error {err:.3e} over {len(pts)} outputs")
    gp.check_guards()


@pytest.mark.parametrize("cfg,split", [(tg.TG_CFG_256x256, 1), (tg.TG_CFG_128x128, 1), (tg.TG_CFG_64x64, 1),
                                       (tg.TG_CFG_256x256, 2), (tg.TG_CFG_F32_64x64, 1)])
@pytest.mark.parametrize("mode,act", [(1, 0), (2, 1), (1, 2)])
def test_fused_equals_two_pass(cfg, split, mode, act):
    """OCANNL epilogue fusion: the fused store-back equals the plain GEMM (alpha 1, beta 0, the same
    tile and split) followed by a separate elementwise pass on the GPU.  Bias add and ReLU are
    single roundings, so bit for bit; GELU goes through the library's Chebyshev fit of erfc on one
    side (within 2.4e-7 |x| of x Phi(x)) and the runtime's erf on the other (within about an ulp
    of x), so the two agree to 4 ulp of x."""
    dt = "f32" if cfg == tg.TG_CFG_F32_64x64 else "bf16"
    p = workloads.custom(dt, 300, 270, 700, ldb_pad=2, alpha=1.0, beta=0.0, seed=cfg * 10 + mode + act,
                         name="twopass")
    bias = make_bias(p, mode, 0, seed=cfg + act)
    bias_t = torch.from_numpy(bias).to("cuda")
    fused = run(p, bias_t, 0, mode, act, config=cfg, split_k=split)
    plain = run(p, None, 0, 0, 0, config=cfg, split_k=split)
    y = plain.c_view()[0] + (bias_t[None, :] if mode == 1 else bias_t[:, None])
    if act == 1:
        y = torch.where(y < 0, torch.zeros_like(y), y)
    x = y
    if act == 2:
        y = torch.nn.functional.gelu(x, approximate="none")
    got = fused.c_view()[0]
    torch.cuda.synchronize()
    if act == 2:
        ax = torch.abs(x)
        ulp = torch.nextafter(ax, torch.full_like(ax, float("inf"))) - ax
        err = torch.abs(got - y)
        assert bool(torch.all(err <= 4 * ulp)), float(torch.max(err / ulp))
    else:
        assert torch.equal(got.contiguous().view(torch.int32), y.contiguous().view(torch.int32))
    fused.check_guards()


@pytest.mark.parametrize("split", [1, 2])
def test_gelu_accuracy(split):
    """A = 0, so every output is GELU(bias): a dense grid of x in [-12, 12] plus small and large
    magnitudes, against the oracle's exact erf, to 2.5e-7 |x| (the store-back for split 1, the
    combine pass for split 2)."""
    grid = np.concatenate([np.linspace(-12, 12, 60001), np.geomspace(1e-6, 40, 2000),
                           -np.geomspace(1e-6, 40, 2000), [0.0, -0.0]]).astype(np.float32)
    N = len(grid)
    p = workloads.custom("bf16", 3, N, 64, seed=5, name="gelu")
    p.A = np.zeros_like(p.A)
    gp = run(p, torch.from_numpy(grid).to("cuda"), 0, 1, 2, config=tg.TG_CFG_256x256, split_k=split)
    got = gp.result()[0]
    ref, _ = oracle_tail(p, grid, 0, 1, 2)
    err = np.abs(got - ref[0])
    bound = 2.5e-7 * np.abs(grid.astype(np.float64))[None, :]
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"split {split}: GELU error at most {worst:.3f} of 2.5e-7 |x|")
    assert np.all(err <= bound), worst
    gp.check_guards()


EDGE_CASES = [
    # dtype, M, N, K, batch, config, split_k, alpha, beta, bias_mode, activation
    ("bf16", 100, 70, 0, 1, 0, 0, 1.5, 0.5, 1, 2),        # K = 0: act(bias) + beta C0
    ("f32", 33, 17, 0, 2, 0, 0, 1.0, 0.0, 2, 1),
    ("bf16", 1, 300, 64, 1, 0, 0, 1.0, 0.5, 1, 1),        # one row
    ("f16", 300, 1, 64, 1, 0, 0, 1.0, 0.0, 2, 2),         # one column
    ("bf16", 1, 1, 1, 3, 0, 0, -2.0, 1.0, 1, 2),          # one element per problem, K = 1
    ("f32", 1, 1, 1, 1, 0, 0, 1.0, 0.0, 2, 1),
]


@pytest.mark.parametrize("dt,M,N,K,batch,cfg,split,alpha,beta,mode,act", EDGE_CASES, ids=lambda v: str(v))
def test_fused_tail_degenerate(dt, M, N, K, batch, cfg, split, alpha, beta, mode, act):
    p = workloads.custom(dt, M, N, K, batch=batch, alpha=alpha, beta=beta, seed=M + 3 * N + K, name="edge")
    stride = N if mode == 1 else M
    bias = make_bias(p, mode, stride, seed=7)
    if K == 0:      # the bias alone sets the activation's input: give it both signs at a useful size
        bias = np.random.default_rng(8).standard_normal(len(bias)).astype(np.float32) * 2
    gp = run(p, torch.from_numpy(bias).to("cuda"), stride, mode, act, config=cfg, split_k=split)
    check(p, gp.result(), bias, stride, mode, act)
    gp.check_guards()

"""tile_gemm under HIP graph capture, on the GPU.

A call launches kernels on the caller's stream and nothing else: no allocation, no memset, no
host synchronisation (the device check is cached by the first call).  So a call can be captured
into a HIP graph and replayed.  Each case runs once eagerly, then is captured (C reset from C0
by a copy in the same graph, since beta reads C), and the graph is replayed three times with
eager work and a synchronisation between replays; every replay must equal the eager result bit
for bit.  The cases cover the plain grid, split-K with its combine, the repack of A, strips, the
fused tail and a call on a packed B.
"""
import numpy as np
import pytest
import torch

import tile_scheduled_dense_amd as tg
import workloads
from tests.gpu_util import device_tensor, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = [
    # name, dtype, M, N, K, batch, lda_pad, ldb_pad, beta, options
    ("plain 256", "bf16", 1024, 1024, 512, 1, 0, 0, 0.0, dict()),
    ("split-K", "bf16", 512, 512, 8192, 1, 0, 0, 0.5, dict(split_k=8)),
    ("repacked A + strips", "bf16", 2100, 2053, 700, 1, 3, 5, 1.0, dict(pack_a=2, config=tg.TG_CFG_256x256)),
    ("fused tail", "f16", 1000, 1000, 300, 2, 0, 0, 0.5, dict(bias_mode=1, activation=2)),
    ("fused tail, split", "bf16", 300, 300, 4096, 1, 0, 0, 0.0, dict(bias_mode=2, activation=1, split_k=4)),
    ("fp32", "f32", 300, 200, 100, 3, 1, 1, 0.5, dict()),
    ("packed B", "bf16", 700, 1025, 600, 1, 0, 3, 0.0, dict(packed_b=1)),
]


@pytest.mark.parametrize("name,dt,M,N,K,batch,lpad,bpad,beta,opts", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_equals_eager(name, dt, M, N, K, batch, lpad, bpad, beta, opts):
    opts = dict(opts)
    p = workloads.custom(dt, M, N, K, batch=batch, lda_pad=lpad, ldb_pad=bpad, alpha=1.25, beta=beta, seed=M + K,
                         name="graph")
    stream = torch.cuda.Stream()
    A, B = device_tensor(p.A), device_tensor(p.B)
    ldb, sB = p.ldb, p.strideB
    if opts.pop("packed_b", 0):
        n = tg.tile_gemm_packed_b_size(batch, K, N, dt)
        packed = torch.empty(n // 4 + 64, dtype=torch.float32, device="cuda")
        tg.tile_gemm_pack_b(batch, K, N, dt, B, p.ldb, p.strideB, packed, n)
        B, ldb = packed, tg.tile_gemm_packed_b_ld(N, dt)
        sB = K * ldb
    bias = None
    if opts.get("bias_mode"):
        length = N if opts["bias_mode"] == 1 else M
        bias = torch.from_numpy(np.random.default_rng(3).standard_normal(length).astype(np.float32) * 4).cuda()
    ws_n = tg.tile_gemm_workspace_size(batch, M, N, K, dt, plan_lda=p.lda, **opts)
    ws = torch.empty(max(ws_n, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    c0 = np.zeros(p.sizeC(), np.float32) if p.C0 is None else np.nan_to_num(p.C0, nan=0.0)
    C0 = torch.from_numpy(c0).cuda()
    C = torch.empty_like(C0)

    def call(s):
        tg.tile_gemm_ex(batch, M, N, K, dt, A, p.lda, p.strideA, B, ldb, sB, C, p.ldc, p.strideC, p.alpha, p.beta,
                        s, workspace=ws, plan_lda=p.lda, bias=bias, **opts)

    # eager reference (also warms the device check and the caching allocator)
    with torch.cuda.stream(stream):
        C.copy_(C0)
        call(stream)
    stream.synchronize()
    ref = C.clone()

    graph = torch.cuda.CUDAGraph()
    C.fill_(-7.0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        C.copy_(C0)
        call(torch.cuda.current_stream())
    noise = torch.empty(1 << 20, device="cuda")
    for replay in range(3):
        C.fill_(float(replay) - 3.0)        # eager work between replays
        noise.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), ref.view(torch.int32)), f"{name}: replay {replay} differs"

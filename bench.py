"""Benchmark of the tiled GEMM hot path on one MI355X.

A "step" is one C = alpha*A.B + beta*C through the C ABI over the resident
synthetic inputs of the workload (default: bf16 A, B, fp32 C, M = N = K = 8192,
N(0,1) inputs rounded to bf16, beta = 0).  W untimed warm-up steps, then K
timed steps between two synchronisations, timed with HIP events on the stream
the kernel is launched on.  Prints one JSON line.

The metric covers square and ragged extents, so with the default workload the
same run then times the ragged problem (bf16 8191 x 8193 x 8190, lda = K + 3,
ldb = N + 5, alpha = 1.5, beta = 0.5) the same way, W warm-up and K timed
steps of its own, and reports it in the line's "ragged" object.  During every
timed region the driver's current shader-clock level (pp_dpm_sclk) and the
board power (hwmon power1_input) are sampled (file reads, no program is
started).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--ragged NAME|none] [--no-cpu-baseline]

The CPU-baseline leg times the fp64 oracle (test infrastructure, untuned) on a
bounded band of output rows of the same workload, and on the whole small fp32
problem (67 x 45 x 53) on one thread and on all of them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the GPU takes a few dozen launches to reach its sustained clock")
    ap.add_argument("--workload", default="c2_bf16_8192")
    ap.add_argument("--ragged", default="c3_bf16_ragged",
                    help="with the default workload, the ragged workload timed in the same run ('none': skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline duration")
    ap.add_argument("--config", type=int, default=0, help="force a tile configuration (tg_config)")
    ap.add_argument("--pipeline-depth", type=int, default=0)
    ap.add_argument("--swizzle", type=int, default=0)
    ap.add_argument("--block-order", type=int, default=0)
    ap.add_argument("--split-k", type=int, default=0,
                    help="K slices (0 = automatic with the workspace the library asks for, 1 = off)")
    ap.add_argument("--pack-a", type=int, default=0,
                    help="repack misaligned A rows into the workspace (0 = automatic, 1 = never, 2 = always)")
    ap.add_argument("--tail-gemm", type=int, default=0,
                    help="thin N/M remainder as a GEMM of its own (0, 1 = strips in the grid, 2 = always)")
    ap.add_argument("--persistent", type=int, default=0,
                    help="persistent workgroups (0, 1 = the plain grid; 2 = persistent where the plan allows)")
    ap.add_argument("--bias-mode", type=int, default=0,
                    help="fused tail bias: 0 none, 1 one value per column, 2 one per row (seeded normal)")
    ap.add_argument("--activation", type=int, default=0, help="fused tail activation: 0 none, 1 ReLU, 2 GELU")
    ap.add_argument("--packed-b", type=int, default=0,
                    help="B packed once before the timed calls by tile_gemm_pack_b (1: from B as stored, "
                         "2: from its transpose); the calls read the packed copy, the pack is timed apart")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times) so HBM "
                         "byte counters can be scaled against a kernel of known traffic")
    return ap.parse_args()


def tail_args(p, bias, bias_mode, activation, row0, rows):
    """The oracle's fused-tail arguments for output rows [row0, row0 + rows) (one shared bias vector)."""
    if bias is None:
        return dict(activation=activation)
    b = bias if bias_mode == 1 else bias[row0: row0 + rows]
    return dict(bias=b, bias_stride=0, bias_mode=bias_mode, activation=activation)


def cpu_baseline(p, seconds, bias=None, bias_mode=0, activation=0):
    """The oracle on rows [0, R) of the workload's output, R grown until ~`seconds` of work."""
    import numpy as np

    import oracle
    from workloads import Problem
    threads = oracle.max_threads()
    rows_done, flops, t_total = 0, 0.0, 0.0
    band = 8
    while t_total < seconds and rows_done < p.M:
        r = min(band, p.M - rows_done)
        sub = Problem("band", p.dtype, r, p.N, p.K, lda=p.lda, ldb=p.ldb, ldc=p.ldc, alpha=p.alpha, beta=p.beta)
        A = np.ascontiguousarray(p.A[rows_done * p.lda: rows_done * p.lda + r * p.lda])
        C0 = None
        if p.beta != 0:
            C0 = np.ascontiguousarray(p.C0[rows_done * p.ldc: rows_done * p.ldc + r * p.ldc])
        t = time.perf_counter()
        oracle.gemm(r, p.N, p.K, p.dtype, A, p.lda, p.B, p.ldb, C0=C0, ldc=p.ldc, alpha=p.alpha, beta=p.beta,
                    **tail_args(p, bias, bias_mode, activation, rows_done, r))
        t_total += time.perf_counter() - t
        rows_done += r
        flops += 2.0 * r * p.N * p.K
        band = min(band * 2, 256)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"output rows 0..{rows_done - 1} of {p.name} ({rows_done}x{p.N}x{p.K}, batch 0), "
                      f"fp64 triple loop, {t_total:.1f} s"}


def oracle_small_latency(reps=200):
    """The oracle on the whole small fp32 problem (67x45x53), mean wall time per call on one
    thread and on all of them (a latency, not a throughput: the problem is 3.2e5 flops)."""
    import oracle
    import workloads
    q = workloads.config("c1_f32_67x45x53")
    out = {"problem": f"{q.name} ({q.M}x{q.N}x{q.K}, whole output)", "reps": reps}
    threads = oracle.max_threads()
    try:
        for n, key in ((1, "one_thread_us"), (threads, "all_threads_us")):
            oracle.set_threads(n)
            oracle.gemm(q.M, q.N, q.K, q.dtype, q.A, q.lda, q.B, q.ldb, ldc=q.ldc)    # warm
            t = time.perf_counter()
            for _ in range(reps):
                oracle.gemm(q.M, q.N, q.K, q.dtype, q.A, q.lda, q.B, q.ldb, ldc=q.ldc)
            out[key] = round((time.perf_counter() - t) / reps * 1e6, 1)
        out["threads"] = threads
    finally:
        oracle.set_threads(threads)
    return out


def oracle_rows(p, rows, bias=None, bias_mode=0, activation=0):
    """The oracle's rows [0, rows) of batch entry 0 and their sum_k |a||b| (not timed)."""
    import numpy as np

    import oracle
    A = np.ascontiguousarray(p.A[: rows * p.lda])
    C0 = np.ascontiguousarray(p.C0[: rows * p.ldc]) if p.beta != 0 else None
    ref, den = oracle.gemm(rows, p.N, p.K, p.dtype, A, p.lda, p.B, p.ldb, C0=C0, ldc=p.ldc, alpha=p.alpha,
                           beta=p.beta, with_absden=True, **tail_args(p, bias, bias_mode, activation, 0, rows))
    return ref[0], den[0]


def rocm_environment():
    """ROCm version and the GPU clock levels from the driver's sysfs files, best effort.

    Files only: no program is started from this process, which has the GPU open."""
    import glob
    env = {"rocm_version": None, "clocks": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm_version"] = f.read().strip()
    except OSError:
        pass
    clocks = []
    for kind in ("sclk", "mclk", "fclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}"))[:1]:
            try:
                with open(path) as f:
                    cur = [l.strip() for l in f if l.strip().endswith("*")]
                clocks.append(f"{kind}: {cur[0] if cur else 'unknown'}")
            except OSError:
                pass
    env["clocks"] = clocks or None
    return env


class ClockSampler:
    """Shader-clock and board-power samples while a timed region runs.

    The amdgpu driver marks the current shader clock with '*' in
    /sys/class/drm/cardN/device/pp_dpm_sclk (a line "S: <MHz>Mhz *" or a level
    line) and reports the board power in microwatts in
    .../device/hwmon/hwmonM/power1_input; the card is the one at the GPU's PCI
    address.  A background thread reads those files every 5 ms: file reads, no
    program is started from this process, which has the GPU open."""

    def __init__(self, props):
        import glob
        self.sclk = self.power = None
        want = None
        try:
            want = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}."
        except AttributeError:
            pass
        cards = sorted(glob.glob("/sys/class/drm/card[0-9]*/device"))
        pick = [c for c in cards if want and os.path.basename(os.path.realpath(c)).startswith(want)]
        if not pick and len(cards) == 1:
            pick = cards
        if pick:
            d = pick[0]
            if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                self.sclk = os.path.join(d, "pp_dpm_sclk")
            pw = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input")))
            self.power = pw[0] if pw else None
        self.samples, self.watts = [], []
        self._stop = None
        self._thread = None

    def _read_sclk(self):
        try:
            with open(self.sclk) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        mhz = line.split(":", 1)[1].strip().split("Mhz")[0]
                        return float(mhz)
        except (OSError, ValueError, IndexError):
            pass
        return None

    def _read_power(self):
        try:
            with open(self.power) as f:
                return int(f.read().strip()) / 1e6
        except (OSError, ValueError):
            return None

    def start(self):
        import threading
        self.samples, self.watts = [], []
        if self.sclk is None and self.power is None:
            return
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                if self.sclk:
                    v = self._read_sclk()
                    if v is not None:
                        self.samples.append(v)
                if self.power:
                    w = self._read_power()
                    if w is not None:
                        self.watts.append(w)
                self._stop.wait(0.005)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        out = {"source": "pp_dpm_sclk (current) and hwmon power1_input", "samples": len(self.samples)}
        s = sorted(self.samples)
        if s:
            out.update({"min_mhz": round(s[0]), "median_mhz": round(s[len(s) // 2]), "max_mhz": round(s[-1]),
                        "in_order_mhz": [round(x) for x in self.samples[:400]]})
        w = sorted(self.watts)
        if w:
            out.update({"power_median_w": round(w[len(w) // 2], 1), "power_max_w": round(w[-1], 1)})
        return out


def time_steps(step, stream, warmup, steps, clock):
    """W untimed calls, then K timed ones between two synchronisations: HIP events on
    the launch stream around the whole region and between consecutive steps."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    clock.start()
    t0 = time.perf_counter()
    start.record(stream)
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk = clock.stop()
    ms_total = start.elapsed_time(end)
    in_order = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    per_step = sorted(in_order)
    stats = {"median_ms": round(per_step[len(per_step) // 2], 4), "min_ms": round(per_step[0], 4),
             "p90_ms": round(per_step[min(len(per_step) - 1, int(0.9 * len(per_step)))], 4),
             "in_order_ms": [round(x, 4) for x in in_order]}
    return ms_total, wall, stats, clk


def upload(p):
    import numpy as np
    import torch
    to_dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")
    A, B = to_dev(p.A), to_dev(p.B)
    C = to_dev(p.C0.copy()) if p.beta != 0 else torch.zeros(p.sizeC(), dtype=torch.float32, device="cuda")
    return A, B, C, to_dev


def roofline_of(p, ms_step, traffic):
    """The binding roof: MFMA when the workload's intensity (algorithmic flops per
    compulsory byte) is above the ridge peak / HBM bandwidth, else HBM."""
    tflops = p.flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.dtype]
    bytes_alg = p.compulsory_bytes()
    gbs = bytes_alg / (ms_step * 1e-3) / 1e9
    hbm_bound = p.flops / bytes_alg < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4)}
    roofline.update({"traffic": None if traffic is None else int(traffic),
                     "algorithmic_flops_per_launch": p.flops, "algorithmic_bytes_per_launch": bytes_alg,
                     "avg_launch_us": round(ms_step * 1e3, 2), "achieved_TFLOPs": round(tflops, 2),
                     "mfma_frac": round(tflops / peak, 4), "achieved_GBps": round(gbs, 1)})
    return roofline, tflops


def plan_config(p, plan, extra=None):
    cfg = {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
           "lda": p.lda, "ldb": p.ldb, "ldc": p.ldc, "alpha": p.alpha, "beta": p.beta,
           "inputs": f"{p.dist} seed {p.seed}", "accumulate": "fp32", "output": "fp32",
           "tile": f"{plan['block_m']}x{plan['block_n']}x{plan['block_k']}",
           "pipeline_depth": plan["pipeline_depth"], "split_k": plan["split_k"],
           "pack_a": plan["pack_a"], "strip_blocks": plan["strip_blocks"], "strip_splits": plan["strip_splits"],
           "tail_n_splits": plan["tail_n_splits"], "tail_m_splits": plan["tail_m_splits"],
           "persistent": plan["persistent"]}
    cfg.update(extra or {})
    cfg["grid"] = plan["grid"]
    return cfg


def band_error(tg, p, A, B, call_opts, stream, rows_list, to_dev):
    """Observed parity error on whole output rows: one fresh call (C reset to C0),
    the oracle on those rows, the stated metric max |C - C_ref| / (sum |a||b| + 1e-30)."""
    import numpy as np
    import torch

    import oracle
    Cf = to_dev(p.C0.copy()) if p.beta != 0 else torch.zeros(p.sizeC(), dtype=torch.float32, device="cuda")
    tg.tile_gemm_ex(p.batch, p.M, p.N, p.K, p.dtype, A, p.lda, p.strideA, B, p.ldb, p.strideB,
                    Cf, p.ldc, p.strideC, p.alpha, p.beta, stream, **call_opts)
    torch.cuda.synchronize()
    worst = 0.0
    for r0, r in rows_list:
        got = Cf[r0 * p.ldc: (r0 + r) * p.ldc].view(r, p.ldc)[:, : p.N].cpu().numpy().astype(np.float64)
        A_band = np.ascontiguousarray(p.A[r0 * p.lda: (r0 + r) * p.lda])
        C0 = np.ascontiguousarray(p.C0[r0 * p.ldc: (r0 + r) * p.ldc]) if p.beta != 0 else None
        ref, den = oracle.gemm(r, p.N, p.K, p.dtype, A_band, p.lda, p.B, p.ldb, C0=C0, ldc=p.ldc, alpha=p.alpha,
                               beta=p.beta, with_absden=True)
        worst = max(worst, float(np.max(np.abs(got - ref[0]) / (den[0] + 1e-30))))
    return worst


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tile_scheduled_dense_amd as tg
    import workloads
    from tile_scheduled_dense_amd.rocprof_summary import traffic_for

    if not args.no_cpu_baseline:
        import oracle
        oracle.load()       # compiled, if it must be, before the GPU is opened
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    clock = ClockSampler(props)

    p = workloads.config(args.workload)
    print(f"# workload {p.name}: {p.batch}x{p.M}x{p.N}x{p.K} {p.dtype}", file=sys.stderr, flush=True)
    A, B, C, to_dev = upload(p)
    stream = torch.cuda.current_stream()
    opts = dict(config=args.config, pipeline_depth=args.pipeline_depth, swizzle=args.swizzle,
                block_order=args.block_order, split_k=args.split_k, pack_a=args.pack_a, plan_lda=p.lda,
                plan_ldb=p.ldb,
                tail_gemm=args.tail_gemm, persistent=args.persistent, bias_mode=args.bias_mode,
                activation=args.activation)
    # fused tail: one seeded bias vector shared by the batch, about the size of alpha * A.B
    bias_np = None
    if args.bias_mode:
        n_bias = p.N if args.bias_mode == 1 else p.M
        bias_np = (np.random.default_rng(p.seed + 101).standard_normal(n_bias)
                   * abs(p.alpha) * max(p.K, 1) ** 0.5 / 3).astype(np.float32)
    call_opts = dict(bias=torch.from_numpy(bias_np).to("cuda") if bias_np is not None else None)
    # workspace (split-K partials, the aligned copy of A, remainder partials): allocated once, outside
    # the timed region, as a caller would
    ws_bytes = tg.tile_gemm_workspace_size(p.batch, p.M, p.N, p.K, p.dtype, **opts)
    if ws_bytes:
        opts["workspace"] = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    plan = tg.tile_gemm_plan(p.batch, p.M, p.N, p.K, p.dtype, **opts)
    call_opts.update(opts)

    # hoisted pack of B: once, outside the timed region, as a caller with fixed weights would
    B_call, ldb_call, sB_call, pack_info = B, p.ldb, p.strideB, None
    if args.packed_b:
        ld = tg.tile_gemm_packed_b_ld(p.N, p.dtype)
        n_packed = tg.tile_gemm_packed_b_size(p.batch, p.K, p.N, p.dtype)
        packed = torch.empty(max(n_packed, 256) // 4 + 64, dtype=torch.float32, device="cuda")
        if args.packed_b == 2:      # the source kept as B's transpose: N x K rows per batch entry
            Bd = torch.as_strided(B, (p.batch, p.K, p.N), (p.strideB, p.ldb, 1))
            src, src_ld, src_stride, tr = Bd.transpose(1, 2).contiguous(), p.K, p.K * p.N, 1
        else:
            src, src_ld, src_stride, tr = B, p.ldb, p.strideB, 0
        pack = lambda: tg.tile_gemm_pack_b(p.batch, p.K, p.N, p.dtype, src, src_ld, src_stride, packed, n_packed,
                                           transposed=tr, stream=stream)
        for _ in range(3):
            pack()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            pack()
        e1.record(stream)
        torch.cuda.synchronize()
        pack_us = e0.elapsed_time(e1) / 10 * 1e3
        esz = 4 if p.dtype == "f32" else 2
        moved = p.batch * p.K * (p.N + ld) * esz          # read B once, write the packed rows
        pack_info = {"source": "transposed" if tr else "as stored", "ldb_packed": ld, "pack_us": round(pack_us, 2),
                     "pack_GBps": round(moved / (pack_us * 1e-6) / 1e9, 1)}
        B_call, ldb_call, sB_call = packed, ld, p.K * ld

    def step():
        tg.tile_gemm_ex(p.batch, p.M, p.N, p.K, p.dtype, A, p.lda, p.strideA, B_call, ldb_call, sB_call,
                        C, p.ldc, p.strideC, p.alpha, p.beta, stream, **call_opts)

    # The ragged workload is prepared before anything is timed, so its timed steps
    # follow the square ones with no idle gap on the GPU.
    do_ragged = (args.ragged != "none" and args.workload == "c2_bf16_8192" and not args.packed_b and
                 not args.bias_mode and not args.activation and args.config == 0 and args.split_k == 0)
    if do_ragged:
        q = workloads.config(args.ragged)
        print(f"# workload {q.name}: {q.batch}x{q.M}x{q.N}x{q.K} {q.dtype}", file=sys.stderr, flush=True)
        qA, qB, qC, _ = upload(q)
        qopts = dict(plan_lda=q.lda, plan_ldb=q.ldb, pipeline_depth=args.pipeline_depth, swizzle=args.swizzle,
                     block_order=args.block_order)
        q_ws = tg.tile_gemm_workspace_size(q.batch, q.M, q.N, q.K, q.dtype, **qopts)
        if q_ws:
            qopts["workspace"] = torch.empty(q_ws // 4, dtype=torch.float32, device="cuda")
        qplan = tg.tile_gemm_plan(q.batch, q.M, q.N, q.K, q.dtype, **qopts)

        def qstep():
            tg.tile_gemm_ex(q.batch, q.M, q.N, q.K, q.dtype, qA, q.lda, q.strideA, qB, q.ldb, q.strideB,
                            qC, q.ldc, q.strideC, q.alpha, q.beta, stream, **qopts)

    ms_total, wall, step_stats, clk = time_steps(step, stream, args.warmup, args.steps, clock)
    ms_step = ms_total / args.steps
    print(f"# {args.steps} steps: {ms_total:.3f} ms on the stream, {wall * 1e3:.3f} ms wall",
          file=sys.stderr, flush=True)

    # The ragged half of the metric, in the same run: its own W warm-up and K timed steps.
    ragged = None
    if do_ragged:
        q_total, q_wall, q_stats, q_clk = time_steps(qstep, stream, args.warmup, args.steps, clock)
        q_ms = q_total / args.steps
        print(f"# {args.steps} steps: {q_total:.3f} ms on the stream, {q_wall * 1e3:.3f} ms wall",
              file=sys.stderr, flush=True)
        q_roof, q_tflops = roofline_of(q, q_ms, traffic_for(q.name))
        ragged = {"metric": "GEMM TFLOP/s, ragged extents", "value": round(q_tflops, 2), "unit": "TFLOP/s",
                  "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(q_ms, 4),
                  "config": plan_config(q, qplan), "roofline": q_roof, "step_stats": q_stats, "sclk": q_clk}
        if not args.no_cpu_baseline:
            # whole rows through the first tile row and the fringe tile row (the last column is a strip)
            ragged["parity_max_rel_err"] = band_error(tg, q, qA, qB, qopts, stream, [(0, 8), (q.M - 4, 4)],
                                                      lambda a: torch.from_numpy(a).to("cuda"))
            ragged["parity_sample"] = (f"output rows 0..7 and {q.M - 4}..{q.M - 1}, metric max |C - C_ref| / "
                                       "(sum |a||b| + 1e-30)")
        del qA, qB, qC
        qopts.pop("workspace", None)

    # Each step is one call: one launch of the GEMM kernel, or with split-K the
    # partial-product launch and its combine; the event time per step is the
    # whole call (plus launch gaps), so a split call is charged for both passes.
    # HBM traffic per launch from the committed FETCH_SIZE / WRITE_SIZE summary
    # of this workload, only while it was taken on the current kernel sources.
    roofline, tflops = roofline_of(p, ms_step, traffic_for(p.name))
    bytes_alg = p.compulsory_bytes()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy calibration: 3 x {args.copy_calibration_mib} MiB read + written", file=sys.stderr)
        del src, dst

    # HBM-bound workloads: the same calls with a 512 MiB write between them, so
    # no operand is still in the 256 MB last-level cache when a call starts
    flushed = None
    if roofline["bound"] == "hbm":
        scratch = torch.empty(512 << 18, dtype=torch.float32, device="cuda")
        n_fl = min(args.steps, 20)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_fl)]
        for a, b in ev:
            scratch.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        fl = sorted(a.elapsed_time(b) for a, b in ev)
        fl_ms = fl[len(fl) // 2]
        flushed = {"median_ms": round(fl_ms, 4), "steps": n_fl,
                   "achieved_GBps": round(bytes_alg / (fl_ms * 1e-3) / 1e9, 1),
                   "frac": round(bytes_alg / (fl_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del scratch

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, args.cpu_seconds, bias_np, args.bias_mode, args.activation)
        cpu["small_fp32_oracle"] = oracle_small_latency()
        # the observed parity error on the oracle's first rows: one fresh call
        # (C reset to C0), compared with the stated metric
        rows = min(8, p.M)
        Cf = to_dev(p.C0.copy()) if p.beta != 0 else torch.zeros(p.sizeC(), dtype=torch.float32, device="cuda")
        tg.tile_gemm_ex(p.batch, p.M, p.N, p.K, p.dtype, A, p.lda, p.strideA, B_call, ldb_call, sB_call,
                        Cf, p.ldc, p.strideC, p.alpha, p.beta, stream, **call_opts)
        torch.cuda.synchronize()
        got = Cf[: rows * p.ldc].view(rows, p.ldc)[:, : p.N].cpu().numpy().astype(np.float64)
        ref, den = oracle_rows(p, rows, bias_np, args.bias_mode, args.activation)
        if bias_np is not None:     # the bias is summed into the output too
            den = den + np.abs(bias_np[None, :] if args.bias_mode == 1 else bias_np[:rows, None])
        cpu["parity_max_rel_err"] = float(np.max(np.abs(got - ref) / (den + 1e-30)))
        cpu["parity_sample"] = f"output rows 0..{rows - 1}, batch 0, metric max |C - C_ref| / (sum |a||b| + 1e-30)"

    line = {
        "metric": "GEMM TFLOP/s and % of MI355X MFMA peak, square + ragged extents, 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": plan_config(p, plan, {"bias_mode": args.bias_mode, "activation": args.activation,
                                        "packed_b": pack_info}),
        "roofline": roofline,
        "step_stats": step_stats,
        "sclk": clk,
        "ragged": ragged,
        "cache_flushed": flushed,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, **rocm_environment()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

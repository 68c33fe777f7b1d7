"""Summaries of rocprofv3 CSV output for the GEMM kernel, and the traffic figure
bench.py reports.

  python -m tile_scheduled_dense_amd.rocprof_summary trace  <kernel_stats.csv> <out.txt> <command...>
  python -m tile_scheduled_dense_amd.rocprof_summary timed  <kernel_stats.csv> <kernel_trace.csv> <K> <out.txt> <command...>
  python -m tile_scheduled_dense_amd.rocprof_summary window <kernel_stats.csv> <kernel_trace.csv> <label:first:count,...> <out.txt> <command...>
  python -m tile_scheduled_dense_amd.rocprof_summary counters <fetch_dir> <write_dir> <copy_mib> <out.txt> <command...>
  python -m tile_scheduled_dense_amd.rocprof_summary sq <sq_dir> <trace_kernel_stats.csv> <out.txt> <command...>

`counters` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) of a command that also ran a plain device copy of `copy_mib` MiB
(bench.py --copy-calibration-mib).  Each counter is scaled by what it reads for
that copy, whose true traffic is known (copy_mib read and copy_mib written).
The summary records a hash of the kernel sources; bench.py reports the traffic
only while the sources still match.

`timed` is `trace` plus the mean duration of the last K dispatches of the GEMM
kernel (the K timed steps of a bench.py run, after its warm-up), the figure to
set beside bench.py's own HIP-event time per launch.

`window` is `trace` plus the mean duration of GEMM dispatches first .. first +
count - 1 for each labelled window: the timed steps of a bench.py run by their
position (W warm-up steps come first; the ragged workload's steps, cache-flushed
calls or a parity call may follow).

`sq` averages the SQ/GRBM counters of one --pmc run over the GEMM dispatches
and derives the shader clock (GRBM_GUI_ACTIVE counts cycles on each of the 8
XCDs) and the fraction of SIMD cycles the matrix cores were busy.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
GEMM_KERNEL_TAG = "tg::gemm"     # gemm_kernel (fp32), gemm_ring_kernel, gemm_ring_chain_kernel and gemm_ring_persistent_kernel


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _counter_file(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return files[0]


def per_kernel(path, counter):
    """{kernel name: [values per dispatch]} for one counter."""
    out = {}
    for r in _rows(path):
        if r["Counter_Name"] == counter:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(d, tag):
    for k, v in d.items():
        if tag in k:
            return k, v
    raise KeyError(tag)


def summarize_counters(fetch_dir, write_dir, copy_mib):
    fetch = per_kernel(_counter_file(fetch_dir), "FETCH_SIZE")
    write = per_kernel(_counter_file(write_dir), "WRITE_SIZE")
    name, fk = _pick(fetch, GEMM_KERNEL_TAG)
    _, wk = _pick(write, GEMM_KERNEL_TAG)
    _, fc = _pick(fetch, "copyBuffer")
    _, wc = _pick(write, "copyBuffer")
    copy_kib = copy_mib * 1024.0
    f_factor = (sum(fc) / len(fc)) / copy_kib
    w_factor = (sum(wc) / len(wc)) / copy_kib
    fetch_kib = sum(fk) / len(fk)
    write_kib = sum(wk) / len(wk)
    return {
        "kernel": name,
        "dispatches_fetch": len(fk), "dispatches_write": len(wk),
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "copy_mib": copy_mib, "copy_fetch_factor": f_factor, "copy_write_factor": w_factor,
        "hbm_read_bytes_per_launch": fetch_kib / f_factor * 1024.0,
        "hbm_write_bytes_per_launch": write_kib / w_factor * 1024.0,
        "traffic_bytes_per_launch": (fetch_kib / f_factor + write_kib / w_factor) * 1024.0,
        "kernel_source_sha256": kernel_source_hash(),
    }


def write_kv(path, title, command, kv):
    with open(path, "w") as f:
        f.write(f"# {title}\n# command: {command}\n")
        for k, v in kv.items():
            f.write(f"{k}: {v}\n")


def read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def traffic_for(workload: str):
    """Bytes per launch from profiles/traffic_<workload>.txt if it matches the sources, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = read_kv(path)
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def summarize_sq(sq_dir, stats_csv):
    rows = _rows(_counter_file(sq_dir))
    vals = {}
    for r in rows:
        if GEMM_KERNEL_TAG in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {k: sum(v) / len(v) for k, v in sorted(vals.items())}
    _, d = _pick(summarize_trace(stats_csv), GEMM_KERNEL_TAG)
    dur_ns = d["average_ns"]
    out["kernel_duration_ns (from the kernel trace)"] = dur_ns
    if "GRBM_GUI_ACTIVE" in out:
        cycles = out["GRBM_GUI_ACTIVE"] / 8.0
        out["derived_clock_GHz (GRBM_GUI_ACTIVE / 8 XCDs / duration)"] = round(cycles / dur_ns, 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in out:
            out["derived_mfma_busy_fraction (MFMA busy / (1024 SIMDs x cycles))"] = round(
                out["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * cycles), 3)
    if "SQ_LDS_BANK_CONFLICT" in out and out.get("SQ_LDS_IDX_ACTIVE"):
        out["derived_lds_conflict_fraction"] = round(out["SQ_LDS_BANK_CONFLICT"] / out["SQ_LDS_IDX_ACTIVE"], 4)
    out["kernel_source_sha256"] = kernel_source_hash()
    return out


def summarize_trace(stats_csv):
    rows = _rows(stats_csv)
    out = {}
    for r in rows:
        out[r["Name"]] = {"calls": int(r["Calls"]), "average_ns": float(r["AverageNs"]),
                          "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                          "percentage": float(r["Percentage"])}
    return out


def timed_average_ns(trace_csv, k):
    """Mean duration of the last k dispatches of the GEMM kernel (in dispatch order)."""
    rows = [r for r in _rows(trace_csv) if GEMM_KERNEL_TAG in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-k:]
    return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in last) / len(last), len(rows)


def window_average_ns(trace_csv, first, count):
    """Mean duration of GEMM dispatches first .. first + count - 1 (in dispatch order): the timed
    steps of a bench.py run, which follow its warm-up steps (further calls may come after)."""
    rows = [r for r in _rows(trace_csv) if GEMM_KERNEL_TAG in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    sel = rows[first:first + count]
    if len(sel) < count:
        raise SystemExit(f"only {len(rows)} GEMM dispatches, window {first}+{count}")
    return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel) / len(sel), len(rows)


def main(argv):
    mode = argv[1]
    if mode == "timed":
        stats, trace, k, out, cmd = argv[2], argv[3], int(argv[4]), argv[5], " ".join(argv[6:])
        kv = {}
        for name, d in summarize_trace(stats).items():
            short = name if len(name) < 120 else name[:117] + "..."
            kv[short] = (f"calls={d['calls']} average_us={d['average_ns'] / 1e3:.2f} "
                         f"min_us={d['min_ns'] / 1e3:.2f} max_us={d['max_ns'] / 1e3:.2f} pct={d['percentage']:.2f}")
        avg, n = timed_average_ns(trace, k)
        kv[f"gemm_timed_average_us (last {k} of {n} GEMM dispatches)"] = f"{avg / 1e3:.2f}"
        kv["kernel_source_sha256"] = kernel_source_hash()
        write_kv(out, "rocprofv3 --kernel-trace --stats summary", cmd, kv)
    elif mode == "window":
        # windows: label:first:count[,label:first:count...]
        stats, trace, windows, out, cmd = argv[2], argv[3], argv[4], argv[5], " ".join(argv[6:])
        kv = {}
        for name, d in summarize_trace(stats).items():
            short = name if len(name) < 120 else name[:117] + "..."
            kv[short] = (f"calls={d['calls']} average_us={d['average_ns'] / 1e3:.2f} "
                         f"min_us={d['min_ns'] / 1e3:.2f} max_us={d['max_ns'] / 1e3:.2f} pct={d['percentage']:.2f}")
        for w in windows.split(","):
            label, first, count = w.split(":")
            avg, n = window_average_ns(trace, int(first), int(count))
            kv[f"gemm_timed_average_us {label} (GEMM dispatches {first}..{int(first) + int(count) - 1} of {n})"] = \
                f"{avg / 1e3:.2f}"
        kv["kernel_source_sha256"] = kernel_source_hash()
        write_kv(out, "rocprofv3 --kernel-trace --stats summary", cmd, kv)
    elif mode == "trace":
        stats, out, cmd = argv[2], argv[3], " ".join(argv[4:])
        kv = {}
        for name, d in summarize_trace(stats).items():
            short = name if len(name) < 120 else name[:117] + "..."
            kv[short] = (f"calls={d['calls']} average_us={d['average_ns'] / 1e3:.2f} "
                         f"min_us={d['min_ns'] / 1e3:.2f} max_us={d['max_ns'] / 1e3:.2f} pct={d['percentage']:.2f}")
        kv["kernel_source_sha256"] = kernel_source_hash()
        write_kv(out, "rocprofv3 --kernel-trace --stats summary", cmd, kv)
    elif mode == "counters":
        fetch_dir, write_dir, copy_mib, out, cmd = argv[2], argv[3], int(argv[4]), argv[5], " ".join(argv[6:])
        write_kv(out, "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, scaled by a plain copy of known size", cmd,
                 summarize_counters(fetch_dir, write_dir, copy_mib))
    elif mode == "sq":
        sq_dir, stats, out, cmd = argv[2], argv[3], argv[4], " ".join(argv[5:])
        write_kv(out, "rocprofv3 --pmc SQ counters of the GEMM kernel, averaged over dispatches", cmd,
                 summarize_sq(sq_dir, stats))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)

"""The C ABI from C: tests/c/abi_host.c, compiled by gcc as C11 against include/tile_gemm.h and
linked to the built library, answers the host-only queries the same way the Python binding
does (no GPU: plans, sizes and argument errors are decided before any device work)."""
import os
import shutil
import subprocess

import pytest

import tile_scheduled_dense_amd as tg

pytestmark = pytest.mark.spawns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_caller(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    lib = tg.library_path()
    exe = tmp_path / "abi_host"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", str(exe), lib,
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert got["abi_version"] == str(tg.abi_version())
    assert got["status_invalid"] == "ok"
    assert got["plan_status"] == "0"
    c2 = tg.tile_gemm_plan(1, 8192, 8192, 8192, "bf16")
    assert got["plan_c2"] == f"{c2['config']} {c2['block_m']} {c2['block_n']} {c2['grid']}"
    c3 = tg.tile_gemm_plan(1, 8191, 8193, 8190, "bf16", bias_mode=1, activation=2)
    assert got["plan_c3_tail"] == f"0 {c3['config']} {c3['strip_blocks']}"
    ws = tg.tile_gemm_workspace_size(1, 512, 512, 131072, "bf16", split_k=4)
    assert got["workspace_split4"] == f"0 {ws}" and ws == 4 * 512 * 512 * 4
    assert got["packed_ld"] == f"{tg.tile_gemm_packed_b_ld(8193, 'bf16')} {tg.tile_gemm_packed_b_ld(45, 'f32')}"
    assert got["packed_size"] == f"0 {tg.tile_gemm_packed_b_size(3, 100, 129, 'f16')}"
    for key in ("err_negative", "err_null", "err_lda", "err_pack_align"):
        assert got[key] == str(tg.TG_ERR_INVALID_ARG), (key, got[key])

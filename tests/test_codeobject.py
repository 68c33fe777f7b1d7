"""Checks on the gfx950 code object of the built library (its AMD assembly).

The buffer-to-LDS copies are inline assembly that sets M0 (the LDS base of a
copy group) and declares it clobbered instead of saving and restoring it; that
is only sound while the compiler itself keeps nothing in M0.  This scans the
disassembly for every M0 access and requires each to be one of the copy
groups: `s_mov_b32 m0, <scalar register>`, `s_nop 0`, then the group's `buffer_load_dwordx4
... lds` instructions, and every such load to follow an M0 write of its group.
"""
import os
import re
import shutil
import subprocess

import pytest

import tile_scheduled_dense_amd as tg

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


def _disassembly(tmp_path):
    lib = tg.library_path()
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not installed")
    local = tmp_path / "lib.so"
    shutil.copy(lib, local)
    # --offloading writes the bundled code objects next to the input
    subprocess.run([OBJDUMP, "--offloading", str(local)], check=True, capture_output=True, cwd=tmp_path)
    objs = [p for p in tmp_path.iterdir() if "amdgcn" in p.name and "gfx950" in p.name]
    assert objs, "no gfx950 code object in the library"
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(objs[0])], check=True, capture_output=True, text=True)
    return [l.split("//")[0].strip() for l in out.stdout.splitlines()]


def test_m0_only_in_copy_groups(tmp_path):
    lines = [l for l in _disassembly(tmp_path) if l and not l.endswith(":")]
    copies = 0
    m0_set = False
    for i, l in enumerate(lines):
        op = l.split()[0] if l.split() else ""
        if re.search(r"\bm0\b", l):
            assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", l), f"unexpected M0 access: {l}"
            assert lines[i + 1] == "s_nop 0", f"M0 write not followed by s_nop 0: {lines[i + 1]}"
            assert lines[i + 2].startswith("buffer_load_dwordx4") and lines[i + 2].endswith(" lds"), lines[i + 2]
            m0_set = True
        elif op.startswith("buffer_load") and l.endswith(" lds"):
            assert m0_set, f"LDS copy without its M0 write: {l}"
            copies += 1
        elif op == "s_nop" and m0_set:
            pass
        else:
            m0_set = False
    assert copies > 0

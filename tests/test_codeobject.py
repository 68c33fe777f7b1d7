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

pytestmark = pytest.mark.spawns

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


def _disassembly(tmp_path):
    lib = tg.library_path()
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not installed")
    local = tmp_path / "lib.so"
    shutil.copy(lib, local)
    # --offloading writes the bundled code objects next to the input
    subprocess.run([OBJDUMP, "--offloading", str(local)], check=True, capture_output=True, cwd=tmp_path)
    objs = sorted(p for p in tmp_path.iterdir() if "amdgcn" in p.name and "gfx950" in p.name)
    assert objs, "no gfx950 code object in the library"
    lines = []
    for obj in objs:     # one code object per translation unit with device code
        out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(obj)], check=True, capture_output=True, text=True)
        lines += [l.split("//")[0].strip() for l in out.stdout.splitlines()]
    return lines


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


# An MFMA written as inline assembly is invisible to the compiler's hazard
# handling: a VALU or memory instruction that reads its accumulator must come
# at least 19 wait states after it (the XDL write-to-read distance), which the
# kernels provide by construction (settle() and reading the accumulators in
# place).  This scans for any instruction other than an MFMA that names an
# AGPR written by a 16x16x32 MFMA fewer than 19 wait states earlier (an
# s_nop N counts N + 1, any other instruction 1), along the text of each
# function.  The fp32 ring tiles' 16x16x4 MFMAs are inline assembly too and
# are held to the same distance.
_AREG = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")
_XDL_WAIT = 19


def _agprs(operands):
    regs = set()
    for m in _AREG.finditer(operands):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


def accumulator_hazards(lines):
    """(instruction, wait states) pairs that read an MFMA result too early."""
    bad = []
    pending = []                      # [registers written, wait states since]
    for l in lines:
        if not l or l.endswith(":"):
            if l.endswith(">:"):      # a new function
                pending = []
            continue
        parts = l.split(None, 1)
        op, rest = parts[0], parts[1] if len(parts) > 1 else ""
        if op.startswith(("v_mfma_f32_16x16x32", "v_mfma_f32_16x16x4")):
            dst = rest.split(",")[0]
            for p in pending:
                p[1] += 1
            pending.append([_agprs(dst), 0])
            continue
        used = _agprs(rest)
        for regs, waited in pending:
            if used & regs and waited < _XDL_WAIT:
                bad.append((l, waited))
        step = int(rest) + 1 if op == "s_nop" else 1
        for p in pending:
            p[1] += step
        pending = [p for p in pending if p[1] < _XDL_WAIT]
    return bad


def test_accumulator_reads_wait_for_mfma(tmp_path):
    lines = _disassembly(tmp_path)
    assert any(l.startswith("v_mfma_f32_16x16x32") for l in lines)
    bad = accumulator_hazards(lines)
    assert not bad, f"{len(bad)} early reads of MFMA results, e.g. {bad[:3]}"


def test_accumulator_hazard_scan_finds_an_early_read():
    # the pattern the compiler once produced: a copy right behind the MFMA
    early = ["v_mfma_f32_16x16x32_bf16 a[252:255], v[8:11], v[72:75], a[252:255]", "s_nop 0",
             "v_accvgpr_read_b32 v60, a252"]
    assert accumulator_hazards(early) == [("v_accvgpr_read_b32 v60, a252", 1)]
    settled = early[:1] + ["s_nop 7"] * 4 + early[2:]
    assert accumulator_hazards(settled) == []
    other = early[:2] + ["v_accvgpr_read_b32 v60, a12"]           # a different accumulator
    assert accumulator_hazards(other) == []


# ---- register, scratch and LDS use of the built kernels -------------------------
# The kernel descriptors' metadata (llvm-readelf --notes): .vgpr_count is the
# whole register allocation of a wave (VGPRs and AGPRs), .private_segment_fixed_size
# its scratch per lane, .group_segment_fixed_size its LDS per workgroup.
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
_RING = re.compile(r"gemm_ring_kernelINS_7RingCfgILi(\d)ELi(\d+)ELi(\d+)ELi(\d)ELi(\d)ELi(\d+)EEELi(\d)ELi(\d)ELi(\d)ELb(\d)E")
_F32 = re.compile(r"gemm_kernelINS_7TileCfgILi0ELi64ELi64ELi2ELi2EEELi(\d)ELi(\d)ELb(\d)E")


def _kernels(tmp_path):
    lib = tg.library_path()
    if not os.path.exists(OBJDUMP) or not os.path.exists(READELF):
        pytest.skip("llvm tools not installed")
    local = tmp_path / "lib.so"
    shutil.copy(lib, local)
    subprocess.run([OBJDUMP, "--offloading", str(local)], check=True, capture_output=True, cwd=tmp_path)
    objs = sorted(p for p in tmp_path.iterdir() if "amdgcn" in p.name and "gfx950" in p.name)
    notes = "".join(subprocess.run([READELF, "--notes", str(o)], check=True, capture_output=True, text=True).stdout
                    for o in objs)
    out, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+(?:- )?\.(name|vgpr_count|agpr_count|group_segment_fixed_size|"
                     r"private_segment_fixed_size|max_flat_workgroup_size):\s+(\S+)", line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if line.lstrip().startswith("- "):
            cur = {}
        if cur is None:
            continue
        cur[key] = val
        if key == "name":
            out[val] = cur
    return {n: {k: (int(v) if k != "name" else v) for k, v in d.items()} for n, d in out.items()}


def _opt_in(name):
    """Kernels only an explicit option reaches: persistent workgroups and the pad_stride ablation."""
    if "persistent" in name:
        return True
    m = _RING.search(name)
    return bool(m) and int(m.group(8)) == 2


def test_no_scratch_outside_opt_in_variants(tmp_path):
    ks = _kernels(tmp_path)
    assert len(ks) > 40
    spills = {n: d["private_segment_fixed_size"] for n, d in ks.items() if d["private_segment_fixed_size"] > 0}
    assert all(_opt_in(n) for n in spills), {n: v for n, v in spills.items() if not _opt_in(n)}


CFG_OF = {(256, 256): tg.TG_CFG_256x256, (128, 128): tg.TG_CFG_128x128, (64, 64): tg.TG_CFG_64x64,
          (288, 160): tg.TG_CFG_288x160}


def test_per_cu_table_matches_code_object(tmp_path):
    """The plan's workgroups per CU equal what each built kernel's registers and LDS allow:
    min(4 SIMDs x floor(512 / registers per wave) / waves per workgroup, floor(160 KiB / LDS))."""
    ks = _kernels(tmp_path)
    checked = 0
    for name, d in ks.items():
        m = _RING.search(name)
        f = _F32.search(name)
        if m and "persistent" not in name:
            bm, bn, wm, wn, stages, swz = (int(m.group(i)) for i in (2, 3, 4, 5, 7, 8))
            if (bm, bn) not in CFG_OF or swz == 2:
                continue
            cfg, waves, depth = CFG_OF[(bm, bn)], wm * wn, stages
            dt = {"0": "f32", "1": "bf16", "2": "f16"}[m.group(1)]
        elif f:
            cfg, waves, depth, dt, swz = tg.TG_CFG_F32_64x64, 4, int(f.group(1)), "f32", int(f.group(2))
        else:
            continue
        by_regs = 4 * (512 // d["vgpr_count"]) // waves
        by_lds = (160 * 1024) // max(d["group_segment_fixed_size"], 1)
        plan = tg.tile_gemm_plan(1, 1024, 1024, 1024, dt, config=cfg, pipeline_depth=depth, swizzle=swz)
        assert plan["per_cu"] == min(by_regs, by_lds), (name, d, plan["per_cu"])
        checked += 1
    assert checked >= 20

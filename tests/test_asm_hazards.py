"""The copies into LDS are written in inline asm (global_load_lds_dwordx4 with a scalar base),
so the compiler does not insert the wait states that the hardware needs before them.  On
this chip a vector instruction that writes a scalar register (v_readfirstlane, v_readlane,
v_cmp ...) must be followed by 5 wait states before a vector memory instruction reads that
register; a copy issued sooner can use the stale base and fault.  This test compiles the
kernels that issue such copies to gfx950 assembly and checks every copy: no vector write of
its base registers within the 5 wait states before it.  CPU only (needs hipcc)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_dit_block_head_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


def sgprs(tok):
    out = set()
    for a, b in re.findall(r"s\[(\d+):(\d+)\]", tok):
        out |= set(range(int(a), int(b) + 1))
    out |= {int(a) for a in re.findall(r"\bs(\d+)\b", tok)}
    return out


def hazards(asm_lines):
    """(copies checked, list of hazards) for the copies in an assembly listing."""
    lines = [l.strip() for l in asm_lines]
    found, n = [], 0
    for i, l in enumerate(lines):
        m = re.match(r"global_load_lds_dwordx4\s+v\d+,\s+(s\[\d+:\d+\])", l)
        if not m:
            continue
        n += 1
        base, ws, j = sgprs(m.group(1)), 0, i - 1
        while j >= 0 and ws < 5:
            t = lines[j]
            j -= 1
            if not t or t.startswith(";") or t.startswith("."):
                continue
            op = t.split()[0]
            if op == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            if op.startswith("v_") and sgprs(t[len(op):].split(",")[0]) & base:
                found.append((i + 1, t, l))
            ws += 1
    return n, found


def test_checker_sees_a_planted_hazard():
    ok = ["v_mov_b32 v1, 0", "s_nop 4", "global_load_lds_dwordx4 v3, s[6:7]"]
    bad = ["v_readfirstlane_b32 s7, v1", "s_nop 0", "global_load_lds_dwordx4 v3, s[6:7]"]
    salu = ["v_readfirstlane_b32 s8, v1", "s_mov_b32 s7, s8", "global_load_lds_dwordx4 v3, s[6:7]"]
    assert hazards(ok) == (1, [])
    assert len(hazards(bad)[1]) == 1
    assert hazards(salu) == (1, [])


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
@pytest.mark.parametrize("src", ["attn.hip", "tilemap.hip"])
def test_no_valu_write_of_a_copy_base(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-S", "--offload-device-only", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    n, found = hazards(open(out).read().split("\n"))
    assert n > 0
    assert not found, found[:5]

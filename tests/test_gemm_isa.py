"""Checks on the GEMM kernels' gfx950 assembly (CPU only; hipcc cross-compiles).

The tile kernels issue their global-to-LDS copies as inline assembly that sets
M0 and issues global_load_lds in one statement.  That is sound only while no
other instruction of those kernels reads M0 (relative register addressing,
messages, LDS-direct reads and the like): the compiler may not keep a value of
its own in M0 across the statement.  The benchmarked kernels must also not
spill to scratch memory.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "blockwise_fp8_gemm_amd", "csrc", "gemm.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                            "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", out, SRC],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read().splitlines()


def test_m0_only_feeds_lds_copies(asm):
    writes = 0
    for i, line in enumerate(asm):
        code = line.split(";")[0]
        if not re.search(r"\bm0\b", code):
            continue
        assert re.match(r"\s*s_mov_b32 m0, s\d+\s*$", code), ("M0 used outside the LDS copies", i, line)
        nxt = asm[i + 1].split(";")[0]
        assert "global_load_lds_dword" in nxt, ("M0 write not followed by its copy", i, nxt)
        writes += 1
    assert writes > 0
    banned = re.compile(r"movrel|set_gpr_idx|s_sendmsg|ds_gws|ds_append|ds_consume|v_interp|lds_direct|ds_ordered")
    assert not any(banned.search(l.split(";")[0]) for l in asm)


def test_step_kernels_do_not_spill(asm):
    name = None
    spills = {}
    for line in asm:
        m = re.match(r"\s*\.amdhsa_kernel (\S+)", line)
        if m:
            name = m.group(1)
        m = re.match(r"\s*\.amdhsa_private_segment_fixed_size (\d+)", line)
        if m and name:
            spills[name] = int(m.group(1))
    # the 256x256 FP32-exact tiles (FastCfg<2,4,8,4,2>, datapath 0) of the grouped launcher and of
    # single calls, and the native and MX 256x256 tiles: none may use scratch memory
    hot = [n for n in spills if "FastCfgILi2ELi4ELi8ELi4ELi2E" in n]
    assert len(hot) >= 8, hot
    assert all(spills[n] == 0 for n in hot), {n: spills[n] for n in hot if spills[n]}

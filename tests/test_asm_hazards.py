"""Wait-state checks on the library's gfx950 assembly (built here from source, host only).

The kernels issue their direct global->LDS loads from inline assembly, whose operands the
compiler's hazard recognizer does not inspect.  Two hardware rules then fall to the source:
  * a vector-memory instruction that reads an SGPR (its scalar base address) needs five wait
    states after a vector instruction (e.g. v_readfirstlane) writes that SGPR;
  * a direct-to-LDS load needs one wait state after the write of M0 that addresses it.
This test compiles fd_kernels.hip to device assembly with the library's flags and scans every
kernel for both patterns.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from streaming_kv_cache_view_amd import build

VMEM = re.compile(r"(global_load_lds_\w+|global_load_\w+|global_store_\w+|buffer_\w+)\s+(.*)")


def device_asm(tmp_path) -> str:
    hipcc = build.hipcc()
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "fd_kernels.s"
    cmd = [hipcc, "-O3", "-std=c++17", f"--offload-arch={build.ARCH}", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans", "-Wno-unused-command-line-argument",
           "-I", os.path.join(build.ROOT, "include"), "-I", build.CSRC,
           os.path.join(build.CSRC, "fd_kernels.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def kernels(asm: str):
    for name in re.findall(r"^\s*\.type\s+(_Z\S+),@function", asm, re.M):
        a = asm.index(name + ":")
        b = asm.index(".Lfunc_end", a)
        body = [x.strip() for x in asm[a:b].split("\n")]
        yield name, [x for x in body if x and not x.startswith((".", ";")) and not x.endswith(":")]


def wait_states(ins: str) -> int:
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


def test_sgpr_base_and_m0_wait_states(tmp_path):
    asm = device_asm(tmp_path)
    bad_sgpr, bad_m0, n_lds_dma = [], [], 0
    for name, body in kernels(asm):
        for i, ins in enumerate(body):
            m = VMEM.match(ins)
            if not m:
                continue
            sm = re.search(r"s\[(\d+):(\d+)\]", m.group(2))
            if sm:   # SGPR base: no vector write of it within 5 wait states
                regs = {f"s{k}" for k in range(int(sm.group(1)), int(sm.group(2)) + 1)}
                ws = 0
                for j in range(i - 1, max(-1, i - 8), -1):
                    prev = body[j]
                    if prev.startswith("v_") and prev.split()[1].rstrip(",") in regs:
                        bad_sgpr.append((name[:60], prev, ins))
                    ws += wait_states(prev)
                    if ws >= 5:
                        break
            if ins.startswith("global_load_lds"):
                n_lds_dma += 1
                if i > 0 and re.match(r"s_\w+\s+m0,", body[i - 1]):
                    bad_m0.append((name[:60], body[i - 1], ins))
    assert n_lds_dma > 0
    assert not bad_sgpr, bad_sgpr[:5]
    assert not bad_m0, bad_m0[:5]

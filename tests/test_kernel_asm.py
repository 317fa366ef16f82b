"""Static checks on the compiled gfx950 kernels (CPU only: hipcc
cross-compiles to assembly here).

The direct HBM -> LDS tile loads are issued from inline assembly that sets
M0 (the LDS address of the load) without saving it: that is only sound while
the compiler emits no M0 use of its own in these kernels.  This test compiles
the kernels that issue such loads and checks that every M0 reference sits
inside an inline-assembly block.
"""
import os
import re
import shutil
import subprocess

import pytest

from invariant_attention_flash_amd import build as ia_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_attention_flash_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


_ASM = {}


def _compile_asm(src, tmp_path):
    """gfx950 assembly of one source (compiled once per test session)."""
    if src in _ASM:
        return _ASM[src]
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
           "-fno-fast-math", "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    _ASM[src] = open(out).read()
    return _ASM[src]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", ["prefill.hip", "prefill_ws.hip", "decode.hip", "backward.hip"])
def test_m0_only_in_direct_loads(name, tmp_path):
    assert name in ia_build.SOURCES
    text = _compile_asm(os.path.join(CSRC, name), tmp_path)
    inside = False
    loads = 0
    for line in text.splitlines():
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            inside = True
            continue
        if t.startswith(";;#ASMEND"):
            inside = False
            continue
        if t.startswith(";") or t.startswith("."):
            continue
        code = t.split(";")[0]
        if re.search(r"\bm0\b", code):
            assert inside, f"compiler-emitted M0 use in {name}: {t}"
        if inside and "buffer_load_dwordx4" in code and code.rstrip().endswith("lds"):
            loads += 1
    assert loads > 0, "no direct loads found"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("name", [s for s in ia_build.SOURCES if s != "api.hip"])
def test_kernels_use_no_scratch(name, tmp_path):
    """Every kernel fits its registers: no spills to scratch memory (the
    two-kind kernels rely on each kind's registers fitting two waves per
    SIMD)."""
    text = _compile_asm(os.path.join(CSRC, name), tmp_path)
    kernels = re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", text, re.M)
    sizes = re.findall(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", text, re.M)
    assert kernels and len(kernels) == len(sizes), name
    spilled = [k for k, s in zip(kernels, sizes) if int(s) != 0]
    assert not spilled, f"kernels with scratch in {name}: {spilled}"

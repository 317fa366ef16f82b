"""Build libinvattn.so (HIP, gfx950) in-tree with hipcc.

Flags are part of the numerical contract: no fast-math, no floating-point
contraction (every multiply and add rounds as written), packed-fp32 VALU
instructions disabled, IEEE-rounded fp32 division.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libinvattn.so")
SOURCES = ["api.hip", "prefill.hip", "prefill_ws.hip", "decode.hip", "backward.hip", "prologue.hip"]
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-fast-math", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    """Run a compiler command; drop the host pass's note that it does not know
    the device-only target feature, show everything else."""
    r = subprocess.run(cmd, capture_output=True, text=True)
    for stream in (r.stdout, r.stderr):
        for line in stream.splitlines():
            if "packed-fp32-ops' is not a recognized feature" not in line:
                print(line, file=sys.stderr)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source (in parallel) and link the shared library
    (always rebuilds)."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    flags = HIP_FLAGS + list(extra_flags or [])
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmds.append([hipcc()] + flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                         "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for cmd in cmds if verbose else ():
        print(" ".join(cmd), flush=True)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as pool:
        for f in [pool.submit(_run, c) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)

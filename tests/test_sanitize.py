"""Sanitizer lane for the host code (CPU only): the fp64 oracle and the C-ABI
library's host side (argument checks, error text, provenance, workspace
arithmetic) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven by tests/sanitize_driver.c.  GPU code is built without sanitizers
(the host pass of hipcc takes them through -Xarch_host); nothing here
launches GPU work."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests")
DRIVER = os.path.join(HERE, "sanitize_driver.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, errors="replace", **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-std=c11", "-fopenmp", "-DORACLE_DRIVER"] + SAN +
         [DRIVER, os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"))
    assert "oracle driver ok" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="hipcc / clang not available")
def test_library_host_code_under_asan_ubsan(tmp_path):
    from invariant_attention_flash_amd import build as B
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(ROOT, "_build", src.replace(".hip", ".o"))
        if src == "api.hip":
            obj = str(tmp_path / "api_san.o")
            flags = [f for f in B.HIP_FLAGS]
            for f in SAN:
                flags += ["-Xarch_host", f]
            _run([HIPCC] + flags + ["-I", os.path.join(ROOT, "include"), "-I", B.CSRC, "-c",
                                    os.path.join(B.CSRC, src), "-o", obj])
        assert os.path.exists(obj), f"{obj} missing: build the library first"
        objs.append(obj)
    lib = str(tmp_path / "libinvattn_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs +
         ["-Xarch_host", "-fsanitize=address,undefined"])
    # The driver links with the same compiler (and so the same sanitizer
    # runtime) as the library's host code.
    exe = str(tmp_path / "abi_san")
    _run([CLANG, "-std=c11", "-DABI_DRIVER", "-I", os.path.join(ROOT, "include")] + SAN +
         [DRIVER, "-o", exe, lib, f"-Wl,-rpath,{tmp_path}", "-lm"])
    r = _run([exe], env=ENV)
    assert "abi driver ok" in r.stdout

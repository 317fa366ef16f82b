"""fp64 CPU oracle for masked softmax attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and never calls
it.  The arithmetic lives in ``oracle.c``: the plain definition
``softmax(scale * Q K^T) V`` per query row over its allowed key set, in fp64,
with no tiling or online softmax.  Mask semantics follow the
"RFC: Gemma-4-31B-it train/rollout consistency" page (sections 1 and 3:
sliding and global layers, bidirectional vision-token spans) and the paged
decode read of the "Vime ROCm Attention operator ablation" page
("Prerequisites").  Readings taken where the pages are silent are listed in
``oracle.c``.

Inputs are numpy arrays: uint16 (bf16 bit patterns, widened exactly),
float32 or float64.  Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16, F32, F64 = 0, 1, 2
NO_WINDOW = -1

_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB, werror: bool = True) -> str:
    """Compile the oracle library with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra"]
        cmd += ["-Werror"] if werror else ["-w"]
        cmd += [src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def open_library(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, vp,
                                   vp, i32, i32, i32, i32, i32, dbl, vp, i32,
                                   vp, i64, i32]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i32,
                                  vp, i32, i32, i32, i32, i32, i32, dbl, vp, vp, i32]
    lib.oracle_prefill_backward.restype = ctypes.c_int
    lib.oracle_prefill_backward.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp,
                                            ctypes.c_int, vp, vp, vp, vp, i32, i32, i32, i32,
                                            i32, dbl, vp, i32, i32]
    lib.oracle_prefill_backward_units.restype = ctypes.c_int
    lib.oracle_prefill_backward_units.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp,
                                                  ctypes.c_int, vp, vp, vp, vp, i32, i32, i32,
                                                  i32, i32, dbl, vp, i32, vp, i64, vp, i64, i32]
    lib.oracle_qk_prologue.restype = ctypes.c_int
    lib.oracle_qk_prologue.argtypes = [vp, ctypes.c_int, i64, i32, i32, vp, vp, ctypes.c_int,
                                       dbl, dbl, i32, i32, dbl, vp, i32]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = [i32]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = open_library(_LIB)
    return _lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle input dtype {a.dtype} not supported")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads(threads: int = 0) -> int:
    """Threads an oracle call runs with (0 = OpenMP default)."""
    return _load().oracle_num_threads(threads)


def prefill(q, k, v, cu_seqlens, window=NO_WINDOW, scale=None, spans=None,
            rows=None, want_lse=False, threads=0, lib=None):
    """Packed varlen prefill.  q [T,Hq,D], k/v [T,Hkv,D]; cu_seqlens [B+1].

    ``spans``: int array [S,2] of packed [start, end) bidirectional ranges.
    ``rows``: optional int array [R,2] of (token, head) pairs; then the output
    is [R, D] (and lse [R]) in list order.  Returns o (and lse if asked).
    ``lib``: a library from ``open_library`` (default: the built oracle).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    T, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    batch = cu.shape[0] - 1
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    sp = None
    ns = 0
    if spans is not None and len(spans):
        sp = np.ascontiguousarray(spans, dtype=np.int32).reshape(-1, 2)
        ns = sp.shape[0]
    rw = None
    nr = 0
    if rows is not None:
        rw = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
        nr = rw.shape[0]
        o = np.zeros((nr, d), np.float64)
        lse = np.zeros((nr,), np.float64) if want_lse else None
    else:
        o = np.zeros((T, hq, d), np.float64)
        lse = np.zeros((T, hq), np.float64) if want_lse else None
    rc = (lib or _load()).oracle_prefill(_ptr(q), _code(q), _ptr(k), _ptr(v), _code(k), _ptr(o),
                                _ptr(lse), _ptr(cu), batch, hq, hkv, d, int(window),
                                float(scale), _ptr(sp), ns, _ptr(rw), nr, int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return (o, lse) if want_lse else o


def decode(q, k_cache, v_cache, block_table, seq_lens, window=NO_WINDOW, scale=None,
           want_lse=False, threads=0, lib=None):
    """Paged decode.  q [B,Hq,D]; caches [NB, BS, Hkv, D]; block_table [B, MB]."""
    q = np.ascontiguousarray(q)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    if kc.dtype != vc.dtype:
        raise TypeError("k and v caches must share a dtype")
    batch, hq, d = q.shape
    _, bs, hkv, _ = kc.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((batch, hq, d), np.float64)
    lse = np.zeros((batch, hq), np.float64) if want_lse else None
    rc = (lib or _load()).oracle_decode(_ptr(q), _code(q), _ptr(kc), _ptr(vc), _code(kc), _ptr(bt),
                               bt.shape[1], _ptr(sl), batch, hq, hkv, d, bs, int(window),
                               float(scale), _ptr(o), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return (o, lse) if want_lse else o


def prefill_backward(q, k, v, dout, cu_seqlens, window=NO_WINDOW, scale=None, spans=None,
                     threads=0, lib=None, dq_units=None, kv_units=None):
    """Gradients (dq, dk, dv) of prefill attention for the upstream gradient
    ``dout`` = dL/dO.  q/dout [T,Hq,D], k/v [T,Hkv,D]; outputs float64 in the
    same shapes.  Same mask, spans and scale conventions as ``prefill``.

    ``dq_units``: optional (token, query head) pairs; dq is then [n, D], one
    row per pair.  ``kv_units``: optional (token, KV head) pairs; dk and dv
    are then [n, D].  Only the softmax statistics those units read are
    formed, so a sample of a long sequence is cheap."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dout = np.ascontiguousarray(dout)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    T, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    sp = None
    ns = 0
    if spans is not None and len(spans):
        sp = np.ascontiguousarray(spans, dtype=np.int32).reshape(-1, 2)
        ns = sp.shape[0]

    def flat(units, heads):
        if units is None:
            return None, 0
        u = np.asarray(units, dtype=np.int64).reshape(-1, 2)
        return np.ascontiguousarray(u[:, 0] * heads + u[:, 1]), u.shape[0]

    dqu, n_dq = flat(dq_units, hq)
    kvu, n_kv = flat(kv_units, hkv)
    dq = np.zeros((T, hq, d) if dqu is None else (n_dq, d), np.float64)
    dk = np.zeros((T, hkv, d) if kvu is None else (n_kv, d), np.float64)
    dv = np.zeros_like(dk)
    rc = (lib or _load()).oracle_prefill_backward_units(
        _ptr(q), _code(q), _ptr(k), _ptr(v), _code(k), _ptr(dout), _code(dout), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(cu), cu.shape[0] - 1, hq, hkv, d, int(window), float(scale),
        _ptr(sp), ns, _ptr(dqu), n_dq, _ptr(kvu), n_kv, int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill_backward_units rejected its arguments")
    return dq, dk, dv


def qk_prologue(x, positions, weight=None, eps=1e-6, offset=0.0, rotary_dims=0, freq_dims=None,
                theta=10000.0, threads=0, lib=None):
    """The layer's attention prologue on Q or K: RMSNorm over the head dim
    (skipped when ``weight`` is None), then RoPE on the first ``rotary_dims``
    dims (pairs i, i + R/2; angle pos * theta^(-2i/F), F = ``freq_dims``,
    default R).  x [T, H, D]; positions [T]; weight [D].  Returns fp64
    [T, H, D].  The readings behind this definition are listed in oracle.c.
    """
    x = np.ascontiguousarray(x)
    T, h, d = x.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32).reshape(-1)
    if pos.shape[0] != T:
        raise ValueError("positions must have one entry per row")
    w = None if weight is None else np.ascontiguousarray(weight)
    R = int(rotary_dims)
    F = R if freq_dims is None else int(freq_dims)
    out = np.zeros((T, h, d), np.float64)
    rc = (lib or _load()).oracle_qk_prologue(_ptr(x), _code(x), T, h, d, _ptr(pos), _ptr(w),
                                             F64 if w is None else _code(w), float(eps),
                                             float(offset), R, F, float(theta), _ptr(out),
                                             int(threads))
    if rc != 0:
        raise ValueError("oracle_qk_prologue rejected its arguments")
    return out

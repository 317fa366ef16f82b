"""Batch-invariant attention forward for MI355X (gfx950).

Thin Python binding over the C ABI of ``libinvattn.so`` (declared in
``include/invattn.h``): argument marshalling only.  Every step of the
attention runs in the library's HIP kernels; PyTorch supplies device memory
and the current stream.  There is no fallback path: if the library is not
built, or the GPU is missing, calls raise.

Entry points (same names as the C ABI):
  attn_prefill_varlen  packed variable-length prefill, sliding or global,
                       GQA, optional bidirectional spans
  attn_prefill_varlen_backward
                       its gradients dq, dk, dv in a fixed order
  attn_prefill_paged   chunked prefill: new query tokens against the keys of
                       a paged KV cache (cached prefix plus the chunk)
  attn_decode_paged    one query token per sequence over a paged KV cache
  attn_decode_paged_noalloc
                       the same without a workspace (the library's static
                       scratch), for callers that cannot allocate
  attn_decode_workspace_size
  attn_qk_prologue     the layer's prologue on Q and K in place: RMSNorm over
                       the head dim, then RoPE on the first rotary_dims dims
"""
from __future__ import annotations

import ctypes
import json
import os

__all__ = ["attn_prefill_varlen", "attn_prefill_varlen_backward", "attn_prefill_paged",
           "attn_decode_paged", "attn_decode_paged_noalloc", "attn_decode_workspace_size",
           "attn_qk_prologue",
           "ATTN_NOALLOC_SCRATCH_BYTES",
           "last_provenance", "last_error", "AttnError", "library", "LIB_PATH",
           "ATTN_WINDOW_NONE", "ATTN_DECODE_CHUNK", "ERROR_CODES", "EXPORTS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libinvattn.so")
ATTN_WINDOW_NONE = -1
ATTN_DECODE_CHUNK = 512
ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20
ERROR_CODES = {0: "ATTN_OK", 1: "ATTN_E_NULL", 2: "ATTN_E_SHAPE", 3: "ATTN_E_UNSUPPORTED",
               4: "ATTN_E_ALIGN", 5: "ATTN_E_WORKSPACE", 6: "ATTN_E_HIP", 7: "ATTN_E_VALIDATE"}
EXPORTS = ["attn_prefill_varlen", "attn_prefill_varlen_backward", "attn_prefill_paged",
           "attn_decode_workspace_size", "attn_decode_paged", "attn_decode_paged_noalloc",
           "attn_qk_prologue", "attn_last_error", "attn_last_provenance", "attn_version"]


class AttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_CODES.get(code, code)}: {message}")
        self.code = code
        self.name = ERROR_CODES.get(code, str(code))


_lib = None


def library():
    """Load ``libinvattn.so`` (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        lib.attn_prefill_varlen.restype = ctypes.c_int
        lib.attn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, f32, vp, i32, vp]
        lib.attn_prefill_paged.restype = ctypes.c_int
        lib.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           i32, i32, i32, i32, i32, i32, f32, vp]
        lib.attn_prefill_varlen_backward.restype = ctypes.c_int
        lib.attn_prefill_varlen_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                     vp, i32, i32, i32, i32, i32, i32, f32, vp,
                                                     i32, vp]
        lib.attn_decode_workspace_size.restype = sz
        lib.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32]
        lib.attn_decode_paged.restype = ctypes.c_int
        lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                          i32, i32, i32, f32, vp, sz, vp, vp]
        lib.attn_decode_paged_noalloc.restype = ctypes.c_int
        lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                                  i32, i32, i32, f32, vp, vp]
        lib.attn_qk_prologue.restype = ctypes.c_int
        lib.attn_qk_prologue.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, f32, f32, i32,
                                         i32, ctypes.c_double, vp]
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_provenance.restype = ctypes.c_int
        lib.attn_last_provenance.argtypes = [ctypes.c_char_p, sz]
        lib.attn_version.restype = ctypes.c_char_p
        lib.attn_version.argtypes = []
        _lib = lib
    return _lib


def last_error() -> str:
    return library().attn_last_error().decode()


def last_provenance():
    """Provenance record (dict) of the last successful call on this thread."""
    lib = library()
    n = lib.attn_last_provenance(None, 0)
    if n < 0:
        return None
    buf = ctypes.create_string_buffer(n + 1)
    lib.attn_last_provenance(buf, n + 1)
    return json.loads(buf.value.decode())


def _check(rc: int):
    if rc != 0:
        raise AttnError(rc, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, dtype, dim=None):
    """Type, layout and rank of one tensor argument (the device is checked
    by _on_one_gpu once every shape has been checked)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")


def _shape(t, name, want):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _on_one_gpu(**tensors):
    """Every tensor argument lives on the same GPU (the kernels read and
    write them there)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen, window=ATTN_WINDOW_NONE,
                        softmax_scale=None, spans=None, out=None, lse=None, stream=None):
    """Packed varlen prefill.

    q [T, Hq, D], k/v [T, Hkv, D] bf16 CUDA tensors; cu_seqlens int32 [B+1];
    spans int32 [S, 2] packed [start, end) bidirectional ranges or None;
    out bf16 [T, Hq, D] (allocated if None); lse fp32 [T, Hq] or None.
    Returns out.
    """
    import torch
    _require(q, "q", torch.bfloat16, 3)
    _require(k, "k", torch.bfloat16, 3)
    _require(v, "v", torch.bfloat16, 3)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16, 3)
    _shape(out, "out", q.shape)
    if lse is not None:
        _require(lse, "lse", torch.float32, 2)
        _shape(lse, "lse", (T, hq))
    ns = 0
    if spans is not None:
        _require(spans, "spans", torch.int32, 2)
        if spans.shape[1] != 2:
            raise ValueError(f"spans must be [S, 2], got {tuple(spans.shape)}")
        ns = spans.shape[0]
        if ns == 0:
            spans = None
    _on_one_gpu(q=q, k=k, v=v, cu_seqlens=cu_seqlens, out=out, lse=lse, spans=spans)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    rc = library().attn_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
        cu_seqlens.shape[0] - 1, int(max_seqlen), hq, hkv, d, int(window),
        float(softmax_scale), _ptr(spans), ns, _stream(stream))
    _check(rc)
    return out


def attn_prefill_varlen_backward(q, k, v, out, lse, dout, cu_seqlens, max_seqlen,
                                 window=ATTN_WINDOW_NONE, softmax_scale=None, spans=None,
                                 dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of attn_prefill_varlen.

    q, k, v, cu_seqlens, max_seqlen, window, softmax_scale, spans as for the
    forward; out bf16 [T, Hq, D] and lse fp32 [T, Hq] are the forward's
    outputs; dout bf16 [T, Hq, D] the upstream gradient.  dq fp32 [T, Hq, D],
    dk/dv fp32 [T, Hkv, D] and workspace fp32 [T, Hq] are allocated if None.
    Returns (dq, dk, dv).
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _require(t, n, torch.bfloat16, 3)
    _require(lse, "lse", torch.float32, 2)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != T or k.shape[2] != d:
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must be [T, Hq, D] matching q")
    if tuple(lse.shape) != (T, hq):
        raise ValueError("lse must be [T, Hq]")
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty((T, hq), dtype=torch.float32, device=q.device)
    _require(dq, "dq", torch.float32, 3)
    _require(dk, "dk", torch.float32, 3)
    _require(dv, "dv", torch.float32, 3)
    _require(workspace, "workspace", torch.float32)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("dq must match q and dk, dv must match k")
    if workspace.numel() < T * hq:
        raise ValueError("workspace must hold T * Hq floats")
    ns = 0
    if spans is not None:
        _require(spans, "spans", torch.int32, 2)
        if spans.shape[1] != 2:
            raise ValueError(f"spans must be [S, 2], got {tuple(spans.shape)}")
        ns = spans.shape[0]
        if ns == 0:
            spans = None
    _on_one_gpu(q=q, k=k, v=v, out=out, lse=lse, dout=dout, cu_seqlens=cu_seqlens, dq=dq, dk=dk,
                dv=dv, workspace=workspace, spans=spans)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    rc = library().attn_prefill_varlen_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(workspace), T, _ptr(cu_seqlens), cu_seqlens.shape[0] - 1,
        int(max_seqlen), hq, hkv, d, int(window), float(softmax_scale), _ptr(spans), ns,
        _stream(stream))
    _check(rc)
    return dq, dk, dv


def attn_prefill_paged(q, k_cache, v_cache, block_table, cu_seqlens, q_start, max_query_len,
                       max_context_len, window=ATTN_WINDOW_NONE, softmax_scale=None, out=None,
                       lse=None, stream=None):
    """Chunked prefill over a paged KV cache.

    q [T, Hq, D] bf16 (packed new tokens); k_cache/v_cache [NB, 16, Hkv, D]
    bf16 holding every key of each sequence up to its last new token;
    block_table int32 [B, MB]; cu_seqlens int32 [B+1] (packed new-token
    ranges); q_start int32 [B] (position of each sequence's first new token);
    out bf16 [T, Hq, D] (allocated if None); lse fp32 [T, Hq] or None.
    Returns out.
    """
    import torch
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _require(q_start, "q_start", torch.int32, 1)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("caches must be [NB, BS, Hkv, D] matching q")
    B = cu_seqlens.shape[0] - 1
    if q_start.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("q_start and block_table must have one entry per sequence")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16, 3)
    _shape(out, "out", q.shape)
    if lse is not None:
        _require(lse, "lse", torch.float32, 2)
        _shape(lse, "lse", (T, hq))
    _on_one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                cu_seqlens=cu_seqlens, q_start=q_start, out=out, lse=lse)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    rc = library().attn_prefill_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
        _ptr(q_start), _ptr(block_table), block_table.shape[1], B, int(max_query_len),
        int(max_context_len), nb, bs, hq, hkv, d, int(window), float(softmax_scale),
        _stream(stream))
    _check(rc)
    return out


def attn_decode_workspace_size(batch, max_seq_len, num_q_heads, head_dim) -> int:
    return int(library().attn_decode_workspace_size(batch, max_seq_len, num_q_heads, head_dim))


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len,
                      window=ATTN_WINDOW_NONE, softmax_scale=None, workspace=None, out=None,
                      stream=None):
    """Paged decode.

    q [B, Hq, D] bf16; k_cache/v_cache [NB, 16, Hkv, D] bf16; block_table
    int32 [B, MB]; seq_lens int32 [B] (current token included);
    workspace: uint8/fp32 CUDA tensor of at least attn_decode_workspace_size
    bytes (allocated if None); out bf16 [B, Hq, D].  Returns out.
    """
    import torch
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(seq_lens, "seq_lens", torch.int32, 1)
    B, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("caches must be [NB, BS, Hkv, D] matching q")
    _shape(seq_lens, "seq_lens", (B,))
    if block_table.shape[0] != B:
        raise ValueError(f"block_table must have {B} rows (one per sequence), got "
                         f"{block_table.shape[0]}")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.bfloat16, 3)
    _shape(out, "out", q.shape)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _on_one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                seq_lens=seq_lens, out=out, workspace=workspace)
    need = attn_decode_workspace_size(B, int(max_seq_len), hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    rc = library().attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), B, int(max_seq_len), nb, bs, hq, hkv, d, int(window),
        float(softmax_scale), _ptr(workspace), wbytes, _ptr(out), _stream(stream))
    _check(rc)
    return out


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out,
                              window=ATTN_WINDOW_NONE, softmax_scale=None, stream=None):
    """Paged decode without a workspace: the library keeps the chunk records
    in its static per-GPU scratch (at most ATTN_NOALLOC_SCRATCH_BYTES), so the
    call allocates nothing; ``out`` bf16 [B, Hq, D] is required.  Calls that
    overlap on one GPU share that scratch and must be serialised.  Returns
    out."""
    import torch
    _require(q, "q", torch.bfloat16, 3)
    _require(k_cache, "k_cache", torch.bfloat16, 4)
    _require(v_cache, "v_cache", torch.bfloat16, 4)
    _require(block_table, "block_table", torch.int32, 2)
    _require(seq_lens, "seq_lens", torch.int32, 1)
    _require(out, "out", torch.bfloat16, 3)
    B, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("caches must be [NB, BS, Hkv, D] matching q")
    _shape(seq_lens, "seq_lens", (B,))
    if block_table.shape[0] != B:
        raise ValueError(f"block_table must have {B} rows (one per sequence), got "
                         f"{block_table.shape[0]}")
    _shape(out, "out", q.shape)
    _on_one_gpu(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                seq_lens=seq_lens, out=out)
    if softmax_scale is None:
        softmax_scale = d ** -0.5
    rc = library().attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), B, int(max_seq_len), nb, bs, hq, hkv, d, int(window),
        float(softmax_scale), _ptr(out), _stream(stream))
    _check(rc)
    return out


def attn_qk_prologue(q, k, positions, q_weight=None, k_weight=None, eps=1e-6, weight_offset=0.0,
                     rotary_dims=0, freq_dims=None, rope_theta=10000.0, stream=None):
    """The layer's attention prologue, in place: RMSNorm of every head vector
    of q (and k) over the head dim, then RoPE on its first ``rotary_dims``
    dims (pairs i, i + R/2; angle pos * rope_theta^(-2i/F), F = ``freq_dims``,
    default R).

    q bf16 [T, Hq, D]; k bf16 [T, Hkv, D] or None; positions int32 [T];
    q_weight / k_weight fp32 [D] or None (no norm on that tensor).  Returns
    (q, k).
    """
    import torch
    _require(q, "q", torch.bfloat16, 3)
    T, hq, d = q.shape
    hkv = 0
    if k is not None:
        _require(k, "k", torch.bfloat16, 3)
        if k.shape[0] != T or k.shape[2] != d:
            raise ValueError(f"k must be [T={T}, Hkv, D={d}], got {tuple(k.shape)}")
        hkv = k.shape[1]
    _require(positions, "positions", torch.int32, 1)
    _shape(positions, "positions", (T,))
    for name, w in (("q_weight", q_weight), ("k_weight", k_weight)):
        if w is not None:
            _require(w, name, torch.float32, 1)
            _shape(w, name, (d,))
    _on_one_gpu(q=q, k=k, positions=positions, q_weight=q_weight, k_weight=k_weight)
    R = int(rotary_dims)
    F = R if freq_dims is None else int(freq_dims)
    _check(library().attn_qk_prologue(_ptr(q), _ptr(k), _ptr(positions), T, hq, hkv, d,
                                      _ptr(q_weight), _ptr(k_weight), float(eps),
                                      float(weight_offset), R, F, float(rope_theta),
                                      _stream(stream)))
    return q, k

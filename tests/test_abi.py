"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects unsupported geometry before touching the GPU
(fail closed, "RFC: Gemma-4-31B-it train/rollout consistency", section 4,
item 7).  No GPU work is launched here."""
import ctypes
import os
import re

import pytest

import invariant_attention_flash_amd as ia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "invattn.h")

E = {v: k for k, v in ia.ERROR_CODES.items()}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_library_builds_and_loads():
    assert os.path.exists(ia.LIB_PATH)
    assert ia.library().attn_version().decode().startswith("invattn")


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(ia.EXPORTS), names
    lib = ctypes.CDLL(ia.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_size_formula():
    f = ia.attn_decode_workspace_size
    assert f(64, 32768, 32, 512) == 64 * 32 * 64 * (512 + 4) * 4
    assert f(1, 1, 32, 512) == 32 * 1 * 516 * 4
    assert f(1, 513, 8, 256) == 8 * 2 * 260 * 4
    assert f(0, 10, 8, 64) == 0
    assert f(3, 0, 8, 64) == 0


def call_prefill(**kw):
    a = dict(q=1 << 20, k=1 << 20, v=1 << 20, o=1 << 20, lse=None, cu=1 << 20, batch=2,
             max_seqlen=16, hq=4, hkv=2, d=64, window=-1, scale=0.125, spans=None, ns=0)
    a.update(kw)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = ia.library().attn_prefill_varlen(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["o"]), ptr(a["lse"]), ptr(a["cu"]),
        a["batch"], a["max_seqlen"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"],
        ptr(a["spans"]), a["ns"], None)
    return rc, ia.last_error()


# Each case fails in argument checking, before any HIP call.
PREFILL_ERRORS = [
    (dict(q=None), "ATTN_E_NULL", "q is NULL"),
    (dict(k=None), "ATTN_E_NULL", "k is NULL"),
    (dict(v=None), "ATTN_E_NULL", "v is NULL"),
    (dict(o=None), "ATTN_E_NULL", "o is NULL"),
    (dict(cu=None), "ATTN_E_NULL", "cu_seqlens"),
    (dict(ns=2, spans=None), "ATTN_E_NULL", "spans_opt"),
    (dict(batch=-1), "ATTN_E_SHAPE", "batch"),
    (dict(max_seqlen=-5), "ATTN_E_SHAPE", "max_seqlen"),
    (dict(hq=6, hkv=4), "ATTN_E_SHAPE", "multiple"),
    (dict(hq=0), "ATTN_E_SHAPE", "positive"),
    (dict(hq=32, hkv=2), "ATTN_E_UNSUPPORTED", "group"),
    (dict(hq=12, hkv=4), "ATTN_E_UNSUPPORTED", "group"),
    (dict(d=128), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(d=96), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(window=0), "ATTN_E_UNSUPPORTED", "window"),
    (dict(window=-7), "ATTN_E_UNSUPPORTED", "window"),
    (dict(scale=0.0), "ATTN_E_UNSUPPORTED", "softmax_scale"),
    (dict(scale=float("nan")), "ATTN_E_UNSUPPORTED", "softmax_scale"),
    (dict(scale=float("inf")), "ATTN_E_UNSUPPORTED", "softmax_scale"),
    (dict(q=(1 << 20) + 8), "ATTN_E_ALIGN", "q is not 16-byte"),
    (dict(o=(1 << 20) + 2), "ATTN_E_ALIGN", "o is not 16-byte"),
    (dict(cu=(1 << 20) + 2), "ATTN_E_ALIGN", "cu_seqlens"),
    (dict(max_seqlen=1 << 22, hq=32, hkv=16, d=256), "ATTN_E_UNSUPPORTED", "2 GiB"),
]


@pytest.mark.parametrize("kw,code,text", PREFILL_ERRORS, ids=[c[2] + str(i) for i, c in enumerate(PREFILL_ERRORS)])
def test_prefill_rejects(kw, code, text):
    rc, msg = call_prefill(**kw)
    assert ia.ERROR_CODES[rc] == code, (rc, msg)
    assert text in msg


def call_decode(**kw):
    a = dict(q=1 << 20, kc=1 << 20, vc=1 << 20, bt=1 << 20, mb=4, sl=1 << 20, batch=2, msl=64,
             nb=100, bs=16, hq=32, hkv=4, d=512, window=-1, scale=0.04, ws=1 << 20,
             wsb=1 << 30, o=1 << 20)
    a.update(kw)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = ia.library().attn_decode_paged(
        ptr(a["q"]), ptr(a["kc"]), ptr(a["vc"]), ptr(a["bt"]), a["mb"], ptr(a["sl"]), a["batch"],
        a["msl"], a["nb"], a["bs"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"],
        ptr(a["ws"]), a["wsb"], ptr(a["o"]), None)
    return rc, ia.last_error()


DECODE_ERRORS = [
    (dict(q=None), "ATTN_E_NULL", "q is NULL"),
    (dict(kc=None), "ATTN_E_NULL", "k_cache"),
    (dict(vc=None), "ATTN_E_NULL", "v_cache"),
    (dict(bt=None), "ATTN_E_NULL", "block_table"),
    (dict(sl=None), "ATTN_E_NULL", "seq_lens"),
    (dict(ws=None), "ATTN_E_NULL", "workspace"),
    (dict(o=None), "ATTN_E_NULL", "o is NULL"),
    (dict(bs=32), "ATTN_E_UNSUPPORTED", "block_size"),
    (dict(d=128), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(hq=64, hkv=4), "ATTN_E_UNSUPPORTED", "group"),
    (dict(window=0), "ATTN_E_UNSUPPORTED", "window"),
    (dict(msl=0), "ATTN_E_SHAPE", "max_seq_len"),
    (dict(mb=3), "ATTN_E_SHAPE", "max_blocks_per_seq"),
    (dict(nb=0), "ATTN_E_SHAPE", "num_blocks"),
    (dict(wsb=100), "ATTN_E_WORKSPACE", "workspace_bytes"),
    (dict(ws=(1 << 20) + 4), "ATTN_E_ALIGN", "workspace"),
    (dict(kc=(1 << 20) + 2), "ATTN_E_ALIGN", "k_cache"),
]


@pytest.mark.parametrize("kw,code,text", DECODE_ERRORS, ids=[c[2] + str(i) for i, c in enumerate(DECODE_ERRORS)])
def test_decode_rejects(kw, code, text):
    rc, msg = call_decode(**kw)
    assert ia.ERROR_CODES[rc] == code, (rc, msg)
    assert text in msg


def test_error_text_is_per_call():
    rc, msg = call_prefill(d=96)
    assert rc != 0 and "head_dim" in msg
    rc, msg = call_prefill(window=0)
    assert "window" in msg and "head_dim" not in msg


def call_prefill_paged(**kw):
    a = dict(q=1 << 20, kc=1 << 20, vc=1 << 20, o=1 << 20, lse=None, cu=1 << 20, qs=1 << 20,
             bt=1 << 20, mb=8, batch=2, mql=32, mcl=128, nb=100, bs=16, hq=32, hkv=16, d=256,
             window=128, scale=0.0625)
    a.update(kw)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = ia.library().attn_prefill_paged(
        ptr(a["q"]), ptr(a["kc"]), ptr(a["vc"]), ptr(a["o"]), ptr(a["lse"]), ptr(a["cu"]),
        ptr(a["qs"]), ptr(a["bt"]), a["mb"], a["batch"], a["mql"], a["mcl"], a["nb"], a["bs"],
        a["hq"], a["hkv"], a["d"], a["window"], a["scale"], None)
    return rc, ia.last_error()


PAGED_PREFILL_ERRORS = [
    (dict(q=None), "ATTN_E_NULL", "q is NULL"),
    (dict(kc=None), "ATTN_E_NULL", "k_cache"),
    (dict(vc=None), "ATTN_E_NULL", "v_cache"),
    (dict(o=None), "ATTN_E_NULL", "o is NULL"),
    (dict(cu=None), "ATTN_E_NULL", "cu_seqlens"),
    (dict(qs=None), "ATTN_E_NULL", "q_start"),
    (dict(bt=None), "ATTN_E_NULL", "block_table"),
    (dict(batch=-1), "ATTN_E_SHAPE", "batch"),
    (dict(mql=-1), "ATTN_E_SHAPE", "max_query_len"),
    (dict(mcl=16), "ATTN_E_SHAPE", "max_context_len"),
    (dict(mb=7), "ATTN_E_SHAPE", "max_blocks_per_seq"),
    (dict(mb=0), "ATTN_E_SHAPE", "max_blocks_per_seq"),
    (dict(nb=0), "ATTN_E_SHAPE", "num_blocks"),
    (dict(bs=32), "ATTN_E_UNSUPPORTED", "block_size"),
    (dict(d=128), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(hq=64, hkv=4), "ATTN_E_UNSUPPORTED", "group"),
    (dict(window=0), "ATTN_E_UNSUPPORTED", "window"),
    (dict(scale=-1.0), "ATTN_E_UNSUPPORTED", "softmax_scale"),
    (dict(kc=(1 << 20) + 2), "ATTN_E_ALIGN", "k_cache"),
    (dict(qs=(1 << 20) + 2), "ATTN_E_ALIGN", "q_start"),
    (dict(bt=(1 << 20) + 1), "ATTN_E_ALIGN", "block_table"),
]


@pytest.mark.parametrize("kw,code,text", PAGED_PREFILL_ERRORS,
                         ids=[c[2] + str(i) for i, c in enumerate(PAGED_PREFILL_ERRORS)])
def test_prefill_paged_rejects(kw, code, text):
    rc, msg = call_prefill_paged(**kw)
    assert ia.ERROR_CODES[rc] == code, (rc, msg)
    assert text in msg


def test_prefill_paged_empty_input_needs_no_pointers():
    rc, msg = call_prefill_paged(q=None, kc=None, vc=None, o=None, cu=None, qs=None, bt=None,
                                 batch=0)
    assert rc == 0, msg
    rc, msg = call_prefill_paged(q=None, kc=None, vc=None, o=None, cu=None, qs=None, bt=None,
                                 mql=0)
    assert rc == 0, msg


def call_backward(**kw):
    a = dict(q=1 << 20, k=1 << 20, v=1 << 20, o=1 << 20, lse=1 << 20, do=1 << 20, dq=1 << 20,
             dk=1 << 20, dv=1 << 20, ws=1 << 20, tt=32, cu=1 << 20, batch=2, max_seqlen=16,
             hq=4, hkv=2, d=64, window=-1, scale=0.125, spans=None, ns=0)
    a.update(kw)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = ia.library().attn_prefill_varlen_backward(
        ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["o"]), ptr(a["lse"]), ptr(a["do"]),
        ptr(a["dq"]), ptr(a["dk"]), ptr(a["dv"]), ptr(a["ws"]), a["tt"], ptr(a["cu"]),
        a["batch"], a["max_seqlen"], a["hq"], a["hkv"], a["d"], a["window"], a["scale"],
        ptr(a["spans"]), a["ns"], None)
    return rc, ia.last_error()


BACKWARD_ERRORS = [
    (dict(q=None), "ATTN_E_NULL", "q is NULL"),
    (dict(k=None), "ATTN_E_NULL", "k is NULL"),
    (dict(v=None), "ATTN_E_NULL", "v is NULL"),
    (dict(o=None), "ATTN_E_NULL", "o is NULL"),
    (dict(lse=None), "ATTN_E_NULL", "lse is NULL"),
    (dict(do=None), "ATTN_E_NULL", "dout is NULL"),
    (dict(dq=None), "ATTN_E_NULL", "dq is NULL"),
    (dict(dk=None), "ATTN_E_NULL", "dk is NULL"),
    (dict(dv=None), "ATTN_E_NULL", "dv is NULL"),
    (dict(ws=None), "ATTN_E_NULL", "workspace is NULL"),
    (dict(cu=None), "ATTN_E_NULL", "cu_seqlens"),
    (dict(ns=1, spans=None), "ATTN_E_NULL", "spans_opt"),
    (dict(batch=-1), "ATTN_E_SHAPE", "batch"),
    (dict(max_seqlen=-1), "ATTN_E_SHAPE", "max_seqlen"),
    (dict(tt=-1), "ATTN_E_SHAPE", "total_tokens"),
    (dict(ns=-1), "ATTN_E_SHAPE", "num_spans"),
    (dict(hq=6, hkv=4), "ATTN_E_SHAPE", "multiple"),
    (dict(d=128), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(window=0), "ATTN_E_UNSUPPORTED", "window"),
    (dict(scale=float("nan")), "ATTN_E_UNSUPPORTED", "softmax_scale"),
    (dict(batch=70000), "ATTN_E_UNSUPPORTED", "65535"),
    (dict(max_seqlen=1 << 30, hq=32, hkv=16, batch=65535), "ATTN_E_UNSUPPORTED", "2^31"),
    (dict(dk=(1 << 20) + 4), "ATTN_E_ALIGN", "dk is not 16-byte"),
    (dict(ws=(1 << 20) + 4), "ATTN_E_ALIGN", "workspace is not 16-byte"),
    (dict(lse=(1 << 20) + 2), "ATTN_E_ALIGN", "lse is not 4-byte"),
]


@pytest.mark.parametrize("kw,code,text", BACKWARD_ERRORS,
                         ids=[c[2] + str(i) for i, c in enumerate(BACKWARD_ERRORS)])
def test_backward_rejects(kw, code, text):
    rc, msg = call_backward(**kw)
    assert ia.ERROR_CODES[rc] == code, (rc, msg)
    assert text in msg


def test_backward_empty_input_needs_no_pointers():
    none = dict(q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                ws=None, cu=None)
    rc, msg = call_backward(batch=0, **none)
    assert rc == 0, msg
    rc, msg = call_backward(max_seqlen=0, **none)
    assert rc == 0, msg


def test_noalloc_decode_rejects_beyond_scratch_before_any_gpu_call():
    """The allocation-free decode keeps its chunk records in a static scratch
    of ATTN_NOALLOC_SCRATCH_BYTES: a batch needing more is refused on the
    host (ATTN_E_WORKSPACE), before the scratch is looked up on a device."""
    need = ia.attn_decode_workspace_size(64, 32768, 32, 512)
    assert need > ia.ATTN_NOALLOC_SCRATCH_BYTES
    assert ia.attn_decode_workspace_size(1, 1016 * 512, 32, 512) <= ia.ATTN_NOALLOC_SCRATCH_BYTES
    x = ctypes.c_void_p(1 << 20)
    rc = ia.library().attn_decode_paged_noalloc(x, x, x, x, 2048, x, 64, 32768, 100, 16, 32, 4,
                                                512, -1, ctypes.c_float(0.044), x, None)
    assert rc == E["ATTN_E_WORKSPACE"]
    assert "scratch" in ia.last_error()


def call_prologue(**kw):
    a = dict(q=1 << 20, k=1 << 20, pos=1 << 20, T=8, hq=4, hkv=2, d=256, qw=1 << 20, kw=1 << 20,
             eps=1e-6, off=0.0, R=256, F=256, theta=10000.0)
    a.update(kw)
    ptr = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = ia.library().attn_qk_prologue(ptr(a["q"]), ptr(a["k"]), ptr(a["pos"]), a["T"], a["hq"],
                                       a["hkv"], a["d"], ptr(a["qw"]), ptr(a["kw"]), a["eps"],
                                       a["off"], a["R"], a["F"], a["theta"], None)
    return rc, ia.last_error()


PROLOGUE_ERRORS = [
    (dict(q=None), "ATTN_E_NULL", "q is NULL"),
    (dict(pos=None), "ATTN_E_NULL", "positions is NULL"),
    (dict(T=-1), "ATTN_E_SHAPE", "num_tokens"),
    (dict(hq=0), "ATTN_E_SHAPE", "num_q_heads"),
    (dict(hkv=0), "ATTN_E_SHAPE", "num_kv_heads"),
    (dict(d=128), "ATTN_E_UNSUPPORTED", "head_dim"),
    (dict(R=258), "ATTN_E_UNSUPPORTED", "rotary_dims"),
    (dict(R=-2), "ATTN_E_UNSUPPORTED", "rotary_dims"),
    (dict(R=4), "ATTN_E_UNSUPPORTED", "multiple of 8"),
    (dict(d=512, R=8), "ATTN_E_UNSUPPORTED", "multiple of 16"),
    (dict(F=0), "ATTN_E_UNSUPPORTED", "freq_dims"),
    (dict(theta=0.0), "ATTN_E_UNSUPPORTED", "rope_theta"),
    (dict(theta=float("inf")), "ATTN_E_UNSUPPORTED", "rope_theta"),
    (dict(eps=-1.0), "ATTN_E_UNSUPPORTED", "eps"),
    (dict(eps=float("nan")), "ATTN_E_UNSUPPORTED", "eps"),
    (dict(off=float("inf")), "ATTN_E_UNSUPPORTED", "weight_offset"),
    (dict(q=(1 << 20) + 4), "ATTN_E_ALIGN", "q is not 16-byte"),
    (dict(k=(1 << 20) + 8), "ATTN_E_ALIGN", "k is not 16-byte"),
    (dict(pos=(1 << 20) + 2), "ATTN_E_ALIGN", "positions is not 4-byte"),
    (dict(qw=(1 << 20) + 2), "ATTN_E_ALIGN", "q_weight is not 4-byte"),
]


@pytest.mark.parametrize("kw,code,text", PROLOGUE_ERRORS,
                         ids=[c[2] + str(i) for i, c in enumerate(PROLOGUE_ERRORS)])
def test_prologue_rejects(kw, code, text):
    rc, msg = call_prologue(**kw)
    assert ia.ERROR_CODES[rc] == code, (rc, msg)
    assert text in msg


def test_prologue_empty_input_needs_no_pointers():
    rc, msg = call_prologue(T=0, q=None, k=None, pos=None, qw=None, kw=None)
    assert rc == 0, msg
    # no RoPE: the rotary checks do not apply
    rc, msg = call_prologue(T=0, R=0, F=0, theta=0.0)
    assert rc == 0, msg

"""The Python binding checks every tensor argument's dtype, rank and shape
before it calls the library, so a wrongly shaped output, LSE, sequence-length
or block-table tensor is rejected on the host instead of letting a kernel
read or write outside the caller's buffers (fail closed, "RFC:
Gemma-4-31B-it train/rollout consistency", section 4, item 7).  CPU tensors
reach these checks first; no GPU work is launched here."""
import pytest
import torch

import invariant_attention_flash_amd as ia

bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32


def t(shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def prefill_args(**kw):
    a = dict(q=t((10, 4, 64)), k=t((10, 2, 64)), v=t((10, 2, 64)), cu_seqlens=t((3,), i32),
             max_seqlen=8)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,text", [
    (dict(out=t((10, 4, 32))), "out must have shape"),
    (dict(out=t((9, 4, 64))), "out must have shape"),
    (dict(lse=t((10, 2), f32)), "lse must have shape"),
    (dict(lse=t((11, 4), f32)), "lse must have shape"),
    (dict(spans=t((2, 3), i32)), "spans must be"),
    (dict(k=t((10, 2, 32))), "k and v must be"),
    ({}, "must be on a GPU device"),
])
def test_prefill_binding_rejects(kw, text):
    with pytest.raises(ValueError, match=text):
        ia.attn_prefill_varlen(**prefill_args(**kw))


def paged_args(**kw):
    a = dict(q=t((10, 4, 64)), k_cache=t((6, 16, 2, 64)), v_cache=t((6, 16, 2, 64)),
             block_table=t((2, 3), i32), cu_seqlens=t((3,), i32), q_start=t((2,), i32),
             max_query_len=8, max_context_len=40)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,text", [
    (dict(out=t((10, 4, 16))), "out must have shape"),
    (dict(lse=t((10, 3), f32)), "lse must have shape"),
    (dict(q_start=t((3,), i32)), "one entry per sequence"),
    (dict(block_table=t((1, 3), i32)), "one entry per sequence"),
    ({}, "must be on a GPU device"),
])
def test_prefill_paged_binding_rejects(kw, text):
    with pytest.raises(ValueError, match=text):
        ia.attn_prefill_paged(**paged_args(**kw))


def decode_args(**kw):
    a = dict(q=t((3, 8, 64)), k_cache=t((6, 16, 2, 64)), v_cache=t((6, 16, 2, 64)),
             block_table=t((3, 4), i32), seq_lens=t((3,), i32), max_seq_len=64)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,text", [
    (dict(seq_lens=t((2,), i32)), "seq_lens must have shape"),
    (dict(seq_lens=t((4,), i32)), "seq_lens must have shape"),
    (dict(block_table=t((2, 4), i32)), "block_table must have 3 rows"),
    (dict(out=t((3, 8, 32))), "out must have shape"),
    (dict(out=t((2, 8, 64))), "out must have shape"),
    (dict(v_cache=t((6, 16, 2, 32))), "caches must be"),
    ({}, "must be on a GPU device"),
])
def test_decode_binding_rejects(kw, text):
    with pytest.raises(ValueError, match=text):
        ia.attn_decode_paged(**decode_args(**kw))


def test_backward_binding_rejects_wrong_lse():
    q = t((10, 4, 64))
    with pytest.raises(ValueError, match="lse must be"):
        ia.attn_prefill_varlen_backward(q, t((10, 2, 64)), t((10, 2, 64)), q, t((10, 2), f32), q,
                                        t((3,), i32), 8)


def test_wrong_dtype_is_a_type_error():
    with pytest.raises(TypeError, match="q must be"):
        ia.attn_prefill_varlen(**prefill_args(q=t((10, 4, 64), f32)))

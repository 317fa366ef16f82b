"""Full-size workloads on the GPU, in the launch configuration the benchmark
times: parity with the fp64 oracle on sampled rows (every sequence's first
and last rows, rows at the window edge and at span edges, plus a seeded
sample), and bitwise invariance of every row across batch composition.

Workloads (synthetic, seeded, built in GPU memory):
  sliding prefill  8 sequences, lengths U[512, 4096], 32/16 heads, head dim
                   256, window 1024
  global prefill   lengths {2048, 4096, 6144, 8192}, 32/4 heads, head dim
                   512, full causal, four batch orders
  paged decode     contexts U[1024, 32768], 32/4 heads, head dim 512,
                   16-token blocks, shuffled tables, batch 1 / 8 / 32 / 64
  hybrid prefill   5 sliding (window 1024, head dim 256, 32/16) + 1 global
                   (head dim 512, 32/4) layers over 4 x 4096 tokens with two
                   256-token bidirectional spans per sequence
Layer types and spans: "RFC: Gemma-4-31B-it train/rollout consistency",
sections 1, 3 and 7; paged decode: "Vime ROCm Attention operator ablation",
"Prerequisites"."""
import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import gate

pytestmark = pytest.mark.gpu


def host_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run(pf, cu_dev=None, spans_dev=None, max_seqlen=None, q=None, k=None, v=None):
    out = torch.empty_like(pf["q"] if q is None else q)
    ia.attn_prefill_varlen(pf["q"] if q is None else q, pf["k"] if k is None else k,
                           pf["v"] if v is None else v,
                           pf["cu_seqlens"] if cu_dev is None else cu_dev,
                           pf["max_seqlen"] if max_seqlen is None else max_seqlen,
                           window=pf["window"], softmax_scale=pf["scale"],
                           spans=pf["spans"] if spans_dev is None else spans_dev, out=out)
    torch.cuda.synchronize()
    return out


def sample_rows(lengths, cu, hq, window, spans_per_seq, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b, L in enumerate(lengths):
        a = int(cu[b])
        picks = {0, 1, L - 1, L // 2}
        if window > 0:
            picks |= {min(L - 1, window - 1), min(L - 1, window), min(L - 1, window + 31)}
        for s, e in (spans_per_seq[b] if spans_per_seq else []):
            picks |= {s, e - 1, min(L - 1, e)}
        for i in picks:
            for h in (0, hq - 1, int(rng.integers(hq))):
                rows.add((a + i, h))
    T = int(cu[-1])
    for _ in range(n_random):
        rows.add((int(rng.integers(T)), int(rng.integers(hq))))
    return np.array(sorted(rows), np.int64)


def check_parity(pf, out, lengths, spans_per_seq=None, n_random=256, seed=0, what=""):
    q, k, v = host_bits(pf["q"]), host_bits(pf["k"]), host_bits(pf["v"])
    rows = sample_rows(lengths, pf["cu_host"], pf["hq"], pf["window"], spans_per_seq, n_random, seed)
    ref = oracle.prefill(q, k, v, pf["cu_host"], window=pf["window"], scale=pf["scale"],
                         spans=pf["spans_host"] if len(pf["spans_host"]) else None, rows=rows)
    got = synth.bf16_to_f32(host_bits(out)[rows[:, 0], rows[:, 1]]).astype(np.float64)
    gate(got, ref, what)


def solo_equals_packed(pf, out, spans_per_seq=None):
    """Each sequence alone (its slice of the packed tensors) gives the same
    bytes as inside the packed batch."""
    cu = pf["cu_host"]
    packed = host_bits(out)
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        sp = None
        if spans_per_seq and spans_per_seq[b]:
            sp = torch.tensor(spans_per_seq[b], dtype=torch.int32, device="cuda")
        solo = torch.empty_like(pf["q"][a:e])
        ia.attn_prefill_varlen(pf["q"][a:e].contiguous(), pf["k"][a:e].contiguous(),
                               pf["v"][a:e].contiguous(),
                               torch.tensor([0, e - a], dtype=torch.int32, device="cuda"), e - a,
                               window=pf["window"], softmax_scale=pf["scale"], spans=sp, out=solo)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(solo), packed[a:e]), f"sequence {b} solo != packed"


def test_sliding_prefill_full_size():
    lengths = synth.sliding_lengths(2, 8, 512, 4096)
    pf = synth.prefill_case_device(2, lengths, 32, 16, 256, 1024)
    out = run(pf)
    check_parity(pf, out, lengths, what="sliding prefill")
    solo_equals_packed(pf, out)
    # prefix batches and an oversized grid give the same bytes
    bits = host_bits(out)
    for nb in (1, 3, 5):
        T = int(pf["cu_host"][nb])
        o2 = run(pf, cu_dev=pf["cu_seqlens"][:nb + 1].contiguous(), max_seqlen=max(lengths[:nb]),
                 q=pf["q"][:T].contiguous(), k=pf["k"][:T].contiguous(), v=pf["v"][:T].contiguous())
        assert np.array_equal(host_bits(o2), bits[:T]), f"prefix batch {nb}"
    o3 = run(pf, max_seqlen=2 * max(lengths))
    assert np.array_equal(host_bits(o3), bits)


def test_global_prefill_full_size_every_order():
    lengths = [2048, 4096, 6144, 8192]
    ref_bytes = None
    for oi, order in enumerate(synth.batch_orders(3, 4, count=2)):
        pf = synth.prefill_case_device(3, lengths, 32, 4, 512, synth.NO_WINDOW, order=order)
        out = run(pf)
        bits = host_bits(out)
        per = {}
        cu = pf["cu_host"]
        for pos, i in enumerate(order):
            per[i] = bits[cu[pos]:cu[pos + 1]]
        if ref_bytes is None:
            ref_bytes = per
            check_parity(pf, out, [lengths[i] for i in order], n_random=128, what="global prefill")
            solo_equals_packed(pf, out)
        else:
            for i in range(4):
                assert np.array_equal(per[i], ref_bytes[i]), f"order {order}: sequence {i}"


def test_hybrid_prefill_full_size():
    spans = synth.hybrid_spans(5, 4, 4096, 256)
    for layer, (hq, hkv, d, w) in enumerate(synth.HYBRID_LAYERS):
        if layer not in (0, 5):
            continue  # layers 1-4 repeat layer 0's geometry with other values
        pf = synth.prefill_case_device(500 + layer, [4096] * 4, hq, hkv, d, w, spans=spans)
        out = run(pf)
        check_parity(pf, out, [4096] * 4, spans_per_seq=spans, n_random=128, seed=layer,
                     what=f"hybrid layer {layer}")
        solo_equals_packed(pf, out, spans_per_seq=spans)


def gather_sequence(dc, b):
    """Host copy of one sequence's query and its blocks, renumbered."""
    L = int(dc["seq_lens"][b])
    nb = (L + 15) // 16
    ids = torch.from_numpy(dc["block_table"][b, :nb].astype(np.int64)).cuda()
    kc = host_bits(dc["k_cache"].index_select(0, ids))
    vc = host_bits(dc["v_cache"].index_select(0, ids))
    q = host_bits(dc["q"][b:b + 1])
    return q, kc, vc, np.arange(nb, dtype=np.int32)[None, :], np.array([L], np.int32)


def test_paged_decode_full_size_every_batch():
    lengths = synth.decode_lengths(4, 64, 1024, 32768)
    dc = synth.decode_case_device(4, lengths, batch=64, hq=32, hkv=4, d=512)
    out64 = None
    seq0 = None
    for B in (64, 32, 8, 1):
        bt = torch.from_numpy(np.ascontiguousarray(dc["block_table"][:B])).cuda()
        sl = torch.from_numpy(dc["seq_lens"][:B].copy()).cuda()
        o = ia.attn_decode_paged(dc["q"][:B].contiguous(), dc["k_cache"], dc["v_cache"], bt, sl,
                                 int(max(lengths[:B])), softmax_scale=dc["scale"])
        torch.cuda.synchronize()
        bits = host_bits(o)
        if out64 is None:
            out64 = bits
            seq0 = bits[0]
        assert np.array_equal(bits, out64[:B]), f"batch {B}"
    # sequence 0 at the last position of a batch of 9
    order = list(range(1, 9)) + [0]
    bt = torch.from_numpy(np.ascontiguousarray(dc["block_table"][order])).cuda()
    sl = torch.from_numpy(dc["seq_lens"][order].copy()).cuda()
    o = ia.attn_decode_paged(dc["q"][order].contiguous(), dc["k_cache"], dc["v_cache"], bt, sl,
                             int(max(lengths[:9])), softmax_scale=dc["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o)[8], seq0)
    # parity on three sequences (the longest, the shortest, sequence 0)
    for b in {0, int(np.argmax(lengths)), int(np.argmin(lengths))}:
        q, kc, vc, bt1, sl1 = gather_sequence(dc, b)
        ref = oracle.decode(q, kc, vc, bt1, sl1, scale=dc["scale"])
        gate(synth.bf16_to_f32(out64[b:b + 1]).astype(np.float64), ref, f"decode seq {b}")

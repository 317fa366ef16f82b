"""Prefill on the GPU: parity with the fp64 oracle, closed forms checked to
the bit, and bitwise batch invariance (solo vs packed vs permuted vs prefix
batches vs grid size vs repeat vs poisoned padding).

Invariance dimensions follow "RFC: Gemma-4-31B-it train/rollout
consistency", section 4, items 2 and 6; the solo-vs-batched comparison of
every row follows the reuse check of "Gated RMSNorm CUDA kernel for the GDN
block" (each row alone vs inside full batches, every start position)."""
import os
import zlib

import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import (bf16_dev, bits, f64, gate, i32_dev, run_case, run_prefill,
                      split_by_seq)

pytestmark = pytest.mark.gpu


def oracle_of(packed, case, want_lse=False, rows=None):
    q, k, v, cu, sp = packed
    return oracle.prefill(q, k, v, cu, window=case.window, scale=case.scale, spans=sp,
                          want_lse=want_lse, rows=rows)


# --------------------------------------------------------------------- parity
@pytest.mark.parametrize("window", [32, synth.NO_WINDOW], ids=["window32", "global"])
def test_tiny_case_parity(window):
    """One sequence of 128 tokens, 4/2 heads, head dim 64 (fp32 inputs; the
    kernel reads their bf16 rounding)."""
    case = synth.tiny_case(seed=1, window=window)
    packed, o, lse = run_case(case, want_lse=True)
    ref, ref_lse = oracle_of(packed, case, want_lse=True)
    gate(f64(o), ref, f"tiny w={window}")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3
    # Against the oracle on the unrounded fp32 inputs (reported; looser gate).
    q32, k32, v32 = case.q32[0]
    ref32 = oracle.prefill(q32, k32, v32, packed[3], window=window, scale=case.scale)
    assert np.abs(f64(o) - ref32).max() <= 5e-2


PARITY_CASES = [
    # (name, lengths, hq, hkv, d, window, spans)
    ("d64-g1", [1, 65, 200], 2, 2, 64, 48, None),
    ("d64-g2", [130, 7], 4, 2, 64, synth.NO_WINDOW, None),
    ("d64-g4", [129, 64, 63], 8, 2, 64, 17, None),
    ("d64-g8", [300], 8, 1, 64, 100, [[(3, 40), (120, 290)]]),
    ("sliding-d256", [1, 37, 300, 513], 32, 16, 256, 128, None),
    ("sliding-d256-g4", [96, 257], 16, 4, 256, 64, None),
    ("sliding-d256-spans", [400, 333], 32, 16, 256, 64, [[(10, 140), (200, 233)], [(0, 50)]]),
    ("global-d512", [1, 130, 333, 600], 32, 4, 512, synth.NO_WINDOW, None),
    ("global-d512-g2", [77, 200], 8, 4, 512, synth.NO_WINDOW, None),
    ("global-d512-spans", [500, 260], 32, 4, 512, synth.NO_WINDOW, [[(100, 356)], [(4, 260)]]),
    ("sliding-d512-g1", [150], 4, 4, 512, 40, None),
]


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window,spans", PARITY_CASES,
                         ids=[c[0] for c in PARITY_CASES])
def test_parity(name, lengths, hq, hkv, d, window, spans):
    case = synth.prefill_case(zlib.crc32(name.encode()) % 1000, lengths, hq, hkv, d, window, std=0.5, spans=spans)
    packed, o, lse = run_case(case, want_lse=True)
    ref, ref_lse = oracle_of(packed, case, want_lse=True)
    gate(f64(o), ref, name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3, name


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("d,hq,hkv,window", [(64, 4, 2, 20), (256, 8, 4, 70), (512, 8, 1, -1)])
def test_zero_query_gives_exact_mean(d, hq, hkv, window):
    """Q = 0: every allowed score is 0, p = 1, l = |A_i| and acc = sum of V
    over A_i, all exact in fp32; the output is bf16(fp32(sum)/fp32(count))
    to the bit.  V_j = (j mod 256, j // 256, 1, 0, ...) makes the sums count
    the allowed set, pinning the window edge, the causal edge and span edges."""
    L = 700
    spans = [(30, 90), (400, 650)]
    q = np.zeros((L, hq, d), np.uint16)
    k = synth.bf16_bits(np.random.default_rng(5).standard_normal((L, hkv, d), dtype=np.float32))
    vf = np.zeros((L, hkv, d), np.float32)
    j = np.arange(L)
    vf[:, :, 0] = (j % 256)[:, None]
    vf[:, :, 1] = (j // 256)[:, None]
    vf[:, :, 2] = 1.0
    v = synth.bf16_bits(vf)
    o, lse = run_prefill(q, k, v, [0, L], L, window, spans, None, want_lse=True)
    got = bits(o)
    want = np.zeros((L, 3), np.uint16)
    count = np.zeros(L)
    for i in range(L):
        keys = set(range(0, i + 1)) if window < 0 else set(range(max(0, i - window + 1), i + 1))
        for s, e in spans:
            if s <= i < e:
                keys |= set(range(s, e))
        keys = np.array(sorted(keys))
        n = np.float32(len(keys))
        count[i] = len(keys)
        sums = [np.float32((keys % 256).sum()), np.float32((keys // 256).sum()), n]
        want[i] = synth.bf16_bits(np.array([np.float32(x) / n for x in sums], np.float32))
    for h in range(hq):
        assert np.array_equal(got[:, h, :3], want), f"head {h}"
        assert not got[:, h, 3:].any()
    assert np.abs(lse.cpu().numpy() - np.log(count)[:, None]).max() <= 1e-5


@pytest.mark.parametrize("d", [64, 256, 512])
def test_single_key_returns_v_exactly(d):
    """Window 1 (or a one-token sequence): each row sees only its own key, so
    p = 1, l = 1 and the output is V itself, bit for bit."""
    case = synth.prefill_case(3, [1, 90, 1], 8, 2, d, 1, std=1.0)
    packed, o, _ = run_case(case)
    v = packed[2]
    assert np.array_equal(bits(o), np.repeat(v, 4, axis=1))


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (256, 8, 4), (512, 8, 1)])
def test_underflowing_rows_take_their_first_max(d, hq, hkv):
    """Softmax scale 30: many rows' scaled scores lie below -150, so every p
    underflows against the provisional reference 0 of a row that has not
    seen an allowed key yet.  The row must still take its first reference
    max (from the allowed keys, not from p > 0): with window 1 the output is
    V to the bit and the LSE is the row's own scaled score; with wider
    windows it matches the oracle.  Every head dim's kernel and the decode of
    the last rows agree with the oracle."""
    scale = 30.0
    case = synth.prefill_case(23, [1, 70, 33], hq, hkv, d, 1, std=0.5)
    case.scale = scale
    packed, o, lse = run_case(case, want_lse=True)
    q, k, v, cu, _ = packed
    assert np.array_equal(bits(o), np.repeat(v, hq // hkv, axis=1))
    ref_o, ref_lse = oracle_of(packed, case, want_lse=True)
    got_lse = lse.cpu().numpy()
    assert np.isfinite(got_lse).all()
    assert (ref_lse < -100).any()                      # the case really underflows
    assert np.abs(got_lse - ref_lse).max() <= 1e-5 * np.abs(ref_lse).max() + 1e-3
    for w in (3, 40, synth.NO_WINDOW):
        case.window = w
        packed, o, lse = run_case(case, want_lse=True)
        ref_o, ref_lse = oracle_of(packed, case, want_lse=True)
        gate(f64(o), ref_o, f"scale 30, window {w}")
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-5 * np.abs(ref_lse).max() + 1e-3
    # the same rows through the paged decode: each sequence's last row
    for b in range(len(cu) - 1):
        L = int(cu[b + 1] - cu[b])
        nblk = (L + 15) // 16
        kc = np.zeros((nblk, 16, hkv, d), np.uint16)
        vc = np.zeros((nblk, 16, hkv, d), np.uint16)
        kc.reshape(-1, hkv, d)[:L] = k[cu[b]:cu[b + 1]]
        vc.reshape(-1, hkv, d)[:L] = v[cu[b]:cu[b + 1]]
        qd = q[cu[b + 1] - 1][None]
        bt = np.arange(nblk, dtype=np.int32)[None]
        sl = np.array([L], np.int32)
        od = ia.attn_decode_paged(bf16_dev(qd), bf16_dev(kc), bf16_dev(vc), i32_dev(bt),
                                  i32_dev(sl), L, window=synth.NO_WINDOW, softmax_scale=scale)
        torch.cuda.synchronize()
        gate(f64(od)[0], ref_o[cu[b + 1] - 1], f"decode seq {b}")


def test_window_covering_sequence_is_global_bytes():
    case = synth.prefill_case(4, [200, 333], 8, 4, 256, synth.NO_WINDOW)
    _, og, _ = run_case(case)
    for w in (333, 334, 5000):
        case.window = w
        _, ow, _ = run_case(case)
        assert torch.equal(og.view(torch.int16), ow.view(torch.int16)), w


# ------------------------------------------------------------ batch invariance
INVARIANCE_CASES = [
    ("sliding-d256", [513, 37, 300, 1, 1024], 32, 16, 256, 128, None),
    ("global-d512", [333, 600, 130, 1], 32, 4, 512, synth.NO_WINDOW, None),
    ("spans-d256", [400, 333, 129], 32, 16, 256, 64, [[(10, 140)], [(0, 50), (300, 333)], []]),
    ("d64-g8", [257, 64, 5], 16, 2, 64, 33, None),
]


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window,spans", INVARIANCE_CASES,
                         ids=[c[0] for c in INVARIANCE_CASES])
def test_bitwise_batch_invariance(name, lengths, hq, hkv, d, window, spans):
    """Every sequence's output bytes are identical alone, packed, in reversed
    and shuffled order, in every prefix batch, with an oversized grid, and on
    repeat."""
    case = synth.prefill_case(11, lengths, hq, hkv, d, window, spans=spans)
    n = len(lengths)
    solo = {}
    for i in range(n):
        sub = synth.PrefillCase([case.seqs[i]], hq, hkv, d, window, case.scale)
        _, o, _ = run_case(sub)
        solo[i] = bits(o)
    runs = []
    for order in synth.batch_orders(11, n, count=2):
        runs.append((order, None))
    runs.append((list(range(n)), 2 * case.max_seqlen() + 77))      # oversized grid
    for b in range(1, n):
        runs.append((list(range(b)), None))                         # prefix batches
    for order, ms in runs:
        packed, o, _ = run_case(case, order=order, max_seqlen=ms)
        per = split_by_seq(bits(o), packed[3], order)
        for i, got in per.items():
            assert np.array_equal(got, solo[i]), f"{name}: seq {i} order {order} max_seqlen {ms}"
    # L0: repeat the same call
    packed, o1, _ = run_case(case)
    for _ in range(3):
        _, o2, _ = run_case(case)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_poisoned_padding_changes_nothing():
    """NaN in buffer rows beyond the packed tokens, and a pre-filled output
    buffer, change no live output byte and no output row outside the batch is
    written."""
    case = synth.prefill_case(12, [300, 129, 64], 16, 8, 256, 96)
    q, k, v, cu, _ = case.pack()
    T = q.shape[0]
    _, clean, _ = run_case(case)
    pad = 50
    nanq = np.full((T + pad,) + q.shape[1:], synth.BF16_NAN, np.uint16)
    nank = np.full((T + pad,) + k.shape[1:], synth.BF16_NAN, np.uint16)
    nanv = nank.copy()
    nanq[:T], nank[:T], nanv[:T] = q, k, v
    out = torch.full((T + pad,) + q.shape[1:], 7.0, dtype=torch.bfloat16, device="cuda")
    o, _ = run_prefill(nanq, nank, nanv, cu, case.max_seqlen(), case.window, None, case.scale, out=out)
    assert np.array_equal(bits(o)[:T], bits(clean))
    assert (o[T:].float() == 7.0).all()


def test_empty_sequences_and_batches():
    case = synth.prefill_case(13, [0, 50, 0, 70, 0], 8, 4, 64, 16)
    packed, o, _ = run_case(case)
    ref = oracle_of(packed, case)
    gate(f64(o), ref, "empty sequences")
    # batch 0 and max_seqlen 0 enqueue nothing
    qt = torch.zeros(0, 8, 64, dtype=torch.bfloat16, device="cuda")
    kt = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    ia.attn_prefill_varlen(qt, kt, kt, i32_dev([0]), 0)
    ia.attn_prefill_varlen(qt, kt, kt, i32_dev([0, 0]), 0)


def test_validation_rejects_bad_indices(monkeypatch):
    monkeypatch.setenv("INVATTN_VALIDATE", "1")
    case = synth.prefill_case(14, [40, 30], 8, 4, 64, 16)
    q, k, v, cu, _ = case.pack()
    with pytest.raises(ia.AttnError) as e:
        run_prefill(q, k, v, np.array([0, 50, 30], np.int32), 64, 16)
    assert e.value.name == "ATTN_E_VALIDATE"
    with pytest.raises(ia.AttnError) as e:
        run_prefill(q, k, v, cu, 35, 16)            # a sequence longer than max_seqlen
    assert e.value.name == "ATTN_E_VALIDATE"
    with pytest.raises(ia.AttnError) as e:
        run_prefill(q, k, v, cu, 64, 16, spans=[(30, 45)])   # span crosses sequences
    assert e.value.name == "ATTN_E_VALIDATE"
    o, _ = run_prefill(q, k, v, cu, 64, 16, spans=[(5, 20), (41, 60)])
    ref = oracle.prefill(q, k, v, cu, window=16, spans=[(5, 20), (41, 60)])
    gate(f64(o), ref, "validated call")


def test_provenance_record():
    case = synth.prefill_case(15, [64], 8, 1, 512, synth.NO_WINDOW)
    run_case(case)
    p = ia.last_provenance()
    assert p["op"] == "attn_prefill_varlen" and p["fallback"] == "none"
    assert p["accumulator_dtype"] == "fp32" and p["layer_type"] == "global"
    assert p["schedule_id"].startswith("prefill_d512_g8")
    assert p["kernel_id"].startswith("prefill_ws_kernel<512,8,")
    assert p["shape"]["max_len"] == 64
    assert p["arch"].startswith("gfx950")

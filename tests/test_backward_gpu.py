"""Attention backward on the GPU: parity of dq, dk, dv with the fp64 oracle
(the chain rule on the forward's definition), the window-1 closed form to
the bit, and bitwise invariance of every gradient to the batch, the packing
and the grid.

The fixed-order, atomic-free reduction rules follow "RFC: Gemma-4-31B-it
train/rollout consistency", section 4, items 1 and 3; the forward's mask,
spans and GQA map are those of the forward tests."""
import zlib

import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import bf16_dev, dev, i32_dev, run_prefill

pytestmark = pytest.mark.gpu

# Gradient gate: the kernel's delta_i uses the forward's bf16 output (the
# oracle's uses its exact output), so the gate is relative to each gradient's
# scale.
GRAD_RTOL = 1e-2   # ||gpu - oracle||_2 / ||oracle||_2
GRAD_ATOL = 2e-2   # max |gpu - oracle| / max |oracle|


def grad_gate(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if scale == 0.0:
        assert not got.any(), f"{what}: expected zeros"
        return
    err = float(np.abs(got - ref).max()) / scale
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert err <= GRAD_ATOL and rel <= GRAD_RTOL, f"{what}: max-abs/max {err:.3g}, rel {rel:.3g}"


def run_backward(q, k, v, cu, max_seqlen, window, spans, scale, dout, total=None,
                 poison=False):
    """Forward then backward on the device; returns (dq, dk, dv) fp32 tensors."""
    qt, kt, vt = bf16_dev(q), bf16_dev(k), bf16_dev(v)
    o, lse = run_prefill(qt, kt, vt, cu, max_seqlen, window, spans, scale, want_lse=True)
    spt = i32_dev(np.asarray(spans).reshape(-1, 2)) if spans is not None and len(spans) else None
    outs = None
    if poison:
        outs = dict(dq=torch.full(qt.shape, float("nan"), device=dev()),
                    dk=torch.full(kt.shape, float("nan"), device=dev()),
                    dv=torch.full(kt.shape, float("nan"), device=dev()))
    res = ia.attn_prefill_varlen_backward(qt, kt, vt, o, lse, bf16_dev(dout), i32_dev(cu),
                                          max_seqlen, window=window, softmax_scale=scale,
                                          spans=spt, **(outs or {}))
    torch.cuda.synchronize()
    return res


def case_grads(case, order=None, max_seqlen=None):
    q, k, v, cu, sp = case.pack(order)
    dout = case.dout if order is None else np.concatenate(
        [case.dout_of[i] for i in order]) if len(order) else case.dout[:0]
    ms = case.max_seqlen() if max_seqlen is None else max_seqlen
    return (q, k, v, cu, sp, dout), run_backward(q, k, v, cu, ms, case.window, sp, case.scale,
                                                 dout)


def make_case(name, lengths, hq, hkv, d, window, spans=None, std=0.5):
    seed = zlib.crc32(name.encode()) % 1000
    case = synth.prefill_case(seed, lengths, hq, hkv, d, window, std=std, spans=spans)
    case.dout_of = [synth.upstream_grad(seed * 100 + i, (L, hq, d)) for i, L in enumerate(lengths)]
    case.dout = np.concatenate(case.dout_of) if lengths else np.zeros((0, hq, d), np.uint16)
    return case


PARITY_CASES = [
    # (name, lengths, hq, hkv, d, window, spans)
    ("d64-g1", [1, 65, 200], 2, 2, 64, 48, None),
    ("d64-g2-global", [130, 7], 4, 2, 64, synth.NO_WINDOW, None),
    ("d64-g4", [129, 64, 63], 8, 2, 64, 17, None),
    ("d64-g8-spans", [300], 8, 1, 64, 100, [[(3, 40), (120, 290)]]),
    ("sliding-d256", [1, 37, 300], 8, 4, 256, 128, None),
    ("sliding-d256-spans", [260, 133], 4, 2, 256, 64, [[(10, 140), (200, 233)], [(0, 50)]]),
    ("global-d512", [1, 130, 290], 8, 1, 512, synth.NO_WINDOW, None),
    ("global-d512-spans", [200, 97], 4, 2, 512, synth.NO_WINDOW, [[(100, 180)], [(4, 97)]]),
]


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window,spans", PARITY_CASES,
                         ids=[c[0] for c in PARITY_CASES])
def test_parity(name, lengths, hq, hkv, d, window, spans):
    case = make_case(name, lengths, hq, hkv, d, window, spans)
    (q, k, v, cu, sp, dout), (dq, dk, dv) = case_grads(case)
    rq, rk, rv = oracle.prefill_backward(q, k, v, dout, cu, window=window, scale=case.scale,
                                         spans=sp)
    grad_gate(dq.cpu().numpy(), rq, f"{name} dq")
    grad_gate(dk.cpu().numpy(), rk, f"{name} dk")
    grad_gate(dv.cpu().numpy(), rv, f"{name} dv")


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (256, 4, 4), (512, 8, 1)])
def test_window_one_closed_form(d, hq, hkv):
    """Window 1: each row sees only its own key and the forward's output is
    V itself, so dp_ii = delta_i to the bit, ds = 0 and dq = dk = 0 exactly;
    p = 1 up to the rounding of the stored LSE, so dv_j is the sum of dout
    over the group's heads to a few fp32 ulps."""
    case = make_case(f"w1-{d}", [1, 90, 33], hq, hkv, d, 1, std=1.0)
    (q, k, v, cu, sp, dout), (dq, dk, dv) = case_grads(case)
    assert not dq.cpu().numpy().any()
    assert not dk.cpu().numpy().any()
    g = hq // hkv
    df = synth.bf16_to_f32(dout).reshape(dout.shape[0], hkv, g, d)
    want = df[:, :, 0].copy()
    for h in range(1, g):
        want = want + df[:, :, h]
    mag = np.abs(df).sum(axis=2)
    assert np.all(np.abs(dv.cpu().numpy() - want) <= 1e-6 * mag + 1e-30)


INVARIANCE_CASES = [
    ("sliding-d256", [300, 37, 1, 200], 8, 4, 256, 64, None),
    ("global-d512-spans", [150, 90, 1], 8, 2, 512, synth.NO_WINDOW, [[(10, 60)], [(0, 90)], []]),
    ("d64-g8", [257, 64, 5], 16, 2, 64, 33, None),
]


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window,spans", INVARIANCE_CASES,
                         ids=[c[0] for c in INVARIANCE_CASES])
def test_bitwise_batch_invariance(name, lengths, hq, hkv, d, window, spans):
    """Each sequence alone, in the packed batch, in reverse order and with a
    larger grid: dq, dk and dv of every token identical to the bit; a repeat
    call returns the same bytes."""
    case = make_case(name, lengths, hq, hkv, d, window, spans)
    n = len(lengths)
    runs = [(list(range(n)), None), (list(reversed(range(n))), None),
            (list(range(n)), 2 * case.max_seqlen() + 17)]
    ref = None
    for order, ms in runs + [runs[0]]:
        (_, _, _, cu, _, _), grads = case_grads(case, order, ms)
        got = {}
        for pos, i in enumerate(order):
            got[i] = [g[cu[pos]:cu[pos + 1]].cpu().numpy().view(np.uint32) for g in grads]
        if ref is None:
            ref = got
            continue
        for i in range(n):
            for a, b, what in zip(ref[i], got[i], ("dq", "dk", "dv")):
                assert np.array_equal(a, b), f"{name}: seq {i} {what} order={order} ms={ms}"
    for i in range(n):
        solo = make_case(name, lengths, hq, hkv, d, window, spans)
        solo.seqs = [case.seqs[i]]
        solo.dout_of = [case.dout_of[i]]
        solo.dout = case.dout_of[i]
        _, grads = case_grads(solo)
        for a, b, what in zip(ref[i], grads, ("dq", "dk", "dv")):
            assert np.array_equal(a, b.cpu().numpy().view(np.uint32)), f"{name}: seq {i} {what} solo"


def test_rows_outside_sequences_untouched_and_empty():
    """Tokens after cu_seqlens[batch] keep their contents; zero-length
    sequences and an empty batch are accepted."""
    case = make_case("pad", [40, 0, 70], 4, 2, 64, 16)
    q, k, v, cu, sp = case.pack()
    pad = 9
    T = q.shape[0]
    qp = np.concatenate([q, np.zeros((pad,) + q.shape[1:], np.uint16)])
    kp = np.concatenate([k, np.zeros((pad,) + k.shape[1:], np.uint16)])
    vp = np.concatenate([v, np.zeros((pad,) + v.shape[1:], np.uint16)])
    dp = np.concatenate([case.dout, np.zeros((pad,) + q.shape[1:], np.uint16)])
    dq, dk, dv = run_backward(qp, kp, vp, cu, case.max_seqlen(), case.window, None, case.scale,
                              dp, poison=True)
    for g in (dq, dk, dv):
        g = g.cpu().numpy()
        assert np.isfinite(g[:T]).all()
        assert np.isnan(g[T:]).all()
    rq, rk, rv = oracle.prefill_backward(q, k, v, case.dout, cu, window=case.window,
                                         scale=case.scale)
    grad_gate(dq.cpu().numpy()[:T], rq, "pad dq")
    grad_gate(dk.cpu().numpy()[:T], rk, "pad dk")
    grad_gate(dv.cpu().numpy()[:T], rv, "pad dv")
    z = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=dev())
    zl = torch.zeros((0, 4), dtype=torch.float32, device=dev())
    zk = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=dev())
    ia.attn_prefill_varlen_backward(z, zk, zk, z, zl, z, i32_dev([0]), 0)
    ia.attn_prefill_varlen_backward(z, zk, zk, z, zl, z, i32_dev([0, 0, 0]), 0)
    torch.cuda.synchronize()


def sampled_parity(full, cu, case, i, seed, n_dq=48, n_kv=32, kv_from=0, kv_heads=None):
    """Gradients of sequence i of a full-size launch against the oracle on
    that sequence alone, at seeded units: dq at n_dq (row, query head) pairs,
    dk and dv at n_kv (key, KV head) pairs with keys in [kv_from, L) and
    heads from kv_heads (default all).  The first and last rows and the last
    key are always among them."""
    s = case.seqs[i]
    L = s.length
    rng = np.random.default_rng([seed, i])
    heads = np.arange(case.hkv) if kv_heads is None else np.asarray(kv_heads)
    dq_units = np.stack([rng.integers(0, L, n_dq), rng.integers(0, case.hq, n_dq)], 1)
    dq_units[0], dq_units[1] = (0, 0), (L - 1, case.hq - 1)
    kv_units = np.stack([rng.integers(kv_from, L, n_kv), rng.choice(heads, n_kv)], 1)
    kv_units[0] = (L - 1, heads[0])
    rq, rk, rv = oracle.prefill_backward(s.q, s.k, s.v, case.dout_of[i], [0, L],
                                         window=case.window, scale=case.scale,
                                         dq_units=dq_units, kv_units=kv_units)
    o = cu[i]
    grad_gate(full[0][o + dq_units[:, 0], dq_units[:, 1]], rq, f"seq {i} (L {L}) dq")
    grad_gate(full[1][o + kv_units[:, 0], kv_units[:, 1]], rk, f"seq {i} (L {L}) dk")
    grad_gate(full[2][o + kv_units[:, 0], kv_units[:, 1]], rv, f"seq {i} (L {L}) dv")


def test_full_size_sliding_workload():
    """The benchmark's sliding prefill (8 sequences, lengths U[512, 4096],
    32/16 heads, head dim 256, window 1024) in the launch the benchmark
    times: every sequence's dq, dk and dv alone equal its rows of the packed
    batch to the bit, the shortest sequence matches the oracle everywhere and
    the longest at seeded units spread over the whole sequence."""
    case = synth.sliding_case()
    case.dout_of = [synth.upstream_grad(900 + i, (s.length, case.hq, case.d))
                    for i, s in enumerate(case.seqs)]
    case.dout = np.concatenate(case.dout_of)
    (q, k, v, cu, sp, dout), grads = case_grads(case)
    full = [g.cpu().numpy() for g in grads]
    for gr in full:
        assert np.isfinite(gr).all()
    lengths = [s.length for s in case.seqs]
    for i in range(len(lengths)):
        solo = make_case("solo", [1], case.hq, case.hkv, case.d, case.window)
        solo.seqs = [case.seqs[i]]
        solo.dout_of = [case.dout_of[i]]
        solo.dout = case.dout_of[i]
        _, sg = case_grads(solo)
        for a, b_, what in zip(full, sg, ("dq", "dk", "dv")):
            assert np.array_equal(a[cu[i]:cu[i + 1]].view(np.uint32),
                                  b_.cpu().numpy().view(np.uint32)), f"seq {i} {what}"
    i = int(np.argmin(lengths))
    s = case.seqs[i]
    rq, rk, rv = oracle.prefill_backward(s.q, s.k, s.v, case.dout_of[i], [0, s.length],
                                         window=case.window, scale=case.scale)
    sl = slice(cu[i], cu[i + 1])
    grad_gate(full[0][sl], rq, "full dq")
    grad_gate(full[1][sl], rk, "full dk")
    grad_gate(full[2][sl], rv, "full dv")
    sampled_parity(full, cu, case, int(np.argmax(lengths)), 77)


def test_validation_rejects_bad_indices(monkeypatch):
    """INVATTN_VALIDATE=1: the backward applies the forward's index checks
    (cu_seqlens, spans) and checks cu_seqlens[batch] against total_tokens."""
    case = make_case("validate", [40, 30], 8, 4, 64, 16)
    q, k, v, cu, _ = case.pack()
    qt, kt, vt = bf16_dev(q), bf16_dev(k), bf16_dev(v)
    o, lse = run_prefill(qt, kt, vt, cu, 64, 16, want_lse=True)
    do = bf16_dev(case.dout)
    monkeypatch.setenv("INVATTN_VALIDATE", "1")

    def call(cu_, ms, spans=None, T=None):
        spt = i32_dev(np.asarray(spans, np.int32).reshape(-1, 2)) if spans else None
        n = q.shape[0] if T is None else T
        return ia.attn_prefill_varlen_backward(qt[:n], kt[:n], vt[:n], o[:n], lse[:n], do[:n],
                                               i32_dev(cu_), ms, window=16, spans=spt)

    for bad in ((np.array([0, 50, 30], np.int32), 64, None, None),   # decreasing
                (cu, 35, None, None),                                 # longer than max_seqlen
                (cu, 64, [(30, 45)], None),                           # span crosses sequences
                (cu, 64, None, 60)):                                  # past total_tokens
        with pytest.raises(ia.AttnError) as e:
            call(*bad)
        assert e.value.name == "ATTN_E_VALIDATE", bad
    dq, dk, dv = call(cu, 64, [(5, 20), (41, 60)])
    torch.cuda.synchronize()
    assert np.isfinite(dq.cpu().numpy()).all()


def test_full_size_global_workload():
    """The global-layer prefill (4 sequences of 2048-8192 tokens, 32/4 heads,
    head dim 512): every sequence's dq, dk and dv alone equal its rows of the
    packed batch to the bit, and the shortest and longest sequences match the
    oracle at seeded units: dq at rows spread over the sequence, dk and dv at
    keys of the last 256 positions of two KV heads (a key's gradient reads
    every later row, so keys near the end keep the oracle's cost small)."""
    case = synth.global_case()
    case.dout_of = [synth.upstream_grad(950 + i, (s.length, case.hq, case.d))
                    for i, s in enumerate(case.seqs)]
    case.dout = np.concatenate(case.dout_of)
    (q, k, v, cu, sp, dout), grads = case_grads(case)
    full = [g.cpu().numpy() for g in grads]
    del grads
    for gr in full:
        assert np.isfinite(gr).all()
    for i in range(len(case.seqs)):
        solo = make_case("solo", [1], case.hq, case.hkv, case.d, case.window)
        solo.seqs = [case.seqs[i]]
        solo.dout_of = [case.dout_of[i]]
        solo.dout = case.dout_of[i]
        _, sg = case_grads(solo)
        for a, b_, what in zip(full, sg, ("dq", "dk", "dv")):
            assert np.array_equal(a[cu[i]:cu[i + 1]].view(np.uint32),
                                  b_.cpu().numpy().view(np.uint32)), f"seq {i} {what}"
    lengths = [s.length for s in case.seqs]
    for i in (int(np.argmin(lengths)), int(np.argmax(lengths))):
        sampled_parity(full, cu, case, i, 78, n_dq=32, n_kv=24,
                       kv_from=lengths[i] - 256, kv_heads=(1, 3))

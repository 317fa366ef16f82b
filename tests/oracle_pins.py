"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself (hand-worked values, brute force, closed forms, invariants).

Each function takes an optional oracle library handle so the same pins can be
run against deliberately broken copies of the oracle (see test_oracle.py).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import bruteforce

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _num(x):
    """Parse the hand-worked fixture's numbers: 3, "8/3", "2ln2", "ln(11/6)"."""
    if isinstance(x, (int, float)):
        return float(x)
    s = x.replace(" ", "")
    coef = 1.0
    if "ln" in s:
        head, arg = s.split("ln", 1)
        if head:
            coef = float(head)
        arg = arg.strip("()")
        return coef * math.log(float(Fraction(arg)))
    return float(Fraction(s))


def pin_golden(lib=None):
    g = json.load(open(GOLDEN))
    k1 = np.array([[_num(x) for x in row] for row in g["k"]])
    v1 = np.array([[_num(x) for x in row] for row in g["v"]], np.float64)
    for case in g["cases"]:
        signs = case["q_sign"]
        hq = len(signs)
        q = np.zeros((3, hq, 4))
        for h, sg in enumerate(signs):
            q[:, h, 0] = sg
        k = k1[:, None, :]
        v = v1[:, None, :]
        o, lse = oracle.prefill(q, k, v, [0, 3], window=case["window"], scale=0.5,
                                spans=case["spans"] or None, want_lse=True, lib=lib)
        want_o = np.array([[[_num(x) for x in head] for head in row] for row in case["o"]])
        want_l = np.array([[_num(x) for x in row] for row in case["lse"]])
        assert np.allclose(o, want_o, rtol=0, atol=1e-12), case["name"]
        assert np.allclose(lse, want_l, rtol=0, atol=1e-12), case["name"]


def _random_case(rng, lengths, hq, hkv, d, span_count=0):
    T = sum(lengths)
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    spans = []
    for b, L in enumerate(lengths):
        for _ in range(span_count):
            if L < 3:
                continue
            s = int(rng.integers(0, L - 2))
            e = int(rng.integers(s + 1, L))   # ends before the sequence end
            if all(e <= a - cu[b] or s >= c - cu[b] for a, c in spans if cu[b] <= a < cu[b + 1]):
                spans.append((int(cu[b]) + s, int(cu[b]) + e))
    spans.sort()
    return q, k, v, cu, spans


def pin_bruteforce(lib=None):
    rng = np.random.default_rng(12345)
    configs = [
        ([17], 2, 1, 8, -1, 0),
        ([5, 31, 1, 12], 4, 2, 16, 3, 1),
        ([40, 9], 4, 4, 8, 1, 1),
        ([33, 20, 2], 8, 1, 4, 7, 2),
        ([64], 4, 2, 32, 100, 2),
    ]
    for lengths, hq, hkv, d, w, nsp in configs:
        q, k, v, cu, spans = _random_case(rng, lengths, hq, hkv, d, nsp)
        o, lse = oracle.prefill(q, k, v, cu, window=w, spans=spans or None, want_lse=True, lib=lib)
        bo, bl = bruteforce.attention(q, k, v, cu, window=w, spans=spans)
        assert np.abs(o - bo).max() <= 1e-12, (lengths, w)
        assert np.abs(lse - bl).max() <= 1e-12, (lengths, w)


def pin_rows_sum_to_one(lib=None):
    rng = np.random.default_rng(7)
    q, k, v, cu, spans = _random_case(rng, [30, 45], 4, 2, 16, 1)
    v = np.ones_like(v)
    for w in (-1, 1, 5):
        o = oracle.prefill(q, k, v, cu, window=w, spans=spans, lib=lib)
        assert np.abs(o - 1.0).max() <= 1e-13


def pin_window_covering_sequence_is_global(lib=None):
    rng = np.random.default_rng(8)
    q, k, v, cu, _ = _random_case(rng, [19, 50], 2, 1, 8)
    og = oracle.prefill(q, k, v, cu, window=-1, lib=lib)
    for w in (50, 51, 1000):
        assert np.array_equal(oracle.prefill(q, k, v, cu, window=w, lib=lib), og)


def pin_one_token_returns_v(lib=None):
    rng = np.random.default_rng(9)
    q, k, v, cu, _ = _random_case(rng, [1, 1, 1], 4, 2, 8)
    o = oracle.prefill(q, k, v, cu, lib=lib)
    assert np.array_equal(o, np.repeat(v, 2, axis=1))
    q, k, v, cu, _ = _random_case(rng, [23], 4, 2, 8)
    o = oracle.prefill(q, k, v, cu, window=1, lib=lib)
    assert np.array_equal(o, np.repeat(v, 2, axis=1))


def _allowed_set(i, L, w, spans):
    keys = set(range(0, i + 1)) if w < 0 else set(range(max(0, i - w + 1), i + 1))
    for s, e in spans:
        if s <= i < e:
            keys |= set(range(s, e))
    return keys


def pin_zero_query_is_mean(lib=None):
    """Q = 0: every allowed score is 0, so the output is the plain mean of V
    over the allowed set and lse = log(count).  V_j = (j mod 256, j // 256, 1)."""
    L, d = 300, 4
    j = np.arange(L)
    v = np.zeros((L, 1, d))
    v[:, 0, 0] = j % 256
    v[:, 0, 1] = j // 256
    v[:, 0, 2] = 1
    q = np.zeros((L, 2, d))
    k = np.random.default_rng(3).standard_normal((L, 1, d))
    spans = [(10, 40), (200, 270)]
    for w in (-1, 1, 16, 64):
        o, lse = oracle.prefill(q, k, v, [0, L], window=w, spans=spans, want_lse=True, lib=lib)
        for i in range(L):
            keys = sorted(_allowed_set(i, L, w, spans))
            want = [np.mean([x % 256 for x in keys]), np.mean([x // 256 for x in keys]), 1.0, 0.0]
            assert np.allclose(o[i, 0], want, rtol=0, atol=1e-12), (w, i)
            assert np.allclose(o[i, 1], want, rtol=0, atol=1e-12), (w, i)
            assert abs(lse[i, 0] - math.log(len(keys))) <= 1e-12, (w, i)


def pin_dominant_key(lib=None):
    """q_i = alpha * k_t for an allowed t: the output tends to v_t; very large
    alpha must not overflow (the max is subtracted before exponentiation)."""
    rng = np.random.default_rng(11)
    L, d = 40, 16
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    for alpha in (200.0, 1e5):
        q = np.zeros((L, 1, d))
        targets = []
        for i in range(L):
            t = int(rng.integers(max(0, i - 7), i + 1))   # inside window 8
            targets.append(t)
            q[i, 0] = alpha * k[t, 0]
        o = oracle.prefill(q, k, v, [0, L], window=8, lib=lib)
        for i in range(L):
            assert np.allclose(o[i, 0], v[targets[i], 0], rtol=0, atol=1e-6), (alpha, i)
    # a key outside the window never wins, however strong
    q = np.zeros((L, 1, d))
    q[20, 0] = 1e5 * k[5, 0]
    o = oracle.prefill(q, k, v, [0, L], window=8, lib=lib)
    assert not np.allclose(o[20, 0], v[5, 0], atol=1e-3)


def pin_gqa_reduces_to_mha(lib=None):
    rng = np.random.default_rng(13)
    q, k, v, cu, spans = _random_case(rng, [25, 14], 8, 2, 8, 1)
    o = oracle.prefill(q, k, v, cu, window=6, spans=spans, lib=lib)
    k4 = np.repeat(k, 4, axis=1)
    v4 = np.repeat(v, 4, axis=1)
    assert np.array_equal(oracle.prefill(q, k4, v4, cu, window=6, spans=spans, lib=lib), o)


def pin_packing_invariance(lib=None):
    rng = np.random.default_rng(17)
    q, k, v, cu, spans = _random_case(rng, [12, 30, 7], 4, 2, 8, 1)
    full = oracle.prefill(q, k, v, cu, window=5, spans=spans, lib=lib)
    for b in range(3):
        a, e = cu[b], cu[b + 1]
        local = [(s - a, t - a) for s, t in spans if a <= s < e]
        solo = oracle.prefill(q[a:e], k[a:e], v[a:e], [0, e - a], window=5,
                              spans=local or None, lib=lib)
        assert np.array_equal(solo, full[a:e])


def pin_row_subset(lib=None):
    rng = np.random.default_rng(19)
    q, k, v, cu, spans = _random_case(rng, [20, 33], 4, 2, 8, 1)
    full, fl = oracle.prefill(q, k, v, cu, window=9, spans=spans, want_lse=True, lib=lib)
    rows = np.array([[0, 0], [52, 3], [20, 1], [33, 2]])
    sub, sl = oracle.prefill(q, k, v, cu, window=9, spans=spans, rows=rows, want_lse=True, lib=lib)
    for n, (t, h) in enumerate(rows):
        assert np.array_equal(sub[n], full[t, h])
        assert sl[n] == fl[t, h]


def _decode_inputs(rng, lengths, hq, hkv, d, bs, spare=5):
    nblk = [(L + bs - 1) // bs for L in lengths]
    nb = sum(nblk) + spare
    kc = rng.standard_normal((nb, bs, hkv, d))
    vc = rng.standard_normal((nb, bs, hkv, d))
    perm = rng.permutation(nb)
    bt = np.zeros((len(lengths), max(nblk)), np.int32)
    c = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[c:c + n]
        c += n
    q = rng.standard_normal((len(lengths), hq, d))
    return q, kc, vc, bt, np.array(lengths, np.int32)


def pin_decode(lib=None):
    """Decode equals brute force over the gathered cache, equals the last
    prefill row of the same sequence, and ignores physical block placement."""
    rng = np.random.default_rng(23)
    lengths = [1, 16, 17, 50]
    q, kc, vc, bt, sl = _decode_inputs(rng, lengths, 4, 2, 8, 16)
    for w in (-1, 1, 10):
        o = oracle.decode(q, kc, vc, bt, sl, window=w, lib=lib)
        assert np.abs(o - bruteforce.decode(q, kc, vc, bt, sl, window=w)).max() <= 1e-12
        for b, L in enumerate(lengths):
            nb = (L + 15) // 16
            kk = kc[bt[b, :nb]].reshape(-1, 2, 8)[:L]
            vv = vc[bt[b, :nb]].reshape(-1, 2, 8)[:L]
            qq = np.zeros((L, 4, 8))
            qq[L - 1] = q[b]
            row = oracle.prefill(qq, kk, vv, [0, L], window=w, lib=lib)[L - 1]
            assert np.abs(row - o[b]).max() <= 1e-12
        # move every block to a new physical id
        nb_total = kc.shape[0]
        perm = rng.permutation(nb_total)
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[perm] = kc
        vc2[perm] = vc
        bt2 = perm[bt].astype(np.int32)
        assert np.array_equal(oracle.decode(q, kc2, vc2, bt2, sl, window=w, lib=lib), o)


# ------------------------------------------------------------------ backward
def _loss(q, k, v, dout, cu, window, spans, lib):
    """L = sum(dout * O) through the forward oracle (fp64 inputs, scale 0.4)."""
    o = oracle.prefill(q, k, v, cu, window=window, scale=0.4, spans=spans, lib=lib)
    return float((dout * o).sum())


def pin_backward_finite_differences(lib=None):
    """Every entry of dq, dk, dv equals the central difference of
    L = sum(dout * O) through the forward oracle (step 1e-5, fp64): the
    gradient is fixed by the forward definition alone."""
    rng = np.random.default_rng(41)
    cu = [0, 5, 8]
    spans = [[1, 4]]
    q = rng.standard_normal((8, 2, 6))
    k = rng.standard_normal((8, 1, 6))
    v = rng.standard_normal((8, 1, 6))
    dout = rng.standard_normal((8, 2, 6))
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, cu, window=3, scale=0.4, spans=spans,
                                         lib=lib)
    eps = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            up = _loss(q, k, v, dout, cu, 3, spans, lib)
            x[idx] = old - eps
            dn = _loss(q, k, v, dout, cu, 3, spans, lib)
            x[idx] = old
            num[idx] = (up - dn) / (2 * eps)
        assert np.abs(num - g).max() <= 1e-7, np.abs(num - g).max()


def pin_backward_single_key(lib=None):
    """Window 1: every row sees only its own key, so p = 1 whatever the
    scores: dq = dk = 0 exactly and dv of key j = the sum over the group's
    query heads of dout at row j."""
    rng = np.random.default_rng(42)
    q = rng.standard_normal((9, 4, 5))
    k = rng.standard_normal((9, 2, 5))
    v = rng.standard_normal((9, 2, 5))
    dout = rng.standard_normal((9, 4, 5))
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, [0, 4, 9], window=1, lib=lib)
    assert not dq.any() and not dk.any()
    want = dout.reshape(9, 2, 2, 5).sum(axis=2)
    assert np.abs(dv - want).max() <= 1e-15


def pin_backward_gqa_is_mha_summed(lib=None):
    """GQA with G query heads per KV head equals multi-head attention with
    each K/V head repeated G times, the repeated heads' dk/dv summed."""
    rng = np.random.default_rng(43)
    cu = [0, 6, 11]
    q = rng.standard_normal((11, 4, 6))
    k = rng.standard_normal((11, 2, 6))
    v = rng.standard_normal((11, 2, 6))
    dout = rng.standard_normal((11, 4, 6))
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, cu, window=4, lib=lib)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.prefill_backward(q, kr, vr, dout, cu, window=4, lib=lib)
    assert np.abs(dq - dq2).max() <= 1e-12
    assert np.abs(dk - dk2.reshape(11, 2, 2, 6).sum(axis=2)).max() <= 1e-12
    assert np.abs(dv - dv2.reshape(11, 2, 2, 6).sum(axis=2)).max() <= 1e-12


# ------------------------------------------------------ stored input formats
# The GPU reads bf16 as given and every parity comparison feeds the oracle
# the same bf16 bit patterns ("RFC: Gemma-4-31B-it train/rollout
# consistency", section 4 item 5: inputs in their declared dtype; "Gated
# RMSNorm CUDA kernel for the GDN block", accuracy against FP64 on the exact
# stored inputs).  These pins fix the oracle's widening of those patterns.

def pin_backward_units(lib=None):
    """A list of (row, head) and (key, KV head) units: each listed entry of
    dq, dk, dv equals the central difference of L = sum(dout * O) through
    the forward oracle, and equals the same entry of the unlisted call."""
    rng = np.random.default_rng(44)
    cu = [0, 7, 13]
    spans = [[8, 11]]
    q = rng.standard_normal((13, 4, 5))
    k = rng.standard_normal((13, 2, 5))
    v = rng.standard_normal((13, 2, 5))
    dout = rng.standard_normal((13, 4, 5))
    dq_units = [(6, 3), (0, 0), (9, 1), (12, 2)]
    kv_units = [(2, 1), (8, 0), (12, 1), (0, 0)]
    dq, dk, dv = oracle.prefill_backward(q, k, v, dout, cu, window=4, scale=0.4, spans=spans,
                                         lib=lib, dq_units=dq_units, kv_units=kv_units)
    fq, fk, fv = oracle.prefill_backward(q, k, v, dout, cu, window=4, scale=0.4, spans=spans,
                                         lib=lib)
    assert np.array_equal(dq, np.stack([fq[t, h] for t, h in dq_units]))
    assert np.array_equal(dk, np.stack([fk[t, g] for t, g in kv_units]))
    assert np.array_equal(dv, np.stack([fv[t, g] for t, g in kv_units]))
    eps = 1e-5
    for x, units, g in ((q, dq_units, dq), (k, kv_units, dk), (v, kv_units, dv)):
        for u, (t, h) in enumerate(units):
            for c in range(x.shape[2]):
                old = x[t, h, c]
                x[t, h, c] = old + eps
                up = _loss(q, k, v, dout, cu, 4, spans, lib)
                x[t, h, c] = old - eps
                dn = _loss(q, k, v, dout, cu, 4, spans, lib)
                x[t, h, c] = old
                assert abs((up - dn) / (2 * eps) - g[u, c]) <= 1e-7


def _bf16_exact(bits):
    """Exact value of one bf16 pattern from its fields, in Fractions."""
    sign = -1 if bits >> 15 else 1
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 255
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(1, 2 ** 126)
    return sign * (1 + Fraction(f, 128)) * (Fraction(2) ** (e - 127))


_BF16_PATTERNS = [0x3F80, 0xBF80, 0x4040, 0x3FC0, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F,
                  0xFF7F, 0x0000, 0x8000, 0x3E2A, 0xC2F7, 0x4B00, 0x3380, 0x1234, 0x5555]


def pin_bf16_widening(lib=None):
    """One-key rows return V exactly, so bf16 V patterns (normal, subnormal,
    largest finite, signed zero) must come out as their exact values, and
    likewise through the paged decode read."""
    pats = np.array(_BF16_PATTERNS, np.uint16)
    n = len(pats)
    d = 4
    v = np.zeros((n, 1, d), np.uint16)
    for t in range(n):
        for c in range(d):
            v[t, 0, c] = pats[(t + c) % n]
    rng = np.random.default_rng(29)
    q = rng.integers(0x3C00, 0x4000, size=(n, 2, d)).astype(np.uint16)
    k = rng.integers(0x3C00, 0x4000, size=(n, 1, d)).astype(np.uint16)
    want = np.array([[float(_bf16_exact(int(v[t, 0, c]))) for c in range(d)] for t in range(n)])
    o = oracle.prefill(q, k, v, np.arange(n + 1), lib=lib)      # every sequence one token
    for h in range(2):
        assert np.array_equal(o[:, h, :], want)
    o = oracle.prefill(q, k, v, [0, n], window=1, lib=lib)      # window 1: own key only
    assert np.array_equal(o[:, 0, :], want)
    # decode: one-token contexts, cache block t holds token t
    kc = np.zeros((n, 16, 1, d), np.uint16)
    vc = np.zeros((n, 16, 1, d), np.uint16)
    kc[:, 0] = k
    vc[:, 0] = v
    bt = np.arange(n, dtype=np.int32)[:, None]
    o = oracle.decode(q, kc, vc, bt, np.ones(n, np.int32), lib=lib)
    assert np.array_equal(o[:, 1, :], want)


def _random_bf16(rng, shape):
    """bf16 patterns with random sign and fraction and exponents 2^-5 .. 2^2."""
    sign = rng.integers(0, 2, size=shape) << 15
    exp = rng.integers(122, 130, size=shape) << 7
    frac = rng.integers(0, 128, size=shape)
    return (sign | exp | frac).astype(np.uint16)


def pin_bruteforce_stored_formats(lib=None):
    """The oracle on bf16 patterns and on fp32 values equals the brute force,
    which decodes bf16 from its fields (prefill with windows, spans, GQA, and
    paged decode)."""
    rng = np.random.default_rng(31)
    for lengths, hq, hkv, d, w, nsp in (([9, 26, 3], 4, 2, 16, 5, 1), ([40], 8, 1, 8, -1, 2)):
        T = sum(lengths)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        _, _, _, _, spans = _random_case(rng, lengths, hq, hkv, d, nsp)
        for make in (lambda s: _random_bf16(rng, s),
                     lambda s: rng.standard_normal(s).astype(np.float32)):
            q, k, v = make((T, hq, d)), make((T, hkv, d)), make((T, hkv, d))
            o, lse = oracle.prefill(q, k, v, cu, window=w, spans=spans or None, want_lse=True,
                                    lib=lib)
            bo, bl = bruteforce.attention(q, k, v, cu, window=w, spans=spans)
            assert np.abs(o - bo).max() <= 1e-12, (q.dtype, lengths)
            assert np.abs(lse - bl).max() <= 1e-12, (q.dtype, lengths)
    lengths = [1, 16, 33]
    for make in (lambda s: _random_bf16(rng, s), lambda s: rng.standard_normal(s).astype(np.float32)):
        q, kc, vc, bt, sl = _decode_inputs(rng, lengths, 4, 2, 8, 16)
        q, kc, vc = make(q.shape), make(kc.shape), make(vc.shape)
        for w in (-1, 7):
            o = oracle.decode(q, kc, vc, bt, sl, window=w, lib=lib)
            assert np.abs(o - bruteforce.decode(q, kc, vc, bt, sl, window=w)).max() <= 1e-12





# ---------------------------------------------------------------------------
# The attention prologue (RMSNorm over the head dim, then RoPE), pinned by
# closed forms, invariants and a brute force written with complex numbers.

def _prologue_brute(x, pos, weight, eps, offset, R, F, theta):
    """numpy: the norm by mean/sqrt, the rotation as a complex product."""
    x = np.asarray(x, np.float64)
    if weight is not None:
        rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
        y = x / rms * (offset + np.asarray(weight, np.float64))
    else:
        y = x.copy()
    h = R // 2
    if h:
        freq = theta ** (-2.0 * np.arange(h) / F)
        rot = np.exp(1j * np.asarray(pos, np.float64)[:, None] * freq[None, :])  # [T, h]
        z = (y[..., :h] + 1j * y[..., h:R]) * rot[:, None, :]
        y[..., :h] = z.real
        y[..., h:R] = z.imag
    return y


def pin_prologue_hand_values(lib=None):
    """Angles written out by hand from the definition pos * theta^(-2i/F):
    theta = 10000, R = 4: pair 0 turns by pos, pair 1 by pos * 10000^(-2/F),
    i.e. pos / 100 for F = 4 and pos / 10 for F = 8 (proportional)."""
    e = np.eye(4)[:, None, :]                              # rows e0 .. e3, one head
    for F, step1 in ((4, 0.01), (8, 0.1)):
        for pos in (1, 3):
            y = oracle.qk_prologue(e, [pos] * 4, rotary_dims=4, freq_dims=F, theta=10000.0,
                                   lib=lib)[:, 0, :]
            a0, a1 = pos * 1.0, pos * step1
            want = np.array([[math.cos(a0), 0, math.sin(a0), 0],
                             [0, math.cos(a1), 0, math.sin(a1)],
                             [-math.sin(a0), 0, math.cos(a0), 0],
                             [0, -math.sin(a1), 0, math.cos(a1)]])
            assert np.abs(y - want).max() <= 1e-13, (F, pos)
    # dims past the rotary width pass through untouched
    x = np.arange(1.0, 9.0)[None, None, :]
    y = oracle.qk_prologue(x, [5], rotary_dims=4, freq_dims=8, lib=lib)
    assert np.array_equal(y[0, 0, 4:], x[0, 0, 4:])


def pin_prologue_norm_closed_form(lib=None):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 3, 16)) * rng.uniform(0.1, 10.0, (5, 3, 1))
    ones = np.ones(16)
    y = oracle.qk_prologue(x, np.zeros(5), weight=ones, eps=0.0, lib=lib)
    assert np.abs(np.mean(y * y, axis=-1) - 1.0).max() <= 1e-12   # unit RMS
    y2 = oracle.qk_prologue(7.5 * x, np.zeros(5), weight=ones, eps=0.0, lib=lib)
    assert np.abs(y2 - y).max() <= 1e-12                           # scale-free
    eps = 0.3
    ye = oracle.qk_prologue(x, np.zeros(5), weight=ones, eps=eps, lib=lib)
    ms = np.mean(x * x, axis=-1)
    assert np.abs(np.mean(ye * ye, axis=-1) - ms / (ms + eps)).max() <= 1e-12
    w = rng.standard_normal(16)
    a = oracle.qk_prologue(x, np.zeros(5), weight=w, eps=eps, offset=1.0, lib=lib)
    b = oracle.qk_prologue(x, np.zeros(5), weight=w + 1.0, eps=eps, offset=0.0, lib=lib)
    assert np.abs(a - b).max() <= 1e-12                            # offset adds to the weight
    c = oracle.qk_prologue(x, np.zeros(5), weight=2.0 * w, eps=eps, lib=lib)
    d = oracle.qk_prologue(x, np.zeros(5), weight=w, eps=eps, lib=lib)
    assert np.abs(c - 2.0 * d).max() <= 1e-12                      # linear in the weight


def pin_prologue_rope_invariants(lib=None):
    rng = np.random.default_rng(43)
    T, H, D, R = 6, 2, 16, 12
    q = rng.standard_normal((T, H, D))
    k = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 40000, T)
    for F in (R, D):
        # position 0 is the identity
        assert np.abs(oracle.qk_prologue(q, np.zeros(T), rotary_dims=R, freq_dims=F, lib=lib)
                      - q).max() == 0
        y = oracle.qk_prologue(q, pos, rotary_dims=R, freq_dims=F, lib=lib)
        # each turned pair keeps its length; other dims are unchanged
        h = R // 2
        n0 = q[..., :h] ** 2 + q[..., h:R] ** 2
        n1 = y[..., :h] ** 2 + y[..., h:R] ** 2
        assert np.abs(n1 - n0).max() <= 1e-9
        assert np.array_equal(y[..., R:], q[..., R:])
        # turning by a then by b is turning by a + b
        a, b = rng.integers(0, 3000, T), rng.integers(0, 3000, T)
        yab = oracle.qk_prologue(oracle.qk_prologue(q, a, rotary_dims=R, freq_dims=F, lib=lib),
                                 b, rotary_dims=R, freq_dims=F, lib=lib)
        assert np.abs(yab - oracle.qk_prologue(q, a + b, rotary_dims=R, freq_dims=F,
                                               lib=lib)).max() <= 1e-9
        # scores depend on the relative position only
        m, n, s = 1234, 77, 5000
        qm = oracle.qk_prologue(q[:1], [m], rotary_dims=R, freq_dims=F, lib=lib)
        kn = oracle.qk_prologue(k[:1], [n], rotary_dims=R, freq_dims=F, lib=lib)
        qs = oracle.qk_prologue(q[:1], [m + s], rotary_dims=R, freq_dims=F, lib=lib)
        ks = oracle.qk_prologue(k[:1], [n + s], rotary_dims=R, freq_dims=F, lib=lib)
        assert abs(np.sum(qm * kn) - np.sum(qs * ks)) <= 1e-9


def pin_prologue_bruteforce(lib=None):
    rng = np.random.default_rng(47)
    T, H = 7, 3
    pos = rng.integers(0, 32768, T)
    for D, R, F in ((64, 64, 64), (32, 8, 32), (32, 16, 16), (16, 0, 16)):
        for make in (lambda s: rng.standard_normal(s),
                     lambda s: rng.standard_normal(s).astype(np.float32),
                     lambda s: _random_bf16(rng, s)):
            x = make((T, H, D))
            w = make((D,))
            xf = bruteforce._f64(x)
            wf = bruteforce._f64(w)
            for weight, eps, off in ((w, 1e-6, 0.0), (w, 0.25, 1.0), (None, 0.0, 0.0)):
                y = oracle.qk_prologue(x, pos, weight=weight, eps=eps, offset=off, rotary_dims=R,
                                       freq_dims=F, theta=10000.0 if R else 1.0, lib=lib)
                want = _prologue_brute(xf, pos, None if weight is None else wf, eps, off, R, F,
                                       10000.0)
                assert np.abs(y - want).max() <= 1e-9 * max(1.0, np.abs(want).max()), (D, R, F)


ALL_PINS = [pin_golden, pin_bruteforce, pin_rows_sum_to_one,
            pin_window_covering_sequence_is_global, pin_one_token_returns_v,
            pin_zero_query_is_mean, pin_dominant_key, pin_gqa_reduces_to_mha,
            pin_packing_invariance, pin_row_subset, pin_decode,
            pin_backward_finite_differences, pin_backward_single_key,
            pin_backward_gqa_is_mha_summed, pin_backward_units, pin_bf16_widening,
            pin_bruteforce_stored_formats, pin_prologue_hand_values,
            pin_prologue_norm_closed_form, pin_prologue_rope_invariants,
            pin_prologue_bruteforce]

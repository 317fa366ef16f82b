"""Dense brute-force attention in numpy, for pinning the oracle on tiny inputs.

This is a second, independent rendering of the same definition as the C
oracle: the mask is built as a whole L x L boolean matrix from vectorised
comparisons and span-membership ids, the scores come from one fp64 matrix
product per head, and softmax is taken over whole rows.  It shares no code
with the oracle or with the GPU library.
"""
from __future__ import annotations

import numpy as np


def bf16_value(bits):
    """Value of bf16 bit patterns (uint16) in fp64, from the format's fields:
    sign bit 15, 8-bit biased exponent (bias 127), 7-bit fraction; exponent 0
    is subnormal (fraction/128 * 2^-126), exponent 255 is inf/NaN.  Written
    from the field definition, not by reinterpreting the upper half of an
    fp32 word, so it is an independent rendering of the widening."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    normal = np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int32))
    sub = np.ldexp(f / 128.0, -126)
    special = np.where(f == 0, np.inf, np.nan)
    val = np.where(e == 0, sub, np.where(e == 255, special, normal))
    return sign * val


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_value(a)
    return a.astype(np.float64)


def dense_mask(length, window, spans=()):
    """allowed[i, j] for one sequence; spans are sequence-relative [s, e)."""
    i = np.arange(length)[:, None]
    j = np.arange(length)[None, :]
    causal = j <= i
    if window is not None and window >= 0:
        causal &= (i - j) < window
    sid = np.full(length, -1)
    for n, (s, e) in enumerate(spans):
        sid[s:e] = n
    same_span = (sid[:, None] == sid[None, :]) & (sid[:, None] >= 0)
    return causal | same_span


def attention(q, k, v, cu_seqlens, window=-1, scale=None, spans=()):
    """q [T,Hq,D], k/v [T,Hkv,D] -> (o [T,Hq,D], lse [T,Hq]) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.zeros((T, hq, d))
    lse = np.zeros((T, hq))
    for b in range(len(cu_seqlens) - 1):
        a, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        local = [(s - a, t - a) for s, t in spans if a <= s < e]
        mask = dense_mask(e - a, window, local)
        for h in range(hq):
            s = scale * (q[a:e, h, :] @ k[a:e, h // g, :].T)
            s = np.where(mask, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            w = np.exp(s - mx)
            z = w.sum(axis=1, keepdims=True)
            o[a:e, h, :] = (w / z) @ v[a:e, h // g, :]
            lse[a:e, h] = (mx + np.log(z))[:, 0]
    return o, lse


def decode(q, k_cache, v_cache, block_table, seq_lens, window=-1, scale=None):
    """Gather each sequence's cache into a dense array, then attend the last row."""
    q = _f64(q)
    kc, vc = _f64(k_cache), _f64(v_cache)
    B, hq, d = q.shape
    bs, hkv = kc.shape[1], kc.shape[2]
    g = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.zeros((B, hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        nb = (L + bs - 1) // bs
        kk = kc[block_table[b, :nb]].reshape(nb * bs, hkv, d)[:L]
        vv = vc[block_table[b, :nb]].reshape(nb * bs, hkv, d)[:L]
        keep = np.ones(L, bool)
        if window is not None and window >= 0:
            keep = (L - 1 - np.arange(L)) < window
        for h in range(hq):
            s = scale * (kk[keep, h // g, :] @ q[b, h, :])
            w = np.exp(s - s.max())
            o[b, h] = (w / w.sum()) @ vv[keep, h // g, :]
    return o

"""Seeded synthetic inputs for the attention library, its tests and its benchmark.

This module generates inputs only; it holds none of the attention arithmetic.
Both the GPU path and the CPU oracle read what it produces, bit for bit.

Recipe (every draw is numpy PCG64, ``np.random.default_rng([seed, index])``):

* Each sequence's Q, K, V are drawn from their own stream ``[seed, 1000 + i]``
  (sequence i of the case), so a sequence holds the same bits whether it runs
  alone, packed with others, or at another batch position.
* Values are N(0, 1) * std in fp32, then rounded to bf16 (round to nearest
  even), stored as uint16 bit patterns.
* Lengths, batch orders, span positions and physical KV-block placement come
  from the case stream ``[seed, 0]``.

The workloads mirror the hybrid decoder the pages describe: sliding-window
layers with head dim 256 and global layers with head dim 512 and only 4 KV
heads ("RFC: Gemma-4-31B-it train/rollout consistency", sections 6 and 7),
packed variable-length prefill, bidirectional soft-token spans (section 1,
Phase B) and single-token decode over a paged KV cache ("Vime ROCm Attention
operator ablation", "Prerequisites").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NO_WINDOW = -1


# --------------------------------------------------------------------------
# bf16 bit patterns
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN kept quiet."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


# --------------------------------------------------------------------------
# prefill cases
# --------------------------------------------------------------------------
@dataclass
class Sequence:
    """One sequence's tensors (bf16 bits) and its bidirectional spans."""
    q: np.ndarray            # [L, Hq, D] uint16
    k: np.ndarray            # [L, Hkv, D] uint16
    v: np.ndarray            # [L, Hkv, D] uint16
    spans: list = field(default_factory=list)   # sequence-relative [start, end)

    @property
    def length(self) -> int:
        return self.q.shape[0]


@dataclass
class PrefillCase:
    seqs: list               # list[Sequence]
    hq: int
    hkv: int
    d: int
    window: int              # NO_WINDOW = global causal
    scale: float
    name: str = ""
    q32: list = None         # optional fp32 originals (tiny case)

    def pack(self, order=None):
        """Pack the sequences in ``order`` (default identity).

        Returns q, k, v (uint16 [T, H, D]), cu_seqlens (int32 [B+1]) and spans
        (int32 [S, 2], packed coordinates, ascending).
        """
        order = list(range(len(self.seqs))) if order is None else list(order)
        lens = [self.seqs[i].length for i in order]
        cu = np.zeros(len(order) + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        T = int(cu[-1])
        q = np.empty((T, self.hq, self.d), np.uint16)
        k = np.empty((T, self.hkv, self.d), np.uint16)
        v = np.empty((T, self.hkv, self.d), np.uint16)
        spans = []
        for pos, i in enumerate(order):
            s = self.seqs[i]
            a, b = int(cu[pos]), int(cu[pos + 1])
            q[a:b], k[a:b], v[a:b] = s.q, s.k, s.v
            spans += [(a + lo, a + hi) for lo, hi in s.spans]
        sp = np.array(spans, np.int32).reshape(-1, 2)
        return q, k, v, cu, sp

    def max_seqlen(self) -> int:
        return max((s.length for s in self.seqs), default=0)


def _seq(seed, idx, length, hq, hkv, d, std, spans=()):
    rng = np.random.default_rng([seed, 1000 + idx])
    return Sequence(q=_normal_bf16(rng, (length, hq, d), std),
                    k=_normal_bf16(rng, (length, hkv, d), std),
                    v=_normal_bf16(rng, (length, hkv, d), std),
                    spans=list(spans))


def prefill_case(seed, lengths, hq, hkv, d, window, std=0.5, spans=None, name=""):
    """Generic prefill case: one sequence per entry of ``lengths``.

    ``spans``: optional list (one entry per sequence) of sequence-relative
    [start, end) span lists.
    """
    seqs = [_seq(seed, i, int(L), hq, hkv, d, std, spans[i] if spans else ())
            for i, L in enumerate(lengths)]
    return PrefillCase(seqs, hq, hkv, d, window, 1.0 / float(np.sqrt(d)), name)


def upstream_grad(seed, shape, std=0.5) -> np.ndarray:
    """Seeded upstream gradient dL/dO for the backward (bf16 bits, normal)."""
    return _normal_bf16(np.random.default_rng([seed, 7777]), shape, std)


def tiny_case(seed=1, window=32):
    """One sequence of 128 tokens, 4 query / 2 KV heads, head dim 64, fp32
    N(0,1) inputs; the kernel consumes their bf16 rounding."""
    rng = np.random.default_rng([seed, 1000])
    L, hq, hkv, d = 128, 4, 2, 64
    q = rng.standard_normal((L, hq, d), dtype=np.float32)
    k = rng.standard_normal((L, hkv, d), dtype=np.float32)
    v = rng.standard_normal((L, hkv, d), dtype=np.float32)
    seq = Sequence(q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v))
    case = PrefillCase([seq], hq, hkv, d, window, 1.0 / 8.0, "tiny")
    case.q32 = [(q, k, v)]
    return case


def sliding_lengths(seed=2, n=8, lo=512, hi=4096):
    rng = np.random.default_rng([seed, 0])
    return [int(x) for x in rng.integers(lo, hi, size=n, endpoint=True)]


def sliding_case(seed=2, n=8, lo=512, hi=4096, hq=32, hkv=16, d=256, window=1024, std=0.5):
    """Sliding-window layer: packed varlen batch, lengths U[lo, hi]."""
    return prefill_case(seed, sliding_lengths(seed, n, lo, hi), hq, hkv, d, window, std,
                        name="sliding")


def global_case(seed=3, lengths=(2048, 4096, 6144, 8192), hq=32, hkv=4, d=512, std=0.5):
    """Global (full causal) layer over a packed varlen batch."""
    return prefill_case(seed, lengths, hq, hkv, d, NO_WINDOW, std, name="global")


def batch_orders(seed, n, count=2):
    """Identity, reversed, then ``count`` seeded permutations of range(n)."""
    rng = np.random.default_rng([seed, 0, 7])
    orders = [list(range(n)), list(range(n))[::-1]]
    for _ in range(count):
        orders.append([int(x) for x in rng.permutation(n)])
    return orders


def hybrid_spans(seed, n, length=4096, span=256):
    """Two contiguous ``span``-token bidirectional spans per sequence: one
    starting in [0, length/2 - span], one in [length/2, length - span]."""
    rng = np.random.default_rng([seed, 0])
    out = []
    half = length // 2
    for _ in range(n):
        s1 = int(rng.integers(0, half - span, endpoint=True))
        s2 = int(rng.integers(half, length - span, endpoint=True))
        out.append([(s1, s1 + span), (s2, s2 + span)])
    return out


HYBRID_LAYERS = (
    # (hq, hkv, d, window)
    (32, 16, 256, 1024),
    (32, 16, 256, 1024),
    (32, 16, 256, 1024),
    (32, 16, 256, 1024),
    (32, 16, 256, 1024),
    (32, 4, 512, NO_WINDOW),
)


def hybrid_case(seed=5, layer=0, n=4, length=4096, span=256, std=0.5, layers=HYBRID_LAYERS):
    """One layer of the hybrid pattern (5 sliding + 1 global) over ``n``
    sequences of ``length`` tokens with two bidirectional spans each.
    Each layer draws independent Q/K/V (seed stream offset by the layer)."""
    hq, hkv, d, w = layers[layer]
    spans = hybrid_spans(seed, n, length, span)
    return prefill_case(seed * 100 + layer, [length] * n, hq, hkv, d, w, std, spans,
                        name=f"hybrid-layer{layer}")


# --------------------------------------------------------------------------
# paged decode cases
# --------------------------------------------------------------------------
@dataclass
class DecodeCase:
    q: np.ndarray            # [B, Hq, D] uint16
    k_cache: np.ndarray      # [NB, BS, Hkv, D] uint16
    v_cache: np.ndarray
    block_table: np.ndarray  # [B, MB] int32
    seq_lens: np.ndarray     # [B] int32
    hq: int
    hkv: int
    d: int
    block_size: int
    window: int
    scale: float


def decode_lengths(seed=4, n=64, lo=1024, hi=32768):
    rng = np.random.default_rng([seed, 0])
    return [int(x) for x in rng.integers(lo, hi, size=n, endpoint=True)]


def decode_case(seed=4, lengths=None, batch=64, hq=32, hkv=4, d=512, block_size=16,
                window=NO_WINDOW, std=0.5, spare_blocks=64, placement_seed=0,
                poison=True, order=None, max_blocks=None):
    """Paged decode batch.  Sequence i's K/V (positions 0..L-1) and its query
    come from stream [seed, 1000 + i] regardless of batch size or position.
    Physical blocks are a seeded permutation (``placement_seed``); unused
    slots, spare blocks and table padding are NaN poison when ``poison``."""
    if lengths is None:
        lengths = decode_lengths(seed, batch)
    lengths = list(lengths)[:batch]
    order = list(range(len(lengths))) if order is None else list(order)
    nblk = [(L + block_size - 1) // block_size for L in lengths]
    total_blocks = sum(nblk) + spare_blocks
    mb = max(nblk) if max_blocks is None else max_blocks
    fill = BF16_NAN if poison else np.uint16(0)
    kc = np.full((total_blocks, block_size, hkv, d), fill, np.uint16)
    vc = np.full((total_blocks, block_size, hkv, d), fill, np.uint16)
    prng = np.random.default_rng([seed, 0, 11, placement_seed])
    phys = prng.permutation(total_blocks).astype(np.int32)
    table_pad = np.int32(total_blocks + 7) if poison else np.int32(0)
    bt = np.full((len(order), mb), table_pad, np.int32)
    q = np.empty((len(order), hq, d), np.uint16)
    sl = np.empty(len(order), np.int32)
    cursor = 0
    first_block = []
    for i in range(len(lengths)):
        first_block.append(cursor)
        cursor += nblk[i]
    for pos, i in enumerate(order):
        L = lengths[i]
        rng = np.random.default_rng([seed, 1000 + i])
        q[pos] = _normal_bf16(rng, (hq, d), std)
        kk = _normal_bf16(rng, (L, hkv, d), std)
        vv = _normal_bf16(rng, (L, hkv, d), std)
        ids = phys[first_block[i]:first_block[i] + nblk[i]]
        bt[pos, :nblk[i]] = ids
        for blk in range(nblk[i]):
            a, b = blk * block_size, min(L, (blk + 1) * block_size)
            kc[ids[blk], :b - a] = kk[a:b]
            vc[ids[blk], :b - a] = vv[a:b]
        sl[pos] = L
    return DecodeCase(q, kc, vc, bt, sl, hq, hkv, d, block_size, window,
                      1.0 / float(np.sqrt(d)))


# --------------------------------------------------------------------------
# chunked prefill over a paged KV cache
# --------------------------------------------------------------------------
@dataclass
class PagedChunks:
    """Query chunks of the sequences of a PrefillCase, their keys in a paged
    cache.  Batch entry c is chunk (seq[c], start[c], end[c]): query positions
    [start, end) of sequence seq[c], whose keys [0, end) are in the cache."""
    q: np.ndarray            # [T, Hq, D] uint16, the chunks' query rows, packed
    k_cache: np.ndarray      # [NB, 16, Hkv, D] uint16
    v_cache: np.ndarray
    block_table: np.ndarray  # [B, MB] int32 (the row of the chunk's sequence)
    cu_seqlens: np.ndarray   # [B+1] int32, packed query-row ranges
    q_start: np.ndarray      # [B] int32
    seq: list
    start: list
    end: list
    block_size: int = 16

    def max_query_len(self) -> int:
        return max((e - a for a, e in zip(self.start, self.end)), default=0)

    def max_context_len(self) -> int:
        return max(self.end, default=0)


def chunk_bounds(seed, length, n_cuts):
    """Sorted chunk boundaries 0 = c0 < ... < L of one sequence: ``n_cuts``
    random interior cuts from stream [seed, 0, 21, length], plus a cut at
    L - 1 (the last chunk is one token) when L > 1."""
    rng = np.random.default_rng([seed, 0, 21, length])
    cuts = set(int(x) for x in rng.integers(1, max(length, 2), size=n_cuts)) if length > 1 else set()
    if length > 1:
        cuts.add(length - 1)
    return [0] + sorted(c for c in cuts if 0 < c < length) + [length]


def paged_chunks(case, chunks, block_size=16, spare_blocks=8, placement_seed=0, poison=True,
                 max_blocks=None):
    """Lay every sequence of ``case`` into a paged cache (seeded physical
    block permutation from stream [0, 11, placement_seed]) and build the batch
    of ``chunks``, a list of (sequence index, start, end).  Unused slots,
    spare blocks and table padding are NaN / out-of-range poison when
    ``poison``."""
    nseq = len(case.seqs)
    lens = [s.length for s in case.seqs]
    nblk = [(L + block_size - 1) // block_size for L in lens]
    total = sum(nblk) + spare_blocks
    mb = max(max(nblk), 1) if max_blocks is None else max_blocks
    fill = BF16_NAN if poison else np.uint16(0)
    kc = np.full((total, block_size, case.hkv, case.d), fill, np.uint16)
    vc = np.full((total, block_size, case.hkv, case.d), fill, np.uint16)
    phys = np.random.default_rng([0, 11, placement_seed]).permutation(total).astype(np.int32)
    rows = np.full((nseq, mb), total + 7 if poison else 0, np.int32)
    cursor = 0
    for i, s in enumerate(case.seqs):
        ids = phys[cursor:cursor + nblk[i]]
        cursor += nblk[i]
        rows[i, :nblk[i]] = ids
        for j, blk in enumerate(ids):
            a, b = j * block_size, min(lens[i], (j + 1) * block_size)
            kc[blk, :b - a] = s.k[a:b]
            vc[blk, :b - a] = s.v[a:b]
    seq = [c[0] for c in chunks]
    start = [int(c[1]) for c in chunks]
    end = [int(c[2]) for c in chunks]
    cu = np.zeros(len(chunks) + 1, np.int32)
    cu[1:] = np.cumsum([e - a for a, e in zip(start, end)])
    q = np.empty((int(cu[-1]), case.hq, case.d), np.uint16)
    for c, (i, a, e) in enumerate(zip(seq, start, end)):
        q[cu[c]:cu[c + 1]] = case.seqs[i].q[a:e]
    bt = rows[seq] if chunks else np.zeros((0, mb), np.int32)
    return PagedChunks(q, kc, vc, np.ascontiguousarray(bt), cu, np.array(start, np.int32), seq,
                       start, end, block_size)


# --------------------------------------------------------------------------
# device-side generation for the full-size paged decode workload
# --------------------------------------------------------------------------
def decode_case_device(seed=4, lengths=None, batch=64, hq=32, hkv=4, d=512, block_size=16,
                       std=0.5, spare_blocks=64, placement_seed=0, poison=True, device="cuda"):
    """The paged decode batch built directly in GPU memory (torch).

    Values come from torch's device generator seeded per sequence
    (``seed * 1_000_003 + i``), so sequence i holds the same bits at any batch
    size; they are NOT the same bits as ``decode_case`` (numpy).  Lengths and
    physical block placement use the same numpy streams as ``decode_case``.
    Returns a dict of device tensors plus the host block table and lengths.
    """
    import torch
    if lengths is None:
        lengths = decode_lengths(seed, batch)
    lengths = list(lengths)[:batch]
    nblk = [(L + block_size - 1) // block_size for L in lengths]
    total_blocks = sum(nblk) + spare_blocks
    mb = max(nblk)
    fill = float("nan") if poison else 0.0
    kc = torch.full((total_blocks, block_size, hkv, d), fill, dtype=torch.bfloat16, device=device)
    vc = torch.full((total_blocks, block_size, hkv, d), fill, dtype=torch.bfloat16, device=device)
    prng = np.random.default_rng([seed, 0, 11, placement_seed])
    phys = prng.permutation(total_blocks).astype(np.int32)
    bt = np.full((len(lengths), mb), total_blocks + 7 if poison else 0, np.int32)
    q = torch.empty((len(lengths), hq, d), dtype=torch.bfloat16, device=device)
    cursor = 0
    for i, L in enumerate(lengths):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1_000_003 + i)
        q[i] = (torch.randn((hq, d), generator=g, device=device) * std).to(torch.bfloat16)
        ids = phys[cursor:cursor + nblk[i]]
        cursor += nblk[i]
        bt[i, :nblk[i]] = ids
        pad = nblk[i] * block_size
        kk = torch.full((pad, hkv, d), fill, dtype=torch.bfloat16, device=device)
        vv = torch.full((pad, hkv, d), fill, dtype=torch.bfloat16, device=device)
        kk[:L] = (torch.randn((L, hkv, d), generator=g, device=device) * std).to(torch.bfloat16)
        vv[:L] = (torch.randn((L, hkv, d), generator=g, device=device) * std).to(torch.bfloat16)
        idx = torch.from_numpy(ids.astype(np.int64)).to(device)
        kc.index_copy_(0, idx, kk.view(nblk[i], block_size, hkv, d))
        vc.index_copy_(0, idx, vv.view(nblk[i], block_size, hkv, d))
    return {"q": q, "k_cache": kc, "v_cache": vc, "block_table": bt,
            "seq_lens": np.array(lengths, np.int32), "hq": hq, "hkv": hkv, "d": d,
            "block_size": block_size, "scale": 1.0 / float(np.sqrt(d))}


def prefill_case_device(seed, lengths, hq, hkv, d, window, std=0.5, spans=None, order=None,
                        device="cuda"):
    """A packed prefill batch built directly in GPU memory (torch).

    Sequence i draws from torch's device generator seeded with
    ``seed * 1_000_003 + i``, so it holds the same bits in any batch and at
    any position (not the same bits as ``prefill_case``).  Returns a dict with
    device tensors q, k, v, cu_seqlens (int32) and spans (int32 [S, 2] or
    None), plus host copies of cu_seqlens and spans.
    """
    import torch
    lengths = [int(L) for L in lengths]
    order = list(range(len(lengths))) if order is None else list(order)
    qs, ks, vs, sp = [], [], [], []
    cu = np.zeros(len(order) + 1, np.int32)
    for pos, i in enumerate(order):
        L = lengths[i]
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1_000_003 + i)
        qs.append((torch.randn((L, hq, d), generator=g, device=device) * std).to(torch.bfloat16))
        ks.append((torch.randn((L, hkv, d), generator=g, device=device) * std).to(torch.bfloat16))
        vs.append((torch.randn((L, hkv, d), generator=g, device=device) * std).to(torch.bfloat16))
        cu[pos + 1] = cu[pos] + L
        if spans:
            sp += [(int(cu[pos]) + a, int(cu[pos]) + b) for a, b in spans[i]]
    spans_np = np.array(sp, np.int32).reshape(-1, 2)
    return {"q": torch.cat(qs), "k": torch.cat(ks), "v": torch.cat(vs),
            "cu_seqlens": torch.from_numpy(cu).to(device), "cu_host": cu,
            "spans": torch.from_numpy(spans_np).to(device) if len(sp) else None,
            "spans_host": spans_np, "max_seqlen": max(lengths) if lengths else 0,
            "hq": hq, "hkv": hkv, "d": d, "window": window, "scale": 1.0 / float(np.sqrt(d)),
            "lengths": [lengths[i] for i in order]}


# --------------------------------------------------------------------------
# prologue cases (RMSNorm + RoPE on Q and K before attention)
# --------------------------------------------------------------------------
# Prologue readings used by the tests and the benchmark (the pages fix none of
# them): eps, RoPE base, and the rotary width of each layer type (sliding:
# every dim; global: a quarter of the dims at the frequencies of a full RoPE).
PROLOGUE_EPS = 1e-6
PROLOGUE_THETA = {"sliding": 10000.0, "global": 1000000.0}


def prologue_rotary(kind: str, d: int):
    """(rotary_dims, freq_dims) of a layer type: full RoPE on sliding layers,
    proportional p-RoPE (p = 1/4, frequencies over the whole head dim) on
    global ones."""
    return (d, d) if kind == "sliding" else (d // 4, d)


@dataclass
class PrologueCase:
    q: np.ndarray          # [T, Hq, D] uint16 bf16 bits
    k: np.ndarray          # [T, Hkv, D] uint16 bf16 bits
    positions: np.ndarray  # [T] int32
    q_weight: np.ndarray   # [D] float32
    k_weight: np.ndarray   # [D] float32


def prologue_case(seed, lengths, hq, hkv, d, std=1.0, weight_std=0.1, start=None):
    """Packed sequences: token t of sequence i sits at position (start_i + t);
    Q, K ~ N(0,1)*std per sequence stream (as in prefill cases), weights ~
    N(0, weight_std^2) from the case stream.  ``start`` defaults to 0 for
    every sequence (a prefill)."""
    rng = np.random.default_rng([seed, 0])
    qs, ks, ps = [], [], []
    for i, L in enumerate(lengths):
        r = np.random.default_rng([seed, 1000 + i])
        qs.append(_normal_bf16(r, (L, hq, d), std))
        ks.append(_normal_bf16(r, (L, hkv, d), std))
        s0 = 0 if start is None else int(start[i])
        ps.append(np.arange(s0, s0 + L, dtype=np.int32))
    qw = (rng.standard_normal(d) * weight_std).astype(np.float32)
    kw = (rng.standard_normal(d) * weight_std).astype(np.float32)
    cat = lambda a, shp: np.concatenate(a) if a else np.zeros(shp, np.uint16)
    return PrologueCase(cat(qs, (0, hq, d)), cat(ks, (0, hkv, d)),
                        np.concatenate(ps) if ps else np.zeros(0, np.int32), qw, kw)

"""Chunked prefill over a paged KV cache on the GPU (attn_prefill_paged).

A query chunk attends to its sequence's cached prefix plus itself, reading
the keys in place through the block table.  Checked here: parity with the
fp64 oracle (each query row computed by the oracle's paged decode with the
context ending at that row, so the oracle reads the same cache through the
same table); every chunk row bitwise equal to the row of the same position
from the unchunked varlen prefill, whatever the chunk boundaries, batch
order, grouping into calls or grid bounds; single-token chunks (a decode
step) equal to the prefill row bytes; nothing outside the attended blocks
read.

Sources: a row is invariant to chunking and unrelated rows ("RFC:
Gemma-4-31B-it train/rollout consistency", section 4, item 6); strict calls
consume the paged KV cache directly ("Vime ROCm Attention operator
ablation", "Prerequisites"); the train/rollout goal of identical attention
bytes (same RFC, section 1)."""
import zlib

import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import bf16_dev, bits, f64, gate, i32_dev, run_case

pytestmark = pytest.mark.gpu

CASES = [
    # (name, lengths, hq, hkv, d, window)
    ("d64-g2-w40", [300, 77, 1], 4, 2, 64, 40),
    ("d64-g8-global", [260, 33], 8, 1, 64, synth.NO_WINDOW),
    ("d256-g2-w128", [513, 300, 37], 32, 16, 256, 128),
    ("d256-g4-global", [257, 100], 16, 4, 256, synth.NO_WINDOW),
    ("d256-g1-w64", [200], 8, 8, 256, 64),
    ("d512-g8-global", [600, 130], 32, 4, 512, synth.NO_WINDOW),
    ("d512-g1-w40", [150, 31], 4, 4, 512, 40),
]


def seed_of(name):
    return zlib.crc32(name.encode()) % 1000


def make_case(name, lengths, hq, hkv, d, window):
    return synth.prefill_case(seed_of(name), lengths, hq, hkv, d, window, std=0.5)


def all_chunks(case, seed, n_cuts=3):
    out = []
    for i, s in enumerate(case.seqs):
        c = synth.chunk_bounds(seed, s.length, n_cuts)
        out += [(i, a, b) for a, b in zip(c[:-1], c[1:])]
    return out


def run_paged(pc, case, want_lse=False, max_query_len=None, max_context_len=None):
    mql = pc.max_query_len() if max_query_len is None else max_query_len
    mcl = pc.max_context_len() if max_context_len is None else max_context_len
    q = bf16_dev(pc.q)
    lse = (torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
           if want_lse else None)
    o = ia.attn_prefill_paged(q, bf16_dev(pc.k_cache), bf16_dev(pc.v_cache),
                              i32_dev(pc.block_table), i32_dev(pc.cu_seqlens),
                              i32_dev(pc.q_start), mql, mcl, window=case.window,
                              softmax_scale=case.scale, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def full_rows(case):
    """Unchunked varlen prefill of the whole case: (out bits, lse, cu)."""
    packed, o, lse = run_case(case, want_lse=True)
    return bits(o), lse.cpu().numpy(), packed[3]


def assert_chunks_equal(pc, o_bits, lse, ref_bits, ref_lse, ref_cu, what):
    for c, (i, a, b) in enumerate(zip(pc.seq, pc.start, pc.end)):
        r0, r1 = int(pc.cu_seqlens[c]), int(pc.cu_seqlens[c + 1])
        f0 = int(ref_cu[i]) + a
        assert np.array_equal(o_bits[r0:r1], ref_bits[f0:f0 + (b - a)]), (what, i, a, b)
        if lse is not None:
            assert np.array_equal(lse[r0:r1].view(np.uint32),
                                  ref_lse[f0:f0 + (b - a)].view(np.uint32)), (what, "lse", i, a, b)


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window", CASES, ids=[c[0] for c in CASES])
def test_chunks_equal_unchunked_rows_bitwise(name, lengths, hq, hkv, d, window):
    case = make_case(name, lengths, hq, hkv, d, window)
    ref_bits, ref_lse, ref_cu = full_rows(case)
    chunks = all_chunks(case, seed_of(name))
    # Every chunk in one call, in a shuffled batch order.
    perm = np.random.default_rng([seed_of(name), 0, 31]).permutation(len(chunks))
    pc = synth.paged_chunks(case, [chunks[p] for p in perm])
    o, lse = run_paged(pc, case, want_lse=True)
    assert_chunks_equal(pc, bits(o), lse.cpu().numpy(), ref_bits, ref_lse, ref_cu, "one call")
    # Chunk r of every sequence in call r (chunked prefill as a server runs
    # it), with another physical block placement.
    per_seq = {}
    for ch in chunks:
        per_seq.setdefault(ch[0], []).append(ch)
    rounds = max(len(v) for v in per_seq.values())
    for r in range(rounds):
        batch = [v[r] for v in per_seq.values() if r < len(v)]
        pc = synth.paged_chunks(case, batch, placement_seed=r + 1)
        o, lse = run_paged(pc, case, want_lse=True)
        assert_chunks_equal(pc, bits(o), lse.cpu().numpy(), ref_bits, ref_lse, ref_cu,
                            f"round {r}")


@pytest.mark.parametrize("name,lengths,hq,hkv,d,window", CASES, ids=[c[0] for c in CASES])
def test_parity_with_oracle(name, lengths, hq, hkv, d, window):
    case = make_case(name, lengths, hq, hkv, d, window)
    pc = synth.paged_chunks(case, all_chunks(case, seed_of(name) + 1))
    o, lse = run_paged(pc, case, want_lse=True)
    # Oracle: query row at position p of sequence i is a decode step with
    # context [0, p] read through sequence i's table row.
    pos = np.concatenate([np.arange(a, b) for a, b in zip(pc.start, pc.end)])
    tab = np.concatenate([np.repeat(pc.block_table[c:c + 1], b - a, axis=0)
                          for c, (a, b) in enumerate(zip(pc.start, pc.end))])
    ref, ref_lse = oracle.decode(pc.q, pc.k_cache, pc.v_cache, tab, (pos + 1).astype(np.int32),
                                 window=case.window, scale=case.scale, want_lse=True)
    gate(f64(o), ref, name)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-3, name


def test_grid_bounds_and_table_padding_do_not_change_bytes():
    case = make_case("bounds", [700, 90], 32, 16, 256, 128)
    chunks = all_chunks(case, 5)
    pc = synth.paged_chunks(case, chunks)
    a, _ = run_paged(pc, case)
    pc2 = synth.paged_chunks(case, chunks, max_blocks=200, spare_blocks=50, placement_seed=9)
    b, _ = run_paged(pc2, case)
    c, _ = run_paged(pc2, case, max_query_len=pc.max_query_len() + 300, max_context_len=3000)
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(a), bits(c))


@pytest.mark.parametrize("d,hq,hkv,window", [(512, 32, 4, synth.NO_WINDOW),
                                             (256, 32, 16, 1024), (64, 8, 2, 100)])
def test_single_token_chunks_equal_prefill_row_bytes(d, hq, hkv, window):
    """A decode step as a one-token chunk at position L-1 gives the bytes of
    prefill row L-1; the split decode gives the same values to the parity
    tolerance (its fixed chunk-and-merge order differs)."""
    lengths = [3000, 1037, 4096, 1]
    case = synth.prefill_case(77, lengths, hq, hkv, d, window, std=0.5)
    ref_bits, ref_lse, ref_cu = full_rows(case)
    pc = synth.paged_chunks(case, [(i, L - 1, L) for i, L in enumerate(lengths)])
    o, lse = run_paged(pc, case, want_lse=True)
    assert_chunks_equal(pc, bits(o), lse.cpu().numpy(), ref_bits, ref_lse, ref_cu, "decode rows")
    ob = ia.attn_decode_paged(bf16_dev(pc.q), bf16_dev(pc.k_cache), bf16_dev(pc.v_cache),
                              i32_dev(pc.block_table), i32_dev(np.array(lengths, np.int32)),
                              max(lengths), window=window, softmax_scale=case.scale)
    torch.cuda.synchronize()
    gate(f64(ob), f64(o), "split decode vs one-token chunks")


def test_never_reads_blocks_outside_the_attended_range():
    """Table entries of blocks wholly below the first new row's window, and
    past each chunk's last key, hold out-of-range ids: nothing changes."""
    W = 40
    case = make_case("evict", [400, 250], 8, 2, 64, W)
    chunks = [(0, 0, 1), (0, 130, 135), (0, 333, 400), (1, 77, 200), (1, 249, 250)]
    pc = synth.paged_chunks(case, chunks)
    clean, _ = run_paged(pc, case)
    bt = pc.block_table.copy()
    for c, (a, b) in enumerate(zip(pc.start, pc.end)):
        klo = max(0, a - W + 1)
        bt[c, :klo // 16] = 2 ** 30
        bt[c, (b + 15) // 16:] = -5
    pc.block_table = bt
    dirty, _ = run_paged(pc, case)
    assert np.array_equal(bits(clean), bits(dirty))


def test_empty_chunks_and_batches():
    case = make_case("empty", [100, 50], 4, 2, 64, synth.NO_WINDOW)
    ref_bits, ref_lse, ref_cu = full_rows(case)
    pc = synth.paged_chunks(case, [(0, 40, 40), (1, 10, 50), (0, 0, 0), (0, 40, 100)])
    o, lse = run_paged(pc, case, want_lse=True)
    assert_chunks_equal(pc, bits(o), lse.cpu().numpy(), ref_bits, ref_lse, ref_cu, "empty")
    # No query rows at all: nothing is enqueued, the output stays as it was.
    pc0 = synth.paged_chunks(case, [(0, 5, 5), (1, 0, 0)])
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    ia.attn_prefill_paged(q, bf16_dev(pc0.k_cache), bf16_dev(pc0.v_cache),
                          i32_dev(pc0.block_table), i32_dev(pc0.cu_seqlens),
                          i32_dev(pc0.q_start), 0, 5, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_paged_validation(monkeypatch):
    case = make_case("validate", [100, 40], 4, 2, 64, synth.NO_WINDOW)
    pc = synth.paged_chunks(case, [(0, 60, 100), (1, 0, 40)])
    plain, _ = run_paged(pc, case)
    monkeypatch.setenv("INVATTN_VALIDATE", "1")
    checked, _ = run_paged(pc, case)
    assert np.array_equal(bits(plain), bits(checked))
    bad = pc.block_table.copy()
    bad[1, 1] = pc.k_cache.shape[0] + 3
    pc.block_table = bad
    with pytest.raises(ia.AttnError) as e:
        run_paged(pc, case)
    assert e.value.name == "ATTN_E_VALIDATE"
    pc = synth.paged_chunks(case, [(0, 60, 100), (1, 0, 40)])
    with pytest.raises(ia.AttnError) as e:
        run_paged(pc, case, max_context_len=90)
    assert e.value.name == "ATTN_E_VALIDATE"
    pc.q_start = np.array([-1, 0], np.int32)
    with pytest.raises(ia.AttnError) as e:
        run_paged(pc, case)
    assert e.value.name == "ATTN_E_VALIDATE"

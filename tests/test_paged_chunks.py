"""Host checks of the chunked-prefill inputs (CPU only).

The paged-chunk generator must place every key of a sequence in the block
its table row names, and the parity reference of the chunked prefill (each
query row as an oracle decode step whose context ends at that row) must
equal the oracle's plain prefill of the unchunked sequences: the chunked
prefill computes the same rows as the prefill ("RFC: Gemma-4-31B-it
train/rollout consistency", section 4, item 6)."""
import numpy as np

import oracle
from invariant_attention_flash_amd import synth


def _case():
    return synth.prefill_case(7, [45, 17, 1], 4, 2, 64, 20, std=0.5)


def test_layout_gathers_back_to_each_sequence():
    case = _case()
    chunks = [(0, 0, 9), (0, 9, 45), (1, 3, 17), (2, 0, 1), (1, 17, 17)]
    pc = synth.paged_chunks(case, chunks, placement_seed=3)
    assert pc.cu_seqlens.tolist() == [0, 9, 45, 59, 60, 60]
    assert pc.q_start.tolist() == [0, 9, 3, 0, 17]
    for c, (i, a, b) in enumerate(chunks):
        s = case.seqs[i]
        assert np.array_equal(pc.q[pc.cu_seqlens[c]:pc.cu_seqlens[c + 1]], s.q[a:b])
        for j in range(s.length):
            blk = pc.block_table[c, j // 16]
            assert np.array_equal(pc.k_cache[blk, j % 16], s.k[j])
            assert np.array_equal(pc.v_cache[blk, j % 16], s.v[j])
        # table padding and unused slots are poison
        nb = (s.length + 15) // 16
        assert (pc.block_table[c, nb:] >= pc.k_cache.shape[0]).all()
        if s.length % 16:
            assert np.isnan(synth.bf16_to_f32(pc.k_cache[pc.block_table[c, nb - 1],
                                                         s.length % 16:])).all()


def test_chunk_bounds_cover_the_sequence():
    for L in (1, 2, 31, 500):
        c = synth.chunk_bounds(11, L, 4)
        assert c[0] == 0 and c[-1] == L
        assert all(x < y for x, y in zip(c[:-1], c[1:]))
        if L > 1:
            assert c[-2] == L - 1


def test_decode_steps_per_row_equal_prefill_rows():
    case = _case()
    chunks = [(0, 0, 9), (0, 9, 45), (1, 3, 17), (2, 0, 1)]
    pc = synth.paged_chunks(case, chunks)
    pos = np.concatenate([np.arange(a, b) for _, a, b in chunks])
    tab = np.concatenate([np.repeat(pc.block_table[c:c + 1], b - a, axis=0)
                          for c, (_, a, b) in enumerate(chunks)])
    got, got_lse = oracle.decode(pc.q, pc.k_cache, pc.v_cache, tab, (pos + 1).astype(np.int32),
                                 window=case.window, scale=case.scale, want_lse=True)
    q, k, v, cu, _ = case.pack()
    rows = []
    for c, (i, a, b) in enumerate(chunks):
        for p in range(a, b):
            rows += [(cu[i] + p, h) for h in range(case.hq)]
    ref, ref_lse = oracle.prefill(q, k, v, cu, window=case.window, scale=case.scale,
                                  rows=np.array(rows), want_lse=True)
    assert np.abs(got.reshape(-1, case.d) - ref).max() <= 1e-12
    assert np.abs(got_lse.reshape(-1) - ref_lse).max() <= 1e-12

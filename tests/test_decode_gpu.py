"""Paged decode on the GPU: parity with the fp64 oracle, bitwise invariance
of a sequence's output to batch size, batch position and physical block
placement, and that nothing outside the attended key range is read.

Sources: strict decode reads the paged KV cache in place ("Vime ROCm
Attention operator ablation", "Prerequisites"); fixed split and merge
("RFC: Gemma-4-31B-it train/rollout consistency", section 4, item 3); a row
is invariant to unrelated rows and padding mutation (item 6)."""
import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import bf16_dev, bits, f64, gate, i32_dev

pytestmark = pytest.mark.gpu


def run_decode(dc, max_seq_len=None, workspace=None):
    ms = int(dc.seq_lens.max()) if max_seq_len is None else max_seq_len
    o = ia.attn_decode_paged(bf16_dev(dc.q), bf16_dev(dc.k_cache), bf16_dev(dc.v_cache),
                             i32_dev(dc.block_table), i32_dev(dc.seq_lens), ms, window=dc.window,
                             softmax_scale=dc.scale, workspace=workspace)
    torch.cuda.synchronize()
    return o


def oracle_decode(dc):
    return oracle.decode(dc.q, dc.k_cache, dc.v_cache, dc.block_table, dc.seq_lens,
                         window=dc.window, scale=dc.scale)


LENGTHS = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1024, 1500]


@pytest.mark.parametrize("d,hq,hkv", [(512, 32, 4), (512, 8, 8), (256, 32, 16), (256, 16, 4),
                                      (64, 16, 2), (64, 4, 4)])
@pytest.mark.parametrize("window", [synth.NO_WINDOW, 1, 100, 600])
def test_decode_parity(d, hq, hkv, window):
    dc = synth.decode_case(seed=21, lengths=LENGTHS, batch=len(LENGTHS), hq=hq, hkv=hkv, d=d,
                           window=window)
    o = run_decode(dc)
    gate(f64(o), oracle_decode(dc), f"decode d={d} {hq}/{hkv} w={window}")


def test_decode_single_key_returns_v():
    """Window 1: the query sees only its own key, so the output is V exactly."""
    dc = synth.decode_case(seed=22, lengths=[1, 16, 17, 700], batch=4, hq=32, hkv=4, d=512,
                           window=1, std=1.0)
    got = bits(run_decode(dc))
    for b, L in enumerate(dc.seq_lens):
        j = L - 1
        blk = dc.block_table[b, j // 16]
        want = dc.v_cache[blk, j % 16]                 # [Hkv, D]
        assert np.array_equal(got[b], np.repeat(want, 8, axis=0)), b


def test_decode_bitwise_across_batches_positions_and_placement():
    lengths = synth.decode_lengths(31, 9, 1, 5000)
    ref = None
    for batch in (1, 2, 5, 9):
        for placement in (0, 1):
            dc = synth.decode_case(seed=31, lengths=lengths, batch=batch, hq=32, hkv=4, d=512,
                                   placement_seed=placement)
            out = bits(run_decode(dc))
            if ref is None:
                ref = out[0]
            assert np.array_equal(out[0], ref), (batch, placement)
    # sequence 0 at the last batch position, larger grid (max_seq_len)
    dc = synth.decode_case(seed=31, lengths=lengths, batch=9, hq=32, hkv=4, d=512,
                           order=[1, 2, 3, 4, 5, 6, 7, 8, 0], max_blocks=400)
    out = bits(run_decode(dc, max_seq_len=6000))
    assert np.array_equal(out[8], ref)


def test_decode_never_reads_outside_the_window():
    """Block-table entries for blocks wholly below the window hold garbage ids:
    the output does not change (they are never read)."""
    dc = synth.decode_case(seed=41, lengths=[3000, 700, 2049], batch=3, hq=32, hkv=4, d=512,
                           window=500)
    clean = bits(run_decode(dc))
    bt = dc.block_table.copy()
    for b, L in enumerate(dc.seq_lens):
        lo = max(0, int(L) - 500)
        bt[b, :lo // 16] = 2 ** 30
    dc.block_table = bt
    assert np.array_equal(bits(run_decode(dc)), clean)


def test_decode_workspace_contents_do_not_matter():
    dc = synth.decode_case(seed=42, lengths=[2000, 5], batch=2, hq=32, hkv=4, d=512)
    need = ia.attn_decode_workspace_size(2, 2000, 32, 512)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    a = bits(run_decode(dc, workspace=ws))
    ws.fill_(1e30)
    b = bits(run_decode(dc, workspace=ws))
    assert np.array_equal(a, b)
    gate(synth.bf16_to_f32(a).astype(np.float64), oracle_decode(dc), "workspace")


def test_decode_validation(monkeypatch):
    monkeypatch.setenv("INVATTN_VALIDATE", "1")
    dc = synth.decode_case(seed=43, lengths=[100, 40], batch=2, hq=32, hkv=4, d=512)
    bad = dc.block_table.copy()
    bad[1, 0] = dc.k_cache.shape[0] + 3
    dc2 = synth.DecodeCase(dc.q, dc.k_cache, dc.v_cache, bad, dc.seq_lens, dc.hq, dc.hkv, dc.d,
                           dc.block_size, dc.window, dc.scale)
    with pytest.raises(ia.AttnError) as e:
        run_decode(dc2)
    assert e.value.name == "ATTN_E_VALIDATE"
    with pytest.raises(ia.AttnError) as e:
        run_decode(dc, max_seq_len=50)
    assert e.value.name == "ATTN_E_VALIDATE"
    gate(f64(run_decode(dc)), oracle_decode(dc), "validated decode")


@pytest.mark.parametrize("d,hq,hkv,window", [(512, 32, 4, synth.NO_WINDOW), (256, 16, 4, 100),
                                             (64, 8, 2, synth.NO_WINDOW)])
def test_decode_v_aliasing_k(d, hq, hkv, window):
    """V = K passed as one cache (global_k_eq_v_projection, "RFC: Gemma-4-31B-it
    train/rollout consistency", section 6): each block is read once, and the
    bytes equal those of a separate V cache holding the same values."""
    dc = synth.decode_case(seed=51, lengths=LENGTHS, batch=len(LENGTHS), hq=hq, hkv=hkv, d=d,
                           window=window)
    kc = bf16_dev(dc.k_cache)
    args = (bf16_dev(dc.q), i32_dev(dc.block_table), i32_dev(dc.seq_lens))
    ms = int(dc.seq_lens.max())

    def run(vc):
        o = ia.attn_decode_paged(args[0], kc, vc, args[1], args[2], ms, window=dc.window,
                                 softmax_scale=dc.scale)
        torch.cuda.synchronize()
        return o

    alias = bits(run(kc))
    copy = bits(run(kc.clone()))
    assert np.array_equal(alias, copy)
    ref = oracle.decode(dc.q, dc.k_cache, dc.k_cache, dc.block_table, dc.seq_lens,
                        window=dc.window, scale=dc.scale)
    gate(synth.bf16_to_f32(alias).astype(np.float64), ref, f"alias d={d}")

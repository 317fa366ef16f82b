"""The allocation-free decode entry point (attn_decode_paged_noalloc),
called through the C ABI: its output equals attn_decode_paged's (same
kernels, so byte for byte, which is within the parity tolerance) on two calls
in a row, the second with a smaller batch and shorter contexts, so the
second call runs on records the first left in the library's scratch."""
import ctypes

import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import bf16_dev, bits, f64, gate, i32_dev

pytestmark = pytest.mark.gpu


def _c_decode(lib, noalloc, dc, q, bt, sl, max_len, out, ws=None):
    vp = ctypes.c_void_p
    p = lambda t: vp(t.data_ptr())
    stream = vp(torch.cuda.current_stream().cuda_stream)
    B, hq, d = q.shape
    nb, bs, hkv, _ = dc["k"].shape
    common = (p(q), p(dc["k"]), p(dc["v"]), p(bt), bt.shape[1], p(sl), B, max_len, nb, bs, hq,
              hkv, d, -1, ctypes.c_float(d ** -0.5))
    if noalloc:
        return lib.attn_decode_paged_noalloc(*common, p(out), stream)
    return lib.attn_decode_paged(*common, p(ws), ctypes.c_size_t(ws.numel()), p(out), stream)


def test_noalloc_equals_workspace_decode_twice():
    lib = ia.library()
    case = synth.decode_case(seed=31, lengths=[5000, 1, 777, 2049, 16, 3000], batch=6, hq=32,
                             hkv=4, d=512)
    dc = {"k": bf16_dev(case.k_cache), "v": bf16_dev(case.v_cache)}
    q_all = bf16_dev(case.q)
    bt_all = i32_dev(case.block_table)
    calls = [(6, int(case.seq_lens.max())), (3, int(case.seq_lens[:3].max()))]
    for n, (B, max_len) in enumerate(calls):
        q, bt = q_all[:B].contiguous(), bt_all[:B].contiguous()
        sl = i32_dev(case.seq_lens[:B])
        need = ia.attn_decode_workspace_size(B, max_len, 32, 512)
        assert need <= ia.ATTN_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        assert _c_decode(lib, False, dc, q, bt, sl, max_len, ref, ws) == 0, ia.last_error()
        assert _c_decode(lib, True, dc, q, bt, sl, max_len, got) == 0, ia.last_error()
        torch.cuda.synchronize()
        assert ia.last_provenance()["op"] == "attn_decode_paged_noalloc"
        assert np.array_equal(bits(got), bits(ref)), f"call {n}: bytes differ"
        # and both meet the parity gate against the oracle
        want = oracle.decode(case.q[:B], case.k_cache, case.v_cache, case.block_table[:B],
                             case.seq_lens[:B])
        gate(f64(got), want, f"noalloc call {n}")


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    lib = ia.library()
    q = torch.zeros((64, 32, 512), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    kc = torch.zeros((4, 16, 4, 512), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, 2048), dtype=torch.int32, device="cuda")
    sl = torch.ones(64, dtype=torch.int32, device="cuda")
    vp = ctypes.c_void_p
    p = lambda t: vp(t.data_ptr())
    rc = lib.attn_decode_paged_noalloc(p(q), p(kc), p(kc), p(bt), 2048, p(sl), 64, 32768, 4, 16,
                                       32, 4, 512, -1, ctypes.c_float(0.044), p(out), None)
    assert rc == 5 and "scratch" in ia.last_error()

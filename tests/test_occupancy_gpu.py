"""Output bytes do not depend on how many CUs run the work or on what else
occupies the GPU ("RFC: Gemma-4-31B-it train/rollout consistency", section
4, item 2: an order independent of the SM/CU count and of runtime
occupancy).  Every entry point runs on the same seeded inputs three ways:
on the whole device; in a child process whose queues the runtime restricts
to a quarter of the CUs (HSA_CU_MASK); and on the whole device while a
second stream keeps the matrix cores busy with a bounded run of plain GEMMs.
The bytes must be identical."""
import os
import subprocess
import sys
import time

import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _inputs():
    """Seeded device-built inputs of every entry point: a sliding-window
    prefill shaped like the sliding workload (8 sequences of U[512, 4096]
    tokens, 32/16 heads, head dim 256, window 1024), a global prefill with
    spans (32/4 heads, head dim 512), a batch-8 paged decode (32/4 heads,
    head dim 512, contexts U[1024, 32768]) and a backward (16/8 heads, head
    dim 256, window 512)."""
    dev = torch.device("cuda:0")
    inp = {}
    lengths = synth.sliding_lengths(2, 8, 512, 4096)
    inp["sliding"] = synth.prefill_case_device(2, lengths, 32, 16, 256, 1024, std=0.5, device=dev)
    spans = [[(100, 356)], [(0, 256), (2000, 2256)]]
    inp["global"] = synth.prefill_case_device(3, [1000, 3000], 32, 4, 512, -1, std=0.5,
                                              spans=spans, device=dev)
    lens = synth.decode_lengths(4, 8, 1024, 32768)
    dc = synth.decode_case_device(4, lens, batch=8, hq=32, hkv=4, d=512, device=dev)
    dc["bt"] = torch.from_numpy(dc["block_table"]).to(dev)
    dc["sl"] = torch.from_numpy(dc["seq_lens"]).to(dev)
    dc["max"] = max(lens)
    dc["ws"] = torch.empty(ia.attn_decode_workspace_size(8, max(lens), 32, 512),
                           dtype=torch.uint8, device=dev)
    inp["decode"] = dc
    case = synth.prefill_case_device(12, [700, 1500], 16, 8, 256, 512, std=0.5, device=dev)
    lse = torch.empty(case["q"].shape[:2], dtype=torch.float32, device=dev)
    case["o"] = ia.attn_prefill_varlen(case["q"], case["k"], case["v"], case["cu_seqlens"],
                                       case["max_seqlen"], window=512, lse=lse)
    case["lse"] = lse
    g = synth.upstream_grad(12, tuple(case["q"].shape))
    case["dout"] = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev)
    inp["backward"] = case
    torch.cuda.synchronize()
    return inp


def _run(inp, stream=None):
    """Every entry point on the inputs, on `stream` (default: the current
    one).  Returns {name: int16/int32 CPU tensor of the output bits}."""
    s = torch.cuda.current_stream() if stream is None else stream
    out = {}
    for name in ("sliding", "global"):
        c = inp[name]
        lse = torch.empty(c["q"].shape[:2], dtype=torch.float32, device="cuda")
        o = torch.empty_like(c["q"])
        ia.attn_prefill_varlen(c["q"], c["k"], c["v"], c["cu_seqlens"], c["max_seqlen"],
                               window=c["window"], softmax_scale=c["scale"], spans=c["spans"],
                               out=o, lse=lse, stream=s)
        out[name] = o
        out[name + "_lse"] = lse
    dc = inp["decode"]
    o = torch.empty_like(dc["q"])
    ia.attn_decode_paged(dc["q"], dc["k_cache"], dc["v_cache"], dc["bt"], dc["sl"], dc["max"],
                         softmax_scale=dc["scale"], workspace=dc["ws"], out=o, stream=s)
    out["decode"] = o
    c = inp["backward"]
    grads = ia.attn_prefill_varlen_backward(c["q"], c["k"], c["v"], c["o"], c["lse"], c["dout"],
                                            c["cu_seqlens"], c["max_seqlen"], window=512,
                                            stream=s)
    for n, t in zip(("dq", "dk", "dv"), grads):
        out[n] = t
    s.synchronize()
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32)).cpu()
            for k, v in out.items()}


def _gemm_ms(size=8192, n=10):
    """Milliseconds of n bf16 GEMMs of size^3 (how much of the chip runs)."""
    a = torch.randn((size, size), device="cuda").to(torch.bfloat16)
    b = torch.randn((size, size), device="cuda").to(torch.bfloat16)
    torch.mm(a, b)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n):
        torch.mm(a, b)
    torch.cuda.synchronize()
    return (time.perf_counter() - t) * 1e3


def _child(path):
    """Run in the CU-masked child process: save the outputs and a GEMM time."""
    res = _run(_inputs())
    res["gemm_ms"] = torch.tensor([_gemm_ms()], dtype=torch.float64)
    torch.save(res, path)


def _same(a, b, what):
    assert set(a) == set(b), what
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} bytes differ"


def test_quarter_of_the_cus_gives_the_same_bytes(tmp_path):
    base = _run(_inputs())
    full_ms = _gemm_ms()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    path = str(tmp_path / "child.pt")
    env = dict(os.environ)
    env["HSA_CU_MASK"] = f"0:0-{n_cu // 4 - 1}"
    code = (f"import sys; sys.path[:0] = [{HERE!r}, {os.path.dirname(HERE)!r}]; "
            f"import test_occupancy_gpu as t; t._child({path!r})")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    child = torch.load(path, weights_only=True)
    masked_ms = float(child.pop("gemm_ms")[0])
    # the mask took effect: the same GEMMs ran on far fewer CUs
    assert masked_ms > 2.0 * full_ms, (masked_ms, full_ms)
    _same(base, child, f"{n_cu // 4} of {n_cu} CUs")


def test_concurrent_gemm_load_gives_the_same_bytes():
    inp = _inputs()
    base = _run(inp)
    side = torch.cuda.Stream()
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(60):
            a = torch.mm(a, b) * 1e-2      # tens of milliseconds of matrix-core work
    loaded = _run(inp)                     # queued behind nothing: runs beside the GEMMs
    torch.cuda.synchronize()
    _same(base, loaded, "beside a GEMM load")

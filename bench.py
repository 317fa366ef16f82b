#!/usr/bin/env python3
"""Benchmark of the batch-invariant attention forward on one MI355X.

One step = one pass of the whole hot path on synthetic inputs resident in
HBM: the hybrid multimodal-style prefill (5 sliding-window layers with head
dim 256, window 1024, 32 query / 16 KV heads, then 1 global layer with head
dim 512, 32 query / 4 KV heads, over a packed batch of 4 sequences of 4096
tokens, each holding two bidirectional 256-token spans; independent bf16
N(0,1)*0.5 Q/K/V per layer), then a paged-KV decode of 64 sequences
(contexts U[1024, 32768], 32 query / 4 KV heads, head dim 512, 16-token
blocks, shuffled block tables).

``value`` is the hybrid prefill's algorithmic TFLOP/s: 4 * head_dim *
query_heads * allowed query-key pairs summed over the six layers (masked work
not counted), over the HIP-event-timed launches of the six layers.  Reported
beside it, each with its own roofline: every layer; the sliding-window
prefill over 8 sequences of U[512, 4096] tokens and the global prefill over
{2048, 4096, 6144, 8192} tokens (their own timed regions); the decode's
algorithmic HBM GB/s (K and V of every attended context token, plus q, o and
block-table reads) at batch 64 in the step and at batches 1, 8, 32, 64 with
the last-level cache flushed before each call; and the backward (dq, dk, dv)
of the sliding prefill.  The fp64 CPU oracle is timed on bounded samples of
the same hybrid rows and decode sequences on the host cores (a reported
baseline, not a target), and its outputs double as parity spot-checks.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FLUSH_BYTES = 512 << 20     # read between decode calls: twice the 256 MB last-level cache

# Kernel instances, by the name rocprofv3 prints (demangled), and the key of
# their HBM traffic in profiles/traffic.json.
KERNELS = {
    "prefill_ws_kernel<256,2,2,3,32>": "prefill_ws_kernel<invattn::PfWsCfg<256, 2, 2, 3, 32> >",
    "prefill_ws_kernel<512,8,1,2,32>": "prefill_ws_kernel<invattn::PfWsCfg<512, 8, 1, 2, 32> >",
    "decode_chunk_kernel<512,8>+decode_merge_kernel<512>": "decode_",
}


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_attention_flash_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def allowed_pairs_per_row(L, window, spans=()):
    """|A_i| for every row of one sequence (causal window plus same-span keys)."""
    i = np.arange(L, dtype=np.int64)
    lo = np.zeros(L, np.int64) if window < 0 else np.maximum(0, i - window + 1)
    cnt = i - lo + 1
    for s, e in spans:
        inside = (i >= s) & (i < e)
        below = np.clip(np.minimum(e, lo) - s, 0, None)          # span keys under the window
        above = np.clip(e - np.maximum(s, i + 1), 0, None)        # span keys after the row
        cnt = cnt + np.where(inside, below + above, 0)
    return cnt


def prefill_flops(lengths, hq, d, window, spans=None):
    pairs = 0
    for n, L in enumerate(lengths):
        pairs += int(allowed_pairs_per_row(L, window, spans[n] if spans else ()).sum())
    return 4.0 * d * hq * pairs, pairs


def decode_bytes(seq_lens, hq, hkv, d, window=-1, block=16):
    b = 0
    for L in seq_lens:
        keys = L if window < 0 else min(L, window)
        b += keys * hkv * d * 2 * 2                  # K and V, bf16
        b += ((L + block - 1) // block - (L - keys) // block) * 4   # block-table entries
        b += 4                                        # seq_lens entry
    b += len(seq_lens) * hq * d * 2 * 2               # q and o
    return b


def bf16_rne_bits(x):
    """fp64 values rounded once to bf16 (round to nearest, ties to even), as
    bf16 bit patterns.  Exact: the value is rounded at its own binade's bf16
    spacing (2^(e-7), floored at the subnormal spacing 2^-133) in fp64, where
    scaling by a power of two is exact and numpy rounds halves to even; the
    result is a bf16 value, which float32 holds exactly."""
    x = np.asarray(x, np.float64)
    finite = np.isfinite(x) & (x != 0)
    _, e2 = np.frexp(np.where(finite, x, 1.0))   # |x| in [2^(e2-1), 2^e2)
    e = np.maximum(e2 - 1, -126)
    ulp = np.ldexp(1.0, e - 7)
    r = np.where(finite, np.round(x / ulp) * ulp, x)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def correctly_rounded_share(got_bits, ref):
    """Share of bf16 outputs equal in value to the bf16 rounding of the fp64
    reference (+0 and -0 count as equal)."""
    def f32(b):
        return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return float(np.mean(f32(got_bits) == f32(bf16_rne_bits(ref))))


def load_traffic(kernel: str):
    """HBM traffic per launch from the committed counter summary, only if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = t.get(kernel)
    if not rec or rec.get("sources_hash") != kernel_sources_hash():
        return None
    return rec.get("bytes_per_launch")


CALIBRATION_BYTES = 1 << 30   # plain streaming kernel used to scale the HBM byte counters


def write_traffic(fetch_dir, write_dir):
    """Turn two rocprofv3 counter runs of `bench.py --calibrate` (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch) into profiles/traffic.json: per-launch
    HBM bytes of each benchmarked kernel, each counter scaled so the
    calibration copy of CALIBRATION_BYTES reads (writes) exactly that much."""
    import csv
    import glob

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"]), int(r["Grid_Size"])))
        return rows

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = load(d, counter)
        # the calibration pass: an elementwise negation reading and writing 1 GiB
        calib = [v for k, v, g in rows if "neg_kernel" in k]
        if not calib:
            raise SystemExit(f"no calibration kernel found in {d}")
        scale = CALIBRATION_BYTES / (1024.0 * float(np.median(calib)))
        for key, match in KERNELS.items():
            first = "decode_chunk_kernel" if key.startswith("decode") else match
            sel = [(k, v, g) for k, v, g in rows if match in k and "KvAliasOf" not in k]
            if key.startswith("decode"):
                # the step's batch-64 decode: the largest grid of the chunk
                # kernels and of the merge kernels (the --step-only run also
                # decodes batch 1, with a chunk kernel of another ring depth)
                fam = lambda k: "chunk" if "decode_chunk_kernel" in k else "merge"
                big = {}
                for k, v, g in sel:
                    big[fam(k)] = max(big.get(fam(k), 0), g)
                sel = [(k, v, g) for k, v, g in sel if g == big[fam(k)]]
            vals = [v for k, v, g in sel]
            launches = sum(1 for k, v, g in sel if first in k)
            if not vals or not launches:
                continue
            per_launch = 1024.0 * scale * sum(vals) / launches
            rec = out.setdefault(key, {"sources_hash": kernel_sources_hash()})
            rec[counter.lower() + "_bytes"] = per_launch
            rec[counter.lower() + "_scale"] = scale
            rec["launches_" + counter.lower()] = launches
    for rec in out.values():
        rec["bytes_per_launch"] = rec.get("fetch_size_bytes", 0.0) + rec.get("write_size_bytes", 0.0)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


def roofline(bound, achieved, peak, unit, kernel, work, ms, traffic_key=None):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak,
            "traffic": load_traffic(traffic_key) if traffic_key else None,
            "kernel": kernel, "work_per_launch": work, "avg_launch_ms": ms}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20,
                    help="timed calls of each reported workload outside the step")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed calls of the backward on the sliding workload (0 disables)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the prefill oracle sample (0 disables every "
                         "oracle leg)")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step (six hybrid layers + batch-64 decode): the "
                         "command the kernel traces and counters are taken on")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB copy (scale for the HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: build profiles/traffic.json from two counter runs")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every box here has one GPU); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_attention_flash_amd as ia
    from invariant_attention_flash_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ia.library()
    stream = torch.cuda.current_stream()   # the library launches on this stream

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------- inputs (resident in HBM before timing)
    HY_N, HY_LEN = 4, 4096
    hy_spans = synth.hybrid_spans(5, HY_N, HY_LEN, 256)
    layers = []
    for li, (hq, hkv, d, w) in enumerate(synth.HYBRID_LAYERS):
        case = synth.prefill_case_device(5 * 100 + li, [HY_LEN] * HY_N, hq, hkv, d, w, std=0.5,
                                         spans=hy_spans, device=dev)
        fl, pr = prefill_flops([HY_LEN] * HY_N, hq, d, w, hy_spans)
        case["flops"], case["pairs"] = fl, pr
        case["out"] = torch.empty_like(case["q"])
        layers.append(case)
    hy_flops = sum(c["flops"] for c in layers)
    log(f"hybrid inputs ready: {hy_flops:.4g} FLOP over {len(layers)} layers")

    sl_len = synth.sliding_lengths(2, 8, 512, 4096)
    sl = synth.prefill_case_device(2, sl_len, 32, 16, 256, 1024, std=0.5, device=dev)
    sl["flops"], sl["pairs"] = prefill_flops(sl_len, 32, 256, 1024)
    sl["out"] = torch.empty_like(sl["q"])
    gl_len = [2048, 4096, 6144, 8192]
    gl = synth.prefill_case_device(3, gl_len, 32, 4, 512, -1, std=0.5, device=dev)
    gl["flops"], gl["pairs"] = prefill_flops(gl_len, 32, 512, -1)
    gl["out"] = torch.empty_like(gl["q"])

    DB = 64
    dlen = synth.decode_lengths(4, DB, 1024, 32768)
    dc = synth.decode_case_device(4, dlen, batch=DB, hq=32, hkv=4, d=512, device=dev)
    d_bt = torch.from_numpy(dc["block_table"]).to(dev)
    d_sl = torch.from_numpy(dc["seq_lens"]).to(dev)
    d_max = int(max(dlen))
    ws = torch.empty(ia.attn_decode_workspace_size(DB, d_max, 32, 512), dtype=torch.uint8,
                     device=dev)
    d_out = torch.empty_like(dc["q"])
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("all inputs resident")

    def prefill(c):
        ia.attn_prefill_varlen(c["q"], c["k"], c["v"], c["cu_seqlens"], c["max_seqlen"],
                               window=c["window"], softmax_scale=c["scale"], spans=c["spans"],
                               out=c["out"])

    def decode(B, out=None):
        ia.attn_decode_paged(dc["q"][:B], dc["k_cache"], dc["v_cache"], d_bt[:B], d_sl[:B],
                             int(max(dlen[:B])), softmax_scale=dc["scale"], workspace=ws,
                             out=d_out[:B] if out is None else out)

    if args.calibrate:
        # plain streaming kernel of known traffic: reads and writes 1 GiB
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for c in layers:
            prefill(c)
        decode(DB)
    torch.cuda.synchronize()

    # ---------------- the step: six hybrid layers, then the batch-64 decode
    nl = len(layers)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 2)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        for li, c in enumerate(layers):
            prefill(c)
            e[li + 1].record(stream)
        decode(DB)
        e[nl + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    layer_ms = [float(np.mean([e[li].elapsed_time(e[li + 1]) for e in evs])) for li in range(nl)]
    hy_ms = float(np.mean([e[0].elapsed_time(e[nl]) for e in evs]))
    dc_ms = float(np.mean([e[nl].elapsed_time(e[nl + 1]) for e in evs]))
    ms_step = wall * 1e3 / args.steps
    hy_tflops = hy_flops / (hy_ms * 1e-3) / 1e12
    log(f"step: hybrid {hy_ms:.3f} ms ({hy_tflops:.1f} TFLOP/s), decode {dc_ms:.3f} ms")

    def layer_kernel(c):
        return ("prefill_ws_kernel<256,2,2,3,32>" if c["d"] == 256 else "prefill_ws_kernel<512,8,1,2,32>")

    per_layer = []
    kern_ms, kern_flops = {}, {}
    for c, ms in zip(layers, layer_ms):
        tf = c["flops"] / (ms * 1e-3) / 1e12
        k = layer_kernel(c)
        kern_ms[k] = kern_ms.get(k, 0.0) + ms
        kern_flops[k] = kern_flops.get(k, 0.0) + c["flops"]
        per_layer.append({"kind": "global" if c["window"] < 0 else "sliding", "kernel": k,
                          "ms": ms, "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS,
                          "pairs": c["pairs"]})
    # the dominant kernel of the step: the instance with the most time
    dom = max(kern_ms, key=kern_ms.get)
    n_dom = sum(1 for c in layers if layer_kernel(c) == dom)
    dom_tf = kern_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    hy_roof = roofline("mfma", dom_tf, PEAK_BF16_TFLOPS, "TFLOP/s", dom,
                       f"{kern_flops[dom] / n_dom:.4g} FLOP per launch ({n_dom} launches per step: "
                       "4*head_dim*32*allowed pairs)", kern_ms[dom] / n_dom, dom)
    hy_roof["all_layers"] = {"achieved": hy_tflops, "frac": hy_tflops / PEAK_BF16_TFLOPS,
                             "flops": hy_flops, "ms": hy_ms}

    # ---------------- the sliding and global prefills (timed regions of their own)
    def time_calls(fn, reps, before=None):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            if before is not None:
                before()
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return [x[0].elapsed_time(x[1]) for x in ev]

    reported = {}
    for name, c, k in (() if args.step_only else
                       (("sliding_prefill", sl, "prefill_ws_kernel<256,2,2,3,32>"),
                        ("global_prefill", gl, "prefill_ws_kernel<512,8,1,2,32>"))):
        prefill(c)
        t = time_calls(lambda: prefill(c), args.reps)
        ms = float(np.mean(t))
        tf = c["flops"] / (ms * 1e-3) / 1e12
        reported[name] = {
            "value": tf, "unit": "TFLOP/s", "ms_mean": ms, "ms_min": float(np.min(t)),
            "tokens": int(sum(c["lengths"])), "lengths": c["lengths"], "pairs": c["pairs"],
            "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", k,
                                 f"{c['flops']:.4g} FLOP = 4*{c['d']}*32*{c['pairs']} allowed "
                                 "pairs", ms, k)}
        log(f"{name}: {ms:.3f} ms ({tf:.1f} TFLOP/s)")

    # ---------------- decode at every batch size, last-level cache flushed
    def flush_llc():
        # Read (not write) twice the last-level cache: a written buffer would
        # leave it full of dirty lines whose write-back then competes with
        # the timed call's reads.
        torch.sum(flush, dim=0, out=flush_sink)

    sweep = {}
    for B in () if args.step_only else (1, 8, 32, 64):
        decode(B)
        t = time_calls(lambda: decode(B), args.reps, before=flush_llc)
        ms = float(np.mean(t))
        nbytes = decode_bytes(dlen[:B], 32, 4, 512)
        gbs = nbytes / (ms * 1e-3) / 1e9
        sweep[str(B)] = {"GB/s": gbs, "frac": gbs / PEAK_HBM_GBS, "ms_mean": ms,
                         "ms_min": float(np.min(t)), "bytes": nbytes,
                         "context_tokens": int(sum(dlen[:B]))}
        log(f"decode B={B}: {ms * 1e3:.1f} us ({gbs:.0f} GB/s)")
    # K = V (one cache holds both): each block is loaded once
    alias = {}
    for B in () if args.step_only else (8, 64):
        def decode_alias():
            ia.attn_decode_paged(dc["q"][:B], dc["k_cache"], dc["k_cache"], d_bt[:B], d_sl[:B],
                                 int(max(dlen[:B])), softmax_scale=dc["scale"], workspace=ws,
                                 out=d_out[:B])
        decode_alias()
        t = time_calls(decode_alias, args.reps, before=flush_llc)
        ms = float(np.mean(t))
        nbytes = decode_bytes(dlen[:B], 32, 4, 512) - sum(dlen[:B]) * 4 * 512 * 2
        gbs = nbytes / (ms * 1e-3) / 1e9
        alias[str(B)] = {"GB/s": gbs, "frac": gbs / PEAK_HBM_GBS, "ms_mean": ms,
                         "ms_min": float(np.min(t)), "bytes": nbytes}
        log(f"decode K=V B={B}: {ms * 1e3:.1f} us ({gbs:.0f} GB/s on the K bytes)")
    # one sequence's output bytes at every batch size (batch invariance, checked live)
    outs = {}
    for B in (1, 64) if args.step_only else (1, 8, 32, 64):
        o = torch.empty_like(dc["q"][:B])
        decode(B, out=o)
        outs[B] = o[0].clone()
    torch.cuda.synchronize()
    invariant = all(torch.equal(outs[1].view(torch.int16), outs[B].view(torch.int16))
                    for B in outs)
    dbytes = decode_bytes(dlen, 32, 4, 512)
    dc_gbs = dbytes / (dc_ms * 1e-3) / 1e9
    dkey = "decode_chunk_kernel<512,8>+decode_merge_kernel<512>"
    dc_roof = roofline("hbm", dc_gbs, PEAK_HBM_GBS, "GB/s", dkey,
                       f"{dbytes} B: K+V of {sum(dlen)} context tokens x 4 KV heads x 512 x 2 B "
                       "x 2, plus q, o, block tables", dc_ms, dkey)

    # ---------------- decode with the prefill's bytes: each sequence's new token
    # as a one-token chunk through the chunked prefill over the same paged
    # cache (batch 64, last-level cache flushed before each call)
    strict = None
    if not args.step_only:
        s_cu = torch.arange(DB + 1, dtype=torch.int32, device=dev)
        s_qs = (d_sl - 1).contiguous()
        s_out = torch.empty_like(dc["q"])

        def strict_decode():
            ia.attn_prefill_paged(dc["q"], dc["k_cache"], dc["v_cache"], d_bt, s_cu, s_qs, 1, d_max,
                                  softmax_scale=dc["scale"], out=s_out)

        strict_decode()
        t = time_calls(strict_decode, max(3, args.reps // 2), before=flush_llc)
        ms = float(np.mean(t))
        gbs = dbytes / (ms * 1e-3) / 1e9
        strict = {"value": gbs, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "ms_mean": ms,
                  "ms_min": float(np.min(t)), "batch": DB,
                  "kernel": "PagedOf prefill_ws_kernel<512,8,1,2,32> (one-token chunks)",
                  "note": "bytes equal to the prefill row L-1 (tested); the split decode agrees "
                          "within the parity tolerance"}
        log(f"strict decode B={DB}: {ms:.3f} ms ({gbs:.0f} GB/s)")

    # ---------------- backward of the sliding prefill (its own timed region)
    bw = None
    if args.backward_steps > 0 and not args.step_only:
        lse = torch.empty(sl["q"].shape[:2], dtype=torch.float32, device=dev)
        ia.attn_prefill_varlen(sl["q"], sl["k"], sl["v"], sl["cu_seqlens"], sl["max_seqlen"],
                               window=1024, softmax_scale=sl["scale"], out=sl["out"], lse=lse)
        g = torch.from_numpy(synth.upstream_grad(2, tuple(sl["q"].shape)).view(np.int16))
        dout = g.view(torch.bfloat16).to(dev)
        dq = torch.empty(sl["q"].shape, dtype=torch.float32, device=dev)
        dk = torch.empty(sl["k"].shape, dtype=torch.float32, device=dev)
        dv = torch.empty(sl["k"].shape, dtype=torch.float32, device=dev)
        bws = torch.empty(sl["q"].shape[:2], dtype=torch.float32, device=dev)

        def backward():
            ia.attn_prefill_varlen_backward(sl["q"], sl["k"], sl["v"], sl["out"], lse, dout,
                                            sl["cu_seqlens"], sl["max_seqlen"], window=1024,
                                            softmax_scale=sl["scale"], dq=dq, dk=dk, dv=dv,
                                            workspace=bws)

        backward()
        t = time_calls(backward, args.backward_steps)
        bw_ms = float(np.mean(t))
        bw_flops = 2.5 * sl["flops"]   # five products of D per allowed pair and head
        bw_tf = bw_flops / (bw_ms * 1e-3) / 1e12
        bw = {"value": bw_tf, "unit": "TFLOP/s", "calls": args.backward_steps,
              "roofline": roofline("mfma", bw_tf, PEAK_BF16_TFLOPS, "TFLOP/s",
                                   "bwd_dq_kernel<256> + bwd_dkv_ws_kernel<256> (one launch pair)",
                                   f"{bw_flops:.4g} FLOP = 10*256*32*{sl['pairs']} allowed pairs "
                                   "(dq, dk, dv of the sliding prefill)", bw_ms)}
        log(f"backward: {bw_ms:.3f} ms ({bw_tf:.1f} TFLOP/s)")
        del dq, dk, dv, bws, dout, lse

        # the global prefill's backward (head dim 512)
        lse = torch.empty(gl["q"].shape[:2], dtype=torch.float32, device=dev)
        ia.attn_prefill_varlen(gl["q"], gl["k"], gl["v"], gl["cu_seqlens"], gl["max_seqlen"],
                               softmax_scale=gl["scale"], out=gl["out"], lse=lse)
        gen = torch.Generator(device=dev)
        gen.manual_seed(3)
        dout = (torch.randn(gl["q"].shape, generator=gen, device=dev) * 0.5).to(torch.bfloat16)
        dq = torch.empty(gl["q"].shape, dtype=torch.float32, device=dev)
        dk = torch.empty(gl["k"].shape, dtype=torch.float32, device=dev)
        dv = torch.empty(gl["k"].shape, dtype=torch.float32, device=dev)
        bws = torch.empty(gl["q"].shape[:2], dtype=torch.float32, device=dev)

        def backward_global():
            ia.attn_prefill_varlen_backward(gl["q"], gl["k"], gl["v"], gl["out"], lse, dout,
                                            gl["cu_seqlens"], gl["max_seqlen"],
                                            softmax_scale=gl["scale"], dq=dq, dk=dk, dv=dv,
                                            workspace=bws)

        backward_global()
        t = time_calls(backward_global, args.backward_steps)
        ms = float(np.mean(t))
        fl = 2.5 * gl["flops"]
        tf = fl / (ms * 1e-3) / 1e12
        bw["global"] = {"value": tf, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                        "ms_mean": ms, "calls": args.backward_steps,
                        "kernel": "bwd_dq_kernel<512> + bwd_dkv_kernel<512>",
                        "work": f"{fl:.4g} FLOP = 10*512*32*{gl['pairs']} allowed pairs"}
        log(f"backward (global, head dim 512): {ms:.3f} ms ({tf:.1f} TFLOP/s)")
        del dq, dk, dv, bws, dout, lse

    # ---------------- the attention prologue (RMSNorm + RoPE on Q and K, in
    # place) at the hybrid layers' shapes; HBM-bound: each vector is read and
    # written once
    prologue = None
    if not args.step_only:
        prologue = {}
        for kind, (hq_, hkv_, d_) in (("sliding", (32, 16, 256)), ("global", (32, 4, 512))):
            R, F = synth.prologue_rotary(kind, d_)
            pc = synth.prologue_case(7, [HY_LEN] * HY_N, hq_, hkv_, d_, std=0.5)
            pq = torch.from_numpy(pc.q.view(np.int16)).view(torch.bfloat16).to(dev)
            pk = torch.from_numpy(pc.k.view(np.int16)).view(torch.bfloat16).to(dev)
            pp = torch.from_numpy(pc.positions).to(dev)
            pqw = torch.from_numpy(pc.q_weight).to(dev)
            pkw = torch.from_numpy(pc.k_weight).to(dev)

            def run_prologue():
                ia.attn_qk_prologue(pq, pk, pp, q_weight=pqw, k_weight=pkw,
                                    eps=synth.PROLOGUE_EPS, rotary_dims=R, freq_dims=F,
                                    rope_theta=synth.PROLOGUE_THETA[kind])

            run_prologue()
            t = time_calls(run_prologue, args.reps, before=flush_llc)
            ms = float(np.mean(t))
            T_ = HY_N * HY_LEN
            pbytes = 2 * T_ * (hq_ + hkv_) * d_ * 2 + 4 * T_ + 2 * 4 * d_
            gbs = pbytes / (ms * 1e-3) / 1e9
            prologue[kind] = {"value": gbs, "unit": "GB/s",
                              "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                                   f"qk_prologue_kernel<{d_}>",
                                                   f"{pbytes} B: q and k read and written once "
                                                   f"({T_} tokens x {hq_}+{hkv_} heads x {d_} x "
                                                   "2 B x 2), positions, weights", ms),
                              "ms_mean": ms, "rotary_dims": R, "freq_dims": F,
                              "theta": synth.PROLOGUE_THETA[kind]}
            log(f"prologue ({kind}, d {d_}): {ms * 1e3:.1f} us ({gbs:.0f} GB/s)")
            del pq, pk, pp, pqw, pkw

    # ---------------- a measured ceiling beside the published peak: a large
    # bf16 GEMM through the vendor library (torch.matmul)
    ceilings = None
    if not args.step_only:
        n = 8192
        ga = torch.randn((n, n), device=dev).to(torch.bfloat16)
        gb = torch.randn((n, n), device=dev).to(torch.bfloat16)
        gc = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
        torch.matmul(ga, gb, out=gc)
        t = time_calls(lambda: torch.matmul(ga, gb, out=gc), args.reps)
        gemm_tf = 2.0 * n ** 3 / (float(np.median(t)) * 1e-3) / 1e12
        del ga, gb, gc
        # HBM: a plain device-to-device copy of 1 GiB (read + write) and a sum
        # over the same GiB (read only), both through torch's own kernels
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        sink = torch.zeros((), dtype=torch.float32, device=dev)
        dst.copy_(src)
        t = time_calls(lambda: dst.copy_(src), args.reps)
        copy_gbs = 2.0 * CALIBRATION_BYTES / (float(np.median(t)) * 1e-3) / 1e9
        torch.sum(src, dim=0, out=sink)
        t = time_calls(lambda: torch.sum(src, dim=0, out=sink), args.reps)
        read_gbs = CALIBRATION_BYTES / (float(np.median(t)) * 1e-3) / 1e9
        del src, dst, sink
        ceilings = {"gemm_bf16_tflops": gemm_tf, "gemm": f"torch.matmul bf16 {n}x{n}x{n}, median",
                    "prefill_frac_of_gemm": hy_tflops / gemm_tf,
                    "torch_streaming": {
                        "copy_gbs": copy_gbs, "sum_gbs": read_gbs,
                        "note": "torch's own copy_ (read + write bytes) and sum (read bytes) over "
                                "1 GiB, median: context, not ceilings (the decode kernel streams "
                                "faster than both)",
                        "decode_over_sum": dc_gbs / read_gbs}}
        log(f"ceiling: bf16 GEMM {gemm_tf:.0f} TFLOP/s; torch copy {copy_gbs:.0f} GB/s, "
            f"torch sum {read_gbs:.0f} GB/s")

    # ---------------- CPU oracle baselines + parity spot-checks on sampled rows
    cpu = None
    parity = None
    if args.cpu_seconds > 0 and not args.step_only:
        import oracle
        threads = oracle.num_threads()

        def host_bits(t):
            return t.cpu().view(torch.int16).numpy().view(np.uint16)

        hosts = []
        for c in layers:
            hosts.append({"q": host_bits(c["q"]), "k": host_bits(c["k"]), "v": host_bits(c["v"]),
                          "out": host_bits(c["out"]), "cu": c["cu_host"],
                          "spans": c["spans_host"],
                          "per_row": np.concatenate([allowed_pairs_per_row(HY_LEN, c["window"],
                                                                           hy_spans[i])
                                                     for i in range(HY_N)])})
        rng = np.random.default_rng(12345)

        def sample(n_per_layer):
            """n rows per layer; returns (CPU seconds, FLOP, per-layer (max-abs, rel, n))."""
            dt, fl, par = 0.0, 0.0, []
            for c, h in zip(layers, hosts):
                T = int(h["cu"][-1])
                rows = np.stack([rng.integers(0, T, n_per_layer),
                                 rng.integers(0, c["hq"], n_per_layer)], 1)
                t = time.perf_counter()
                o = oracle.prefill(h["q"], h["k"], h["v"], h["cu"], window=c["window"],
                                   scale=c["scale"], spans=h["spans"], rows=rows)
                dt += time.perf_counter() - t
                fl += float((4.0 * c["d"] * h["per_row"][rows[:, 0]]).sum())
                bits = h["out"][rows[:, 0], rows[:, 1]]
                got = synth.bf16_to_f32(bits).astype(np.float64)
                err = np.abs(got - o)
                par.append((err.max(), float((err ** 2).sum()), float((o ** 2).sum()),
                            correctly_rounded_share(bits, o)))
            return dt, fl, par

        # rounds of 256 rows per layer until the oracle has run cpu_seconds
        dt = fl = 0.0
        n = 0
        acc = [[0.0, 0.0, 0.0, 0.0] for _ in layers]
        rounds = 0
        while dt < args.cpu_seconds and n < HY_N * HY_LEN * 32:
            d_, f_, par = sample(256)
            dt, fl, n = dt + d_, fl + f_, n + 256
            rounds += 1
            for a, (mx, e2, o2, cr) in zip(acc, par):
                a[0] = max(a[0], mx)
                a[1] += e2
                a[2] += o2
                a[3] += cr
        par = [(a[0], float(np.sqrt(a[1] / a[2])), a[3] / max(rounds, 1)) for a in acc]
        cpu = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{n} seeded (token, head) rows of each of the {nl} hybrid layers "
                         f"({n * nl} rows, {n / (HY_N * HY_LEN * 32):.2%} of each layer), fp64, "
                         f"{dt:.1f} s"}
        log(f"prefill oracle: {n * nl} rows in {dt:.1f} s")
        parity = {"rows_per_layer": n,
                  "layers": [{"max_abs": a, "rel_l2": r, "correctly_rounded": cr}
                             for a, r, cr in par],
                  "max_abs": max(a for a, _, _ in par), "rel_l2": max(r for _, r, _ in par),
                  "correctly_rounded_min": min(cr for _, _, cr in par),
                  "correctly_rounded_note": "share of sampled outputs equal to the bf16 "
                                            "round-to-nearest-even of the fp64 oracle"}
        parity["pass"] = parity["max_abs"] <= 2e-2 and parity["rel_l2"] <= 1e-2

        # decode oracle: the batch-1 decode (sequence 0, whole context) on the host
        L0 = int(dlen[0])
        nb0 = (L0 + 15) // 16
        ids = d_bt[0, :nb0].long()
        kc0 = host_bits(dc["k_cache"].index_select(0, ids))
        vc0 = host_bits(dc["v_cache"].index_select(0, ids))
        q0 = host_bits(dc["q"][:1])
        bt0 = np.arange(nb0, dtype=np.int32)[None]
        t = time.perf_counter()
        od = oracle.decode(q0, kc0, vc0, bt0, np.array([L0], np.int32), scale=dc["scale"])
        ddt = time.perf_counter() - t
        dbits = host_bits(outs[1])
        got = synth.bf16_to_f32(dbits).astype(np.float64)
        cpu["decode"] = {"value": decode_bytes(dlen[:1], 32, 4, 512) / ddt / 1e9, "unit": "GB/s",
                         "cores": threads, "kind": "oracle",
                         "sample": f"the batch-1 decode (context {L0}), fp64, {ddt:.2f} s"}
        parity["decode_batch1"] = {"max_abs": float(np.abs(got - od[0]).max()),
                                   "rel_l2": float(np.linalg.norm(got - od[0])
                                                   / np.linalg.norm(od[0])),
                                   "correctly_rounded": correctly_rounded_share(dbits, od[0])}
        parity["pass"] = parity["pass"] and parity["decode_batch1"]["max_abs"] <= 2e-2 and \
            parity["decode_batch1"]["rel_l2"] <= 1e-2

    rec = {
        "metric": "prefill TFLOP/s + decode HBM GB/s at 1 GPU, bitwise batch-invariant",
        "value": hy_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "hybrid multimodal-style prefill: 5 sliding layers (window 1024, head_dim "
                        "256, 32 query / 16 KV heads) + 1 global layer (head_dim 512, 32 query / "
                        "4 KV heads) over a packed batch of 4 sequences of 4096 tokens, each with "
                        "two bidirectional 256-token spans (seed 5), bf16 N(0,1)*0.5, fp32 "
                        "accumulation; then paged decode, batch 64",
            "tokens": HY_N * HY_LEN,
            "spans": hy_spans,
            "decode_workload": f"paged decode: batch {DB}, contexts U[1024,32768] (seed 4), "
                               "32 query / 4 KV heads, head_dim 512, block 16, shuffled tables",
        },
        "roofline": hy_roof,
        "hybrid_layers": per_layer,
        "decode": {"value": dc_gbs, "unit": "GB/s", "roofline": dc_roof,
                   "context_tokens": int(sum(dlen)),
                   "batch_sweep_llc_flushed": sweep,
                   "seq0_bytes_equal_at_every_batch": bool(invariant),
                   "strict_prefill_bytes": strict,
                   "k_eq_v_llc_flushed": alias},
        **reported,
        "backward": bw,
        "prologue": prologue,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "kernel_sources": kernel_sources_hash(),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

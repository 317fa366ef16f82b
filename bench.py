#!/usr/bin/env python3
"""Benchmark of the batch-invariant attention forward on one MI355X.

One step = one pass of the whole hot path on synthetic inputs resident in
HBM: a packed varlen sliding-window prefill (8 sequences, lengths U[512, 4096],
32 query / 16 KV heads, head dim 256, window 1024, bf16 N(0,1)*0.5), then a
paged-KV decode of 64 sequences (contexts U[1024, 32768], 32 query / 4 KV
heads, head dim 512, 16-token blocks, shuffled block tables, global layer).

Printed: one JSON line.  ``value`` is the prefill's algorithmic TFLOP/s
(4 * head_dim * query_heads * allowed query-key pairs, masked work not
counted) over its HIP-event-timed launches; the decode's algorithmic HBM GB/s
(K and V of every attended context token, plus q, o and block-table reads) is
reported beside it with its own roofline, and the backward (dq, dk, dv) of
the same prefill in a timed region of its own.  The fp64 CPU oracle is timed on a
bounded sample of the same prefill rows on the host cores (reported baseline,
not a target), and its outputs double as a parity spot-check.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# The prefill kernel the benchmark times (head dim 256, group 2): its name in
# rocprofv3 output and the key of its HBM traffic in profiles/traffic.json.
PREFILL_TRAFFIC_KEY = "prefill_ws_kernel<256,2>"
PREFILL_KERNEL_MATCH = "prefill_ws_kernel<invattn::PfWsCfg<256, 2, "
PREFILL_KERNEL_FIRST = "prefill_ws_kernel"
PREFILL_KERNEL_LABEL = "prefill_ws_kernel (head_dim 256, group 2)"


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_attention_flash_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


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


# The backward's two kernels form their five products (and the recomputed
# scores and dP) as bf16 MFMAs, so their roofline is the bf16 matrix peak.
BACKWARD_BOUND = "mfma"
BACKWARD_PEAK = PEAK_BF16_TFLOPS
BACKWARD_KERNEL_LABEL = "bwd_dq_kernel<256> + bwd_dkv_kernel<256> (one launch pair)"

CALIBRATION_BYTES = 1 << 30   # plain streaming kernel used to scale the HBM byte counters


def write_traffic(fetch_dir, write_dir):
    """Turn two rocprofv3 counter runs of `bench.py --calibrate` (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch) into profiles/traffic.json: per-launch
    HBM bytes of the prefill and decode kernels, each counter scaled so the
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
        for key, match, first in ((PREFILL_TRAFFIC_KEY, PREFILL_KERNEL_MATCH, PREFILL_KERNEL_FIRST),
                                  ("decode_chunk_kernel+decode_merge_kernel<512,8>", "decode_",
                                   "decode_chunk_kernel")):
            vals = [v for k, v, g in rows if match in k]
            launches = sum(1 for k, v, g in rows if match in k and first in k)
            if not vals or not launches:
                continue
            per_launch = 1024.0 * scale * sum(vals) / launches
            rec = out.setdefault(key, {"sources_hash": kernel_sources_hash()})
            rec[counter.lower() + "_bytes"] = per_launch
            rec[counter.lower() + "_scale"] = scale
    for rec in out.values():
        rec["bytes_per_launch"] = rec.get("fetch_size_bytes", 0.0) + rec.get("write_size_bytes", 0.0)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed calls of the backward on the prefill workload (0 disables)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample (0 disables)")
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

    # ---------------- inputs (resident in HBM before timing)
    lengths = synth.sliding_lengths(2, 8, 512, 4096)
    HQ, HKV, D, W = 32, 16, 256, 1024
    pf = synth.prefill_case_device(2, lengths, HQ, HKV, D, W, std=0.5, device=dev)
    pf_out = torch.empty_like(pf["q"])
    flops, pairs = prefill_flops(lengths, HQ, D, W)

    DB = args.decode_batch
    dlen = synth.decode_lengths(4, 64, 1024, 32768)[:DB]
    dc = synth.decode_case_device(4, dlen, batch=DB, hq=32, hkv=4, d=512, device=dev)
    d_bt = torch.from_numpy(dc["block_table"]).to(dev)
    d_sl = torch.from_numpy(dc["seq_lens"]).to(dev)
    d_max = int(max(dlen))
    ws = torch.empty(ia.attn_decode_workspace_size(DB, d_max, 32, 512), dtype=torch.uint8,
                     device=dev)
    d_out = torch.empty_like(dc["q"])
    dbytes = decode_bytes(dlen, 32, 4, 512)
    torch.cuda.synchronize()

    def prefill():
        ia.attn_prefill_varlen(pf["q"], pf["k"], pf["v"], pf["cu_seqlens"], pf["max_seqlen"],
                               window=W, softmax_scale=pf["scale"], out=pf_out)

    def decode():
        ia.attn_decode_paged(dc["q"], dc["k_cache"], dc["v_cache"], d_bt, d_sl, d_max,
                             softmax_scale=dc["scale"], workspace=ws, out=d_out)

    if args.calibrate:
        # plain streaming kernel of known traffic: reads and writes 1 GiB
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()   # the library launches on this stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        decode()
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dc_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_step = wall * 1e3 / args.steps

    pf_tflops = flops / (pf_ms * 1e-3) / 1e12

    # ---------------- backward of the same prefill (its own timed region,
    # not part of the step): dq, dk, dv for a seeded upstream gradient
    bw = None
    if args.backward_steps > 0:
        lse = torch.empty(pf["q"].shape[:2], dtype=torch.float32, device=dev)
        ia.attn_prefill_varlen(pf["q"], pf["k"], pf["v"], pf["cu_seqlens"], pf["max_seqlen"],
                               window=W, softmax_scale=pf["scale"], out=pf_out, lse=lse)
        g = torch.from_numpy(synth.upstream_grad(2, tuple(pf["q"].shape)).view(np.int16))
        dout = g.view(torch.bfloat16).to(dev)
        dq = torch.empty(pf["q"].shape, dtype=torch.float32, device=dev)
        dk = torch.empty(pf["k"].shape, dtype=torch.float32, device=dev)
        dv = torch.empty(pf["k"].shape, dtype=torch.float32, device=dev)
        bws = torch.empty(pf["q"].shape[:2], dtype=torch.float32, device=dev)

        def backward():
            ia.attn_prefill_varlen_backward(pf["q"], pf["k"], pf["v"], pf_out, lse, dout,
                                            pf["cu_seqlens"], pf["max_seqlen"], window=W,
                                            softmax_scale=pf["scale"], dq=dq, dk=dk, dv=dv,
                                            workspace=bws)

        backward()
        torch.cuda.synchronize()
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.backward_steps)]
        for e in bev:
            e[0].record(stream)
            backward()
            e[1].record(stream)
        torch.cuda.synchronize()
        bw_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
        bw_flops = 2.5 * flops   # five products of D per allowed pair and head
        bw_tf = bw_flops / (bw_ms * 1e-3) / 1e12
        bw = {"value": bw_tf, "unit": "TFLOP/s", "calls": args.backward_steps,
              "roofline": {"bound": BACKWARD_BOUND, "achieved": bw_tf, "peak": BACKWARD_PEAK,
                           "unit": "TFLOP/s", "frac": bw_tf / BACKWARD_PEAK, "traffic": None,
                           "kernel": BACKWARD_KERNEL_LABEL,
                           "work_per_launch": f"{bw_flops:.4g} FLOP = 10*256*32*{pairs} "
                                              "allowed pairs (dq, dk, dv of the prefill)",
                           "avg_launch_ms": bw_ms}}
        del dq, dk, dv, bws, dout, lse
    dc_gbs = dbytes / (dc_ms * 1e-3) / 1e9

    # ---------------- CPU oracle baseline + parity spot-check on sampled rows
    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        import oracle
        q = pf["q"].cpu().view(torch.int16).numpy().view(np.uint16)
        k = pf["k"].cpu().view(torch.int16).numpy().view(np.uint16)
        v = pf["v"].cpu().view(torch.int16).numpy().view(np.uint16)
        got = pf_out.cpu().view(torch.int16).numpy().view(np.uint16)
        cu = pf["cu_host"]
        T = int(cu[-1])
        per_row = np.concatenate([allowed_pairs_per_row(L, W) for L in lengths])
        rng = np.random.default_rng(12345)
        threads = oracle.num_threads()

        def run(n):
            rows = np.stack([rng.integers(0, T, n), rng.integers(0, HQ, n)], 1)
            t = time.perf_counter()
            o = oracle.prefill(q, k, v, cu, window=W, scale=pf["scale"], rows=rows)
            return rows, o, time.perf_counter() - t

        rows, o, dt = run(512)
        rate = (4.0 * D * per_row[rows[:, 0]]).sum() / max(dt, 1e-6)
        n = int(min(T * HQ, max(512, rate * args.cpu_seconds / (4.0 * D * per_row.mean()))))
        rows, o, dt = run(n)
        cpu_flops = float((4.0 * D * per_row[rows[:, 0]]).sum())
        cpu = {"value": cpu_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{n} seeded (token, head) rows of the same prefill "
                         f"({n / (T * HQ):.1%} of {T * HQ}), fp64, {dt:.1f} s"}
        g = synth.bf16_to_f32(got[rows[:, 0], rows[:, 1]]).astype(np.float64)
        err = float(np.abs(g - o).max())
        rel = float(np.linalg.norm(g - o) / np.linalg.norm(o))
        parity = {"rows": n, "max_abs": err, "rel_l2": rel, "pass": err <= 2e-2 and rel <= 1e-2}

    pf_roof = {"bound": "mfma", "achieved": pf_tflops, "peak": PEAK_BF16_TFLOPS,
               "unit": "TFLOP/s", "frac": pf_tflops / PEAK_BF16_TFLOPS,
               "traffic": load_traffic(PREFILL_TRAFFIC_KEY),
               "kernel": PREFILL_KERNEL_LABEL,
               "work_per_launch": f"{flops:.4g} FLOP = 4*256*32*{pairs} allowed pairs",
               "avg_launch_ms": pf_ms}
    dc_roof = {"bound": "hbm", "achieved": dc_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": dc_gbs / PEAK_HBM_GBS,
               "traffic": load_traffic("decode_chunk_kernel+decode_merge_kernel<512,8>"),
               "kernel": "decode_chunk_kernel + decode_merge_kernel (head_dim 512, group 8)",
               "work_per_launch": f"{dbytes} B: K+V of {sum(dlen)} context tokens x 4 KV heads "
                                  f"x 512 x 2 B x 2, plus q, o, block tables",
               "avg_launch_ms": dc_ms}
    rec = {
        "metric": "prefill TFLOP/s + decode HBM GB/s at 1 GPU, bitwise batch-invariant",
        "value": pf_tflops,
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
            "workload": "sliding-window prefill: packed varlen batch of 8 sequences, lengths "
                        f"U[512,4096] (seed 2: {lengths}), 32 query / 16 KV heads, head_dim 256, "
                        "causal window 1024, bf16 N(0,1)*0.5, fp32 accumulation",
            "tokens": int(sum(lengths)),
            "decode_workload": f"paged decode: batch {DB}, contexts U[1024,32768] (seed 4), "
                               "32 query / 4 KV heads, head_dim 512, block 16, shuffled tables",
        },
        "roofline": pf_roof,
        "decode": {"value": dc_gbs, "unit": "GB/s", "roofline": dc_roof,
                   "context_tokens": int(sum(dlen))},
        "backward": bw,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "kernel_sources": kernel_sources_hash(),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

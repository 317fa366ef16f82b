"""Helpers shared by the GPU tests: moving bf16 bit patterns to and from the
device, running the library, and the parity gate."""
from __future__ import annotations

import numpy as np
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth

ATOL = 2e-2   # max |gpu - oracle|
RTOL = 1e-2   # ||gpu - oracle||_2 / ||oracle||_2


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t_or_bits) -> np.ndarray:
    b = t_or_bits if isinstance(t_or_bits, np.ndarray) else bits(t_or_bits)
    return synth.bf16_to_f32(b).astype(np.float64)


def gate(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else err
    assert err <= ATOL and rel <= RTOL, f"{what}: max-abs {err:.3g} (<= {ATOL}), rel {rel:.3g} (<= {RTOL})"
    return err, rel


def run_prefill(q, k, v, cu, max_seqlen, window, spans=None, scale=None, want_lse=False,
                out=None):
    """q/k/v: numpy bf16 bits or device tensors.  Returns (out tensor, lse tensor|None)."""
    qt = q if isinstance(q, torch.Tensor) else bf16_dev(q)
    kt = k if isinstance(k, torch.Tensor) else bf16_dev(k)
    vt = v if isinstance(v, torch.Tensor) else bf16_dev(v)
    cut = cu if isinstance(cu, torch.Tensor) else i32_dev(cu)
    spt = None
    if spans is not None and len(spans):
        spt = spans if isinstance(spans, torch.Tensor) else i32_dev(np.asarray(spans).reshape(-1, 2))
    lse = torch.empty(qt.shape[0], qt.shape[1], dtype=torch.float32, device=dev()) if want_lse else None
    o = ia.attn_prefill_varlen(qt, kt, vt, cut, max_seqlen, window=window, softmax_scale=scale,
                               spans=spt, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def run_case(case, order=None, max_seqlen=None, want_lse=False):
    q, k, v, cu, sp = case.pack(order)
    ms = case.max_seqlen() if max_seqlen is None else max_seqlen
    o, lse = run_prefill(q, k, v, cu, ms, case.window, sp, case.scale, want_lse)
    return (q, k, v, cu, sp), o, lse


def split_by_seq(out_bits, cu, order):
    """Map packed output rows back to sequence ids: {seq id: bits}."""
    res = {}
    for pos, i in enumerate(order):
        res[i] = out_bits[cu[pos]:cu[pos + 1]]
    return res

"""The attention prologue on the GPU (attn_qk_prologue: RMSNorm over the head
dim, then RoPE, in place on Q and K): parity with the fp64 oracle, exact
special cases, and bitwise invariance of a vector to the batch it runs in.

Sources: the layer prologue of "RFC: Gemma-4-31B-it train/rollout
consistency", section 6 (Q/K RMSNorm at head dims 256 and 512, sliding
RoPE, global proportional RoPE); the norm's fp32 math and single store cast
("Gated RMSNorm CUDA kernel for the GDN block", Summary); a row's bytes do
not depend on other rows (RFC section 4, items 2 and 6)."""
import numpy as np
import pytest
import torch

import invariant_attention_flash_amd as ia
from invariant_attention_flash_amd import synth
import oracle
from gpu_util import bf16_dev, bits, f64, gate, i32_dev

pytestmark = pytest.mark.gpu


def run(c, R, F, theta, norm=True, offset=0.0, with_k=True, eps=synth.PROLOGUE_EPS):
    q = bf16_dev(c.q)
    k = bf16_dev(c.k) if with_k else None
    qw = torch.from_numpy(c.q_weight).to(q.device) if norm else None
    kw = torch.from_numpy(c.k_weight).to(q.device) if norm else None
    ia.attn_qk_prologue(q, k, i32_dev(c.positions), q_weight=qw, k_weight=kw, eps=eps,
                        weight_offset=offset, rotary_dims=R, freq_dims=F, rope_theta=theta)
    torch.cuda.synchronize()
    return q, k


def ref(x, c, w, R, F, theta, norm=True, offset=0.0, eps=synth.PROLOGUE_EPS):
    return oracle.qk_prologue(x, c.positions, weight=w if norm else None, eps=eps, offset=offset,
                              rotary_dims=R, freq_dims=F, theta=theta)


CONFIGS = [
    # (d, hq, hkv, R, F, theta, norm, offset)
    (256, 32, 16, 256, 256, 10000.0, True, 0.0),      # sliding layer: full RoPE
    (512, 32, 4, 128, 512, 1000000.0, True, 0.0),     # global layer: proportional p-RoPE
    (512, 8, 8, 256, 256, 10000.0, True, 1.0),        # plain partial RoPE, offset weight
    (256, 16, 4, 0, 0, 1.0, True, 0.0),               # norm only
    (256, 8, 2, 64, 256, 500000.0, False, 0.0),       # RoPE only
    (64, 4, 4, 64, 64, 10000.0, True, 1.0),
    (64, 8, 2, 2, 64, 10000.0, True, 0.0),            # narrowest rotary width
]


@pytest.mark.parametrize("d,hq,hkv,R,F,theta,norm,offset", CONFIGS)
def test_prologue_parity(d, hq, hkv, R, F, theta, norm, offset):
    c = synth.prologue_case(60 + d, [37, 300, 1], hq, hkv, d, std=1.5,
                            start=[0, 32000, 1 << 20])
    q, k = run(c, R, F, theta, norm, offset)
    gate(f64(q), ref(c.q, c, c.q_weight, R, F, theta, norm, offset), f"q d={d} R={R}")
    gate(f64(k), ref(c.k, c, c.k_weight, R, F, theta, norm, offset), f"k d={d} R={R}")


def test_prologue_q_only_leaves_nothing_else():
    c = synth.prologue_case(71, [64], 8, 4, 256)
    q, _ = run(c, 256, 256, 10000.0, with_k=False)
    gate(f64(q), ref(c.q, c, c.q_weight, 256, 256, 10000.0), "q only")


def test_position_zero_without_norm_is_exact():
    """Turning by angle 0 (c = 1, s = 0) and no norm give the input bytes."""
    c = synth.prologue_case(72, [1, 1, 1], 16, 8, 512)
    c.positions[:] = 0
    q, k = run(c, 512, 512, 10000.0, norm=False)
    assert np.array_equal(bits(q), c.q) and np.array_equal(bits(k), c.k)


def test_unit_weight_gives_unit_rms():
    """With weight 1, no offset, eps 0 and no RoPE, every output vector has
    RMS 1 up to the bf16 rounding of its elements."""
    c = synth.prologue_case(73, [40], 8, 2, 256, std=3.0)
    c.q_weight[:] = 1.0
    c.k_weight[:] = 1.0
    q, k = run(c, 0, 0, 1.0, eps=0.0)
    for t in (q, k):
        rms = np.sqrt(np.mean(f64(t) ** 2, axis=-1))
        assert np.abs(rms - 1.0).max() < 4e-3


def test_vector_bytes_do_not_depend_on_the_batch():
    """A sequence's vectors give the same bytes alone, packed with others at
    another batch position, and with a different number of heads around it
    (only the head count of its own tensor matters)."""
    c = synth.prologue_case(74, [50, 129, 7], 32, 4, 512, start=[5, 900, 30000])
    q_all, k_all = run(c, 128, 512, 1000000.0)
    # the second sequence alone
    lo, hi = 50, 179
    solo = synth.PrologueCase(c.q[lo:hi].copy(), c.k[lo:hi].copy(), c.positions[lo:hi].copy(),
                              c.q_weight, c.k_weight)
    q1, k1 = run(solo, 128, 512, 1000000.0)
    assert np.array_equal(bits(q1), bits(q_all)[lo:hi])
    assert np.array_equal(bits(k1), bits(k_all)[lo:hi])
    # the same sequence packed in front of the others, in reverse order
    order = [1, 2, 0]
    cuts = [(0, 50), (50, 179), (179, 186)]
    perm = np.concatenate([np.arange(*cuts[i]) for i in order])
    shuf = synth.PrologueCase(c.q[perm].copy(), c.k[perm].copy(), c.positions[perm].copy(),
                              c.q_weight, c.k_weight)
    q2, k2 = run(shuf, 128, 512, 1000000.0)
    assert np.array_equal(bits(q2), bits(q_all)[perm])
    assert np.array_equal(bits(k2), bits(k_all)[perm])


def test_hybrid_layer_shapes_full_size():
    """The hybrid prefill's shapes (4 x 4096 tokens): the sliding layer's
    prologue (32/16 heads, head dim 256, full RoPE) and the global layer's
    (32/4 heads, head dim 512, p-RoPE), on sampled tokens against the oracle."""
    for kind, (hq, hkv, d) in (("sliding", (32, 16, 256)), ("global", (32, 4, 512))):
        R, F = synth.prologue_rotary(kind, d)
        th = synth.PROLOGUE_THETA[kind]
        c = synth.prologue_case(75, [4096] * 4, hq, hkv, d, std=0.5)
        q, k = run(c, R, F, th)
        rows = np.random.default_rng(3).choice(c.q.shape[0], 256, replace=False)
        sub = synth.PrologueCase(c.q[rows], c.k[rows], c.positions[rows], c.q_weight,
                                 c.k_weight)
        gate(f64(q)[rows], ref(sub.q, sub, c.q_weight, R, F, th), f"{kind} q")
        gate(f64(k)[rows], ref(sub.k, sub, c.k_weight, R, F, th), f"{kind} k")


def test_empty_input():
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda:0")
    pos = torch.empty((0,), dtype=torch.int32, device="cuda:0")
    ia.attn_qk_prologue(q, None, pos, rotary_dims=64)
    torch.cuda.synchronize()
    assert ia.last_provenance()["op"] == "attn_qk_prologue"

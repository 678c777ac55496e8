"""The seeded workload generators produce the stated structure (CPU only)."""
import numpy as np
import pytest

import oracle
from train_rollout_logprob_amd import synth


def test_tiny_structure():
    c = synth.make_logits_case("tiny")
    assert (c.N, c.V, c.dtype, c.layout) == (128, 1024, "f32", "right")
    att = c.attention.reshape(2, 64)
    assert att[0].sum() == 64 and att[1].sum() == 56
    act = c.action.reshape(2, 64)
    assert act[:, :16].sum() == 0                      # prompt rows never active
    assert act[1, 56:].sum() == 0                      # padding rows never active
    assert 70 <= c.n_active() <= 100
    assert tuple(c.train.shape) == (128, 1024)
    d = (c.train - c.rollout).abs().max().item()
    assert 1e-4 < d < 1e-2
    assert not oracle.validate_inputs(c.attention, c.action, c.ids, c.V, c.N, c.layout, c.B, c.L)


def test_qwen8b_structure_full_host_side():
    c = synth.make_logits_case("qwen8b", generate_logits=False)
    assert (c.B, c.L, c.V, c.layout) == (8, 2048, 151936, "left")
    assert c.n_active() == 8 * 1536
    p = np.array(c.meta["prompt_lengths"])
    assert p.min() >= 256 and p.max() <= 512
    att = c.attention.reshape(8, 2048)
    for b in range(8):
        assert att[b].sum() == 1536 + p[b]
    assert not oracle.validate_inputs(c.attention, c.action, c.ids, c.V, c.N, c.layout, c.B, c.L)


def test_large_structure_full_host_side():
    c = synth.make_logits_case("large", generate_logits=False)
    assert (c.B, c.L, c.N) == (32, 4096, 131072)
    r = np.array(c.meta["response_lengths"])
    assert r.min() >= 1024 and r.max() <= 3072
    assert c.n_active() == int(r.sum())
    assert not oracle.validate_inputs(c.attention, c.action, c.ids, c.V, c.N, c.layout, c.B, c.L)


def test_packed_structure_full_host_side():
    c = synth.make_logits_case("packed", generate_logits=False)
    cu = c.cu_seqlens
    assert cu[0] == 0 and np.all(np.diff(cu) >= 64) and np.all(np.diff(cu) <= 2048)
    assert len(cu) == 257 and c.N == int(cu[-1])
    frac = c.n_active() / c.N
    assert 0.6 < frac < 0.75                           # 3/4 response x 0.9 kept
    assert not oracle.validate_inputs(None, c.action, c.ids, c.V, c.N, "packed",
                                      cu_seqlens=cu)


def test_scaled_variants_and_bf16_rounding():
    import torch
    c = synth.make_logits_case("qwen8b", B=2, L=64, V=1000)
    assert c.train.dtype == torch.bfloat16
    # the selected logit carries the +8 boost on average
    sel = c.rollout.float()[torch.arange(c.N), torch.as_tensor(c.ids, dtype=torch.long)]
    assert sel.mean().item() > 6.0
    c2 = synth.make_logits_case("qwen8b", B=2, L=64, V=1000)
    assert torch.equal(c.train, c2.train)              # seeded


def test_lmhead_small():
    c = synth.make_lmhead_case(T=8, H=32, V=100)
    assert tuple(c.hidden.shape) == (8, 32) and tuple(c.weight.shape) == (32, 100)
    assert 0.01 < c.weight.float().std().item() < 0.03

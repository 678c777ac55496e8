"""Seeded synthetic inputs for the selected-token logprob drift path.

This module only draws random numbers and lays out shapes. It holds none of the
method's arithmetic (no softmax, no log-sum-exp, no statistics), so both the
fp64 CPU oracle and the HIP path can take their inputs from it.

Workloads (the shapes and value distributions of the five scoring workloads):

* ``tiny``    fp32, B=2, L=64 (prompt 16 + response 48), right padding, the second
              sequence has 8 pad rows, V=1024. Rollout ~ N(0, 2^2), train = rollout +
              N(0, 1e-3^2). Action mask Bernoulli(0.9) on response rows.
* ``qwen8b``  bf16, B=8, L=2048 (prompt 512 + response 1536), left padding with prompt
              lengths U{256..512}, V=151936. Rollout ~ N(0, 3^2) with the selected
              logit raised by +8, rounded to bf16; train = bf16(rollout + N(0, 5e-3^2)).
* ``large``   bf16, B=32, L=4096 (prompt 1024 + response U{1024..3072}), right padding,
              V=151936, the ``qwen8b`` value distribution.
* ``packed``  fp32, V=32000, 256 sequences packed by cu_seqlens with lengths
              U{64..2048}; rollout ~ N(0, 2^2), train = rollout + 1e-3 * Student-t(2).
              Prompt = first floor(len/4) rows of a sequence, response = the rest, 10%
              of response rows masked out of the action mask.
* ``lmhead``  hidden [T, 4096] bf16 ~ N(0, 1), W [4096, 151936] bf16 ~ N(0, 0.02^2),
              T = 8 x 2048, every row active.

Host-side structure (lengths, masks, ids) comes from ``numpy.random.default_rng(seed)``;
logits come from a ``torch.Generator`` on the target device, generated in row chunks so
that peak memory stays near the size of the two logits tensors. Seeds default to
``20261202 + workload index``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

WORKLOADS = ("tiny", "qwen8b", "large", "packed", "lmhead")
BASE_SEED = 20261202


def default_seed(name: str) -> int:
    return BASE_SEED + WORKLOADS.index(name)


@dataclass
class LogitsCase:
    """One synthetic scoring batch: both sides' logits plus the logical inputs."""

    name: str
    dtype: str                      # "f32" | "bf16"
    V: int
    N: int                          # rows of the logits tensors
    layout: str                     # "right" | "left" | "packed"
    B: int                          # sequences (packed: number of sequences)
    L: int                          # padded length (packed: 0)
    ids: np.ndarray                 # int32 [N] selected (pre-shifted target) ids
    attention: Optional[np.ndarray]  # uint8 [N] or None (= all ones)
    action: np.ndarray              # uint8 [N]
    cu_seqlens: Optional[np.ndarray] = None  # int32 [B + 1] for packed
    train: object = None            # torch.Tensor [N, V] on the target device
    rollout: object = None
    eps_low: float = 0.2
    eps_high: float = 0.2
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def n_active(self) -> int:
        att = np.ones(self.N, np.uint8) if self.attention is None else self.attention
        act = self.action
        if self.layout == "packed":
            att = att * (np.arange(self.N) < int(self.cu_seqlens[-1])).astype(np.uint8)
        return int(np.count_nonzero((att == 1) & (act == 1)))


@dataclass
class LMHeadCase:
    name: str
    T: int
    H: int
    V: int
    ids: np.ndarray                 # int32 [T]
    hidden: object = None           # torch bf16 [T, H]
    weight: object = None           # torch bf16 [H, V]
    seed: int = 0


# ---------------------------------------------------------------------------
# host-side structure
# ---------------------------------------------------------------------------

def _right_padded(rng, B, L, prompt, resp_lo, resp_hi, action_keep=1.0):
    """prompt rows [0, prompt), response rows [prompt, prompt + r_b), padding after."""
    att = np.zeros((B, L), np.uint8)
    act = np.zeros((B, L), np.uint8)
    resp = rng.integers(resp_lo, resp_hi + 1, size=B)
    for b in range(B):
        r = int(resp[b])
        att[b, : prompt + r] = 1
        if action_keep >= 1.0:
            act[b, prompt: prompt + r] = 1
        else:
            act[b, prompt: prompt + r] = (rng.random(r) < action_keep).astype(np.uint8)
    return att.reshape(-1), act.reshape(-1), resp


def _left_padded(rng, B, L, prompt_slot, prompt_lo, prompt_hi):
    """padding [0, slot - p_b), prompt [slot - p_b, slot), response [slot, L)."""
    att = np.zeros((B, L), np.uint8)
    act = np.zeros((B, L), np.uint8)
    p = rng.integers(prompt_lo, prompt_hi + 1, size=B)
    for b in range(B):
        att[b, prompt_slot - int(p[b]):] = 1
        act[b, prompt_slot:] = 1
    return att.reshape(-1), act.reshape(-1), p


def _packed(rng, nseq, len_lo, len_hi, mask_frac=0.1):
    lens = rng.integers(len_lo, len_hi + 1, size=nseq)
    cu = np.zeros(nseq + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    act = np.zeros(T, np.uint8)
    for s in range(nseq):
        a, ln = int(cu[s]), int(lens[s])
        pr = ln // 4
        keep = (rng.random(ln - pr) >= mask_frac).astype(np.uint8)
        act[a + pr: a + ln] = keep
    return cu.astype(np.int32), act, T


# ---------------------------------------------------------------------------
# logits on the device
# ---------------------------------------------------------------------------

def _chunks(N, V, budget_elems=1 << 28):
    step = max(1, budget_elems // max(V, 1))
    for a in range(0, N, step):
        yield a, min(N, a + step)


def _gen_gauss(torch, N, V, sigma, noise, ids, device, gen, boost=0.0, to_bf16=False,
               noise_kind="normal"):
    """rollout = sigma * z (+ boost at the selected id); train = rollout + noise."""
    dt = torch.bfloat16 if to_bf16 else torch.float32
    roll = torch.empty((N, V), dtype=dt, device=device)
    train = torch.empty((N, V), dtype=dt, device=device)
    ids_t = torch.as_tensor(ids.astype(np.int64), device=device)
    for a, b in _chunks(N, V):
        x = torch.randn((b - a, V), generator=gen, device=device, dtype=torch.float32)
        x.mul_(sigma)
        if boost:
            sel = ids_t[a:b].clamp(0, V - 1)
            x.scatter_add_(1, sel[:, None],
                           torch.full((b - a, 1), boost, device=device, dtype=torch.float32))
        if to_bf16:
            xr = x.to(torch.bfloat16)
            roll[a:b] = xr
            base = xr.to(torch.float32)
        else:
            roll[a:b] = x
            base = x
        if noise_kind == "normal":
            e = torch.randn((b - a, V), generator=gen, device=device, dtype=torch.float32)
        else:  # Student-t with 2 degrees of freedom: z / sqrt(Exp(1))
            z = torch.randn((b - a, V), generator=gen, device=device, dtype=torch.float32)
            w = torch.empty((b - a, V), device=device, dtype=torch.float32)
            w.exponential_(1.0, generator=gen)
            e = z / torch.sqrt(w)
            del z, w
        e.mul_(noise).add_(base)
        train[a:b] = e.to(dt)
        del x, e, base
    return train, roll


def make_logits_case(name: str, device="cpu", seed: Optional[int] = None, *,
                     B=None, L=None, V=None, prompt=None, nseq=None, len_lo=None,
                     len_hi=None, generate_logits=True, large_reading="qwen8b") -> LogitsCase:
    """Build one scoring batch. Keyword overrides give scaled-down variants of a
    workload with the same structure (used by the parity tests)."""
    import torch

    seed = default_seed(name) if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    if name == "tiny":
        B = B or 2
        L = L or 64
        V = V or 1024
        prompt = prompt or 16
        pad_last = 8 if L == 64 else max(1, L // 8)
        att = np.ones((B, L), np.uint8)
        att[B - 1, L - pad_last:] = 0
        act = np.zeros((B, L), np.uint8)
        for b in range(B):
            real = int(att[b].sum())
            act[b, prompt:real] = (rng.random(real - prompt) < 0.9).astype(np.uint8)
        att, act = att.reshape(-1), act.reshape(-1)
        N = B * L
        ids = rng.integers(0, V, size=N).astype(np.int32)
        case = LogitsCase(name, "f32", V, N, "right", B, L, ids, att, act, seed=seed)
        if generate_logits:
            case.train, case.rollout = _gen_gauss(torch, N, V, 2.0, 1e-3, ids, device, gen)
        return case

    if name == "qwen8b":
        B = B or 8
        L = L or 2048
        V = V or 151936
        slot = prompt or (L // 4)
        att, act, p = _left_padded(rng, B, L, slot, slot // 2, slot)
        N = B * L
        ids = rng.integers(0, V, size=N).astype(np.int32)
        case = LogitsCase(name, "bf16", V, N, "left", B, L, ids, att, act, seed=seed,
                          meta={"prompt_lengths": p.tolist()})
        if generate_logits:
            case.train, case.rollout = _gen_gauss(torch, N, V, 3.0, 5e-3, ids, device, gen,
                                                  boost=8.0, to_bf16=True)
        return case

    if name == "large":
        B = B or 32
        L = L or 4096
        V = V or 151936
        prompt = prompt or (L // 4)
        att, act, r = _right_padded(rng, B, L, prompt, prompt, L - prompt)
        N = B * L
        ids = rng.integers(0, V, size=N).astype(np.int32)
        case = LogitsCase(name, "bf16", V, N, "right", B, L, ids, att, act, seed=seed,
                          meta={"response_lengths": r.tolist(), "reading": large_reading})
        if generate_logits:
            if large_reading == "qwen8b":
                case.train, case.rollout = _gen_gauss(torch, N, V, 3.0, 5e-3, ids, device, gen,
                                                      boost=8.0, to_bf16=True)
            else:  # the tiny workload's distribution, rounded to bf16
                case.train, case.rollout = _gen_gauss(torch, N, V, 2.0, 1e-3, ids, device, gen,
                                                      to_bf16=True)
        return case

    if name == "packed":
        V = V or 32000
        nseq = nseq or 256
        len_lo = len_lo or 64
        len_hi = len_hi or 2048
        cu, act, T = _packed(rng, nseq, len_lo, len_hi)
        ids = rng.integers(0, V, size=T).astype(np.int32)
        case = LogitsCase(name, "f32", V, T, "packed", nseq, 0, ids, None, act,
                          cu_seqlens=cu, seed=seed)
        if generate_logits:
            case.train, case.rollout = _gen_gauss(torch, T, V, 2.0, 1e-3, ids, device, gen,
                                                  noise_kind="student_t2")
        return case

    raise ValueError(f"unknown logits workload {name!r}")


def make_lmhead_case(device="cpu", seed: Optional[int] = None, *, T=16384, H=4096,
                     V=151936, generate=True) -> LMHeadCase:
    import torch

    seed = default_seed("lmhead") if seed is None else seed
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, V, size=T).astype(np.int32)
    case = LMHeadCase("lmhead", T, H, V, ids, seed=seed)
    if generate:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        hid = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        for a, b in _chunks(T, H):
            hid[a:b] = torch.randn((b - a, H), generator=gen, device=device).to(torch.bfloat16)
        w = torch.empty((H, V), dtype=torch.bfloat16, device=device)
        for a, b in _chunks(H, V):
            w[a:b] = (torch.randn((b - a, V), generator=gen, device=device) * 0.02).to(torch.bfloat16)
        case.hidden, case.weight = hid, w
    return case


def rows_to_host(t, rows) -> np.ndarray:
    """Copy selected rows of a device logits tensor to host as the raw storage type
    (float32, or uint16 bit patterns for bf16)."""
    import torch

    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
    sub = t.index_select(0, idx).cpu()
    if sub.dtype == torch.bfloat16:
        return sub.view(torch.int16).numpy().view(np.uint16)
    return sub.numpy()

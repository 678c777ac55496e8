"""Shared helpers of the GPU tests: run the library on a synthetic batch, and run the
oracle on the same inputs copied to the host."""
import math

import numpy as np
import torch

import oracle
from train_rollout_logprob_amd import synth

LOGP_TOL = 2e-5          # per-token |logp_gpu - logp_fp64|
MEAN_RTOL = 1e-5         # aggregate means, relative


def gpu_available():
    return torch.cuda.is_available()


_POOL = None


def start_oracle_pool():
    """Starts the oracle's host worker pool (called at test-session start, before any test
    touches the GPU)."""
    global _POOL
    if _POOL is None:
        from oracle.pool import OraclePool
        _POOL = OraclePool()


def stop_oracle_pool():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL = None


def oracle_pool():
    """The session's oracle worker pool, or None if it was not started."""
    return _POOL


def device_inputs(case, dev="cuda"):
    ids = torch.as_tensor(case.ids, device=dev)
    att = torch.as_tensor(case.attention, device=dev) if case.attention is not None else None
    act = torch.as_tensor(case.action, device=dev) if case.action is not None else None
    cu = torch.as_tensor(case.cu_seqlens, device=dev) if case.cu_seqlens is not None else None
    return ids, att, act, cu


def run_library(case, dev="cuda", ids_dtype=None, train=None, rollout=None, **kw):
    from train_rollout_logprob_amd import binding as B
    ids, att, act, cu = device_inputs(case, dev)
    if ids_dtype is not None:
        ids = ids.to(ids_dtype)
    tr = case.train if train is None else train
    ro = case.rollout if rollout is None else rollout
    t, r, d, a, ws = B.selected_logprob(tr, ro, ids, att, act, case.layout, case.B, case.L, cu,
                                        **kw)
    st, bad = B.drift_get_status(ws)
    return {"train_logp": t.cpu().numpy(), "rollout_logp": r.cpu().numpy(),
            "dlogp": d.cpu().numpy(), "active": a.cpu().numpy(), "status": st,
            "first_bad": bad, "ws": ws, "d_dev": d, "a_dev": a}


def host_logits(t):
    """Whole logits tensor to host as float32 or bf16 bit patterns."""
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_oracle(case, train=None, rollout=None):
    tr = host_logits(case.train if train is None else train)
    ro = host_logits(case.rollout if rollout is None else rollout)
    return oracle.selected_logprob(tr, ro, case.dtype, case.ids, case.attention, case.action,
                                   case.V, case.layout, case.B, case.L, case.cu_seqlens)


def status_name(code):
    from train_rollout_logprob_amd import binding as B
    return B.STATUS_NAMES[code]


def assert_logprob_parity(got, want, tol=LOGP_TOL):
    assert np.array_equal(got["active"], want["active"])
    act = want["active"] == 1
    for k in ("train_logp", "rollout_logp", "dlogp"):
        g = got[k].astype(np.float64)
        w = want[k]
        assert np.all(g[~act] == 0.0), k
        err = np.abs(g[act] - w[act])
        assert err.size == 0 or float(err.max()) <= tol, (k, float(err.max()))


# Gate A (the library's statistics of an array against the oracle's statistics of the same
# array): both sides sum the same fp64 terms, the oracle exactly rounded (math.fsum), the
# library in a fixed tree. A tree whose longest chain has D additions is within D * 2^-53
# of the exact sum relative to the sum of |terms|; the library's chains stay below a few
# hundred additions at the sizes tested (1024-row tiles, 64 lanes per fold; a segment's
# thread takes at most ~400 rows), so 1e-12 leaves a margin of more than 20. The per-term
# functions differ by at most an ulp on each side: exp(d) is then within 4 * 2^-53
# relative; expm1(d) - d, which cancels, within 4 * 2^-53 * |expm1(d)| absolute, and
# |expm1(d)| <= |d| * e^|d|, whence the absolute term on approx_kl0.
GATE_A_RTOL = 1e-12


def assert_stats_exact(got, want):
    """Gate A. Counts, order statistics and argmax bit-exact; clipfrac0 too (the same
    counts divided by the same n); means to GATE_A_RTOL relative (mean_dlogp and
    mismatch_kl, which sit near 0, relative to mean |d|; approx_kl0 with the absolute term
    above)."""
    for k in ("n_active", "n_clip_low", "n_clip_high", "n_nonfinite", "argmax_row"):
        assert got[k] == want[k], (k, got[k], want[k])
    for k in ("p95_abs_dlogp", "p99_abs_dlogp", "max_abs_dlogp"):
        g, w = got[k], want[k]
        assert (np.isnan(g) and np.isnan(w)) or np.float32(g) == np.float32(w), (k, g, w)
    for k in ("ratio0", "clipfrac0", "approx_kl0", "mean_abs_dlogp"):
        g, w = got[k], want[k]
        if np.isnan(w):
            assert np.isnan(g), k
        elif k == "clipfrac0":
            assert g == w, (k, g, w)
        else:
            tol = GATE_A_RTOL * abs(w) + 1e-300
            if k == "approx_kl0":
                tol += 4.5e-16 * math.exp(min(want["max_abs_dlogp"], 700.0)) * want["mean_abs_dlogp"]
            assert abs(g - w) <= tol, (k, g, w)
    for k in ("mean_dlogp", "mismatch_kl"):
        g, w = got[k], want[k]
        if not np.isnan(w):
            assert abs(g - w) <= GATE_A_RTOL * max(abs(w), want["mean_abs_dlogp"]), (k, g, w)


def small_variants():
    """Scaled-down versions of the scoring workloads: several tiles, ragged tails, every
    layout and dtype."""
    return {
        "tiny": dict(name="tiny"),
        "qwen8b_small": dict(name="qwen8b", B=3, L=96),
        "large_small": dict(name="large", B=4, L=64),
        "packed_small": dict(name="packed", nseq=6, len_lo=64, len_hi=300),
        "bf16_ragged_V": dict(name="qwen8b", B=2, L=32, V=1001),
        "f32_ragged_V": dict(name="packed", nseq=3, len_lo=20, len_hi=60, V=4099),
        "f32_V37": dict(name="tiny", B=2, L=16, V=37, prompt=4),
        "bf16_V8": dict(name="large", B=2, L=16, V=8, prompt=4),
    }


def make_small(spec, dev="cuda"):
    spec = dict(spec)
    name = spec.pop("name")
    return synth.make_logits_case(name, device=dev, **spec)


def assert_gate_b(got, want, d_oracle_active, eps_low=0.2, eps_high=0.2, tol=LOGP_TOL):
    """Gate B: the library's statistics of its fp32 dlogp against the oracle's statistics of
    its own fp64 dlogp. Means to MEAN_RTOL relative (mean_dlogp and mismatch_kl, which sit
    near 0, to MEAN_RTOL of mean |d|). Each GPU dlogp is within `tol` of the oracle's, so an
    order statistic of |d| is too, and a clip decision can differ only for rows within
    `tol` of a clip edge: the clip counts may differ by at most the number of such rows,
    and the worst row must match when its lead over the runner-up exceeds 2 tol."""
    assert got["n_active"] == want["n_active"]
    assert got["n_nonfinite"] == want["n_nonfinite"] == 0
    for k in ("ratio0", "approx_kl0", "mean_abs_dlogp"):
        g, w = got[k], want[k]
        assert abs(g - w) <= MEAN_RTOL * abs(w), (k, g, w)
    for k in ("mean_dlogp", "mismatch_kl"):
        g, w = got[k], want[k]
        assert abs(g - w) <= MEAN_RTOL * want["mean_abs_dlogp"], (k, g, w)
    d = np.asarray(d_oracle_active, dtype=np.float64)
    near_lo = int((np.abs(d - math.log1p(-eps_low)) <= tol).sum())
    near_hi = int((np.abs(d - math.log1p(eps_high)) <= tol).sum())
    assert abs(got["n_clip_low"] - want["n_clip_low"]) <= near_lo
    assert abs(got["n_clip_high"] - want["n_clip_high"]) <= near_hi
    n_clip = got["n_clip_low"] + got["n_clip_high"]
    assert abs(got["clipfrac0"] - n_clip / got["n_active"]) <= 1e-15
    for k in ("p95_abs_dlogp", "p99_abs_dlogp", "max_abs_dlogp"):
        assert abs(got[k] - want[k]) <= tol, (k, got[k], want[k])
    a = np.sort(np.abs(d))
    if len(a) > 1 and a[-1] - a[-2] > 2 * tol:
        assert got["argmax_row"] == want["argmax_row"]


FULL_CHUNK_BYTES = 2 << 30  # rows of both sides copied to the host per round (full sizes)


def copy_rows(dst, src, idx):
    """Rows `idx` of a device tensor into a host array of the stored type (bf16 as bits)."""
    sub = src.index_select(0, idx)
    if sub.dtype == torch.bfloat16:
        torch.from_numpy(dst.view(np.int16)).copy_(sub.view(torch.int16))
    else:
        torch.from_numpy(dst).copy_(sub)


def oracle_all_rows(pool, case, rows, transforms=(None, None)):
    """Oracle logps and dlogp (float64, [3, len(rows)]) of the given rows of a case whose
    logits are on the GPU, scored in the worker pool chunk by chunk."""
    per = max(1, FULL_CHUNK_BYTES // (2 * case.V * case.elem_bytes))
    per = min(per, len(rows))
    out = np.empty((3, len(rows)))
    for a in range(0, len(rows), per):
        sel = rows[a:a + per]
        bt, br = pool.buffers(per, case.V, case.dtype)
        idx = torch.as_tensor(sel, device=case.train.device)
        copy_rows(bt[:len(sel)], case.train, idx)
        copy_rows(br[:len(sel)], case.rollout, idx)
        t, r, d, _ = pool.score(len(sel), case.V, case.dtype, case.ids[sel],
                                transforms=transforms)
        out[:, a:a + len(sel)] = (t, r, d)
    return out

"""Throughput of the paired selected-token logprob + drift path on one MI355X.

One step = drift_selected_logprob (classification, paired one-pass log-softmax gather of
both sides, drift) + drift_diagnostics_async (sums, counts, exact nearest-rank select; the
statistics written into pinned host memory) over one batch, inputs resident in HBM before
timing starts. Steps run two deep: a step's diagnostics run on a second stream beside the
next step's scoring pass, and the host waits for step i and checks its statistics while
step i + 1 runs; the last step is collected before the clock stops.

The main line is the large-batch workload, the largest that fits one GPU: bf16 logits,
V=151936, B=32, L=4096 (prompt 1024 + response U[1024,3072]), right padding, about 40 GB
of logits per side. `roofline` is for its dominant kernel, the paired scoring kernel:
algorithmic bytes = active rows x V x 2 bytes x 2 sides, divided by the kernel's duration
measured with HIP events the library records around it on the launch stream (average,
median and min over the timed steps). `cpu_baseline` is the fp64 CPU oracle timed on a
pool of host worker processes over a bounded sample of the same batch's active rows.

`configs` carries the same measurement for the other scoring workloads, each generated
after the previous one is freed: the Qwen3-8B-shaped batch (bf16, B=8, L=2048, left
padding), the packed varlen batch (fp32, V=32000, 256 sequences by cu_seqlens) and the
tiny correctness batch (fp32, V=1024). Further legs are measured outside the timed region:
`segments` and `active_rows` on the main batch; `training` (entropy + LSE from the scoring
pass, dlogits), `exact` (order-independent reduction, unsharded and as vocabulary shards)
and `transforms` (temperature and soft-cap chains) on the Qwen3-8B-shaped batch; `lmhead`,
the fused LM-head selected logprob.
"""
import argparse
import collections
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "active tokens/sec + logits HBM GB/s (% of peak) for paired logprob+drift"
WORKLOAD_TEXT = {
    "qwen8b": "qwen8b-shaped paired scoring: bf16 logits, V=151936, B=8, L=2048 "
              "(prompt 512 + response 1536), left padding",
    "large": "large-batch paired scoring: bf16 logits, V=151936, B=32, L=4096 "
             "(prompt 1024 + response U[1024,3072]), right padding",
    "packed": "packed varlen paired scoring: fp32 logits, V=32000, 256 sequences "
              "U[64,2048] via cu_seqlens, Student-t(2) drift",
    "tiny": "tiny paired scoring: fp32 logits, V=1024, B=2, L=64, right padding",
}
# legs measured beside the main line (outside its timed region)
LEGS = ("segments", "configs", "training", "exact", "transforms", "lmhead")
# the other scoring workloads measured beside the main one, in this order
OTHER_CONFIGS = {"large": ("qwen8b", "packed", "tiny"), "qwen8b": ("large", "packed", "tiny"),
                 "packed": ("large", "qwen8b", "tiny"), "tiny": ("large", "qwen8b", "packed")}


SCORE_SOURCES = ("logprob.hip", "classify.h", "lse.h", "rowio.h", "common.h:score")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "score_rows_bf16_qwen8b.md")
SCORE_PROFILES = {"qwen8b": TRAFFIC_PROFILE,
                  "large": os.path.join(ROOT, "profiles", "score_rows_bf16_large.md"),
                  "packed": os.path.join(ROOT, "profiles", "score_rows_f32_packed.md")}
DLOGITS_SOURCES = ("dlogits.hip", "classify.h", "rowio.h", "common.h:score",
                   "common.h:dlogits")
DLOGITS_PROFILE = os.path.join(ROOT, "profiles", "dlogits_rows_bf16_qwen8b.md")


def _source_text(name):
    """A source file of the library, or the part of common.h that a kernel compiles
    against ("common.h:score": everything up to the scoring launcher's declaration;
    "common.h:dlogits": the dlogits parameter block)."""
    fname, _, part = name.partition(":")
    with open(os.path.join(ROOT, "train_rollout_logprob_amd", "csrc", fname), "rb") as fh:
        text = fh.read()
    if part == "score":
        end = text.index(b"hipError_t launch_score(")
        return text[:end]
    if part == "dlogits":
        start = text.index(b"struct DlogitsParams {")
        return text[start:text.index(b"hipError_t launch_dlogits(", start)]
    return text


def source_hash(files=SCORE_SOURCES):
    """Hash of a kernel's sources, to tie a recorded counter reading to them."""
    import hashlib

    h = hashlib.sha256()
    for f in files:
        h.update(_source_text(f))
    return h.hexdigest()[:16]


def score_source_hash():
    return source_hash(SCORE_SOURCES)


def recorded_traffic(profile=TRAFFIC_PROFILE, files=SCORE_SOURCES):
    """HBM bytes per launch of a kernel from its committed PMC summary (FETCH_SIZE +
    WRITE_SIZE, calibrated on a copy of known size), or None when the kernel's sources
    changed since the counters were taken."""
    try:
        vals = {}
        with open(profile) as fh:
            for line in fh:
                if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch",
                                                          "traffic_sources"):
                    k, v = line.split(":", 1)
                    vals[k] = v.strip()
        if vals.get("traffic_sources") != source_hash(files):
            return None
        return float(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def read_ceiling(case, reps=10, warmup=2):
    """Pure-read rate (GB/s) of the same logits tensors with the scoring kernels' access
    pattern: every row pair, one block per pair, 16-byte nontemporal loads
    (libdrift_ceiling.so, measurement only). HIP events on the launch stream, median."""
    import torch

    from train_rollout_logprob_amd import build as Bd

    if not os.path.exists(Bd.CEILING_LIB):
        raise RuntimeError(f"{Bd.CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(Bd.CEILING_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.drift_read_ceiling.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.drift_read_ceiling.restype = ctypes.c_int
    esz = case.train.element_size()
    rows = case.train.shape[0]
    row_bytes = case.train.shape[1] * esz // 16 * 16
    stride = case.train.stride(0) * esz
    sink = torch.empty(rows * 4, dtype=torch.int32, device=case.train.device)
    stream = torch.cuda.current_stream()

    def call():
        st = lib.drift_read_ceiling(case.train.data_ptr(), case.rollout.data_ptr(), rows,
                                    row_bytes, stride, sink.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"drift_read_ceiling: status {st}")

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    return 2 * rows * row_bytes / (ms * 1e-3) / 1e9, ms


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_sample(pool, case, max_rows=16384):
    """Copies a bounded sample of the batch's active rows (every k-th active row, in
    order) of both sides into the oracle pool's shared host buffer, outside any timing."""
    import numpy as np

    from train_rollout_logprob_amd import synth

    att = case.attention if case.attention is not None else np.ones(case.N, np.uint8)
    live = (att != 0) & (case.action != 0)
    if case.cu_seqlens is not None:
        live &= np.arange(case.N) < int(case.cu_seqlens[-1])
    rows = np.nonzero(live)[0]
    step = max(1, -(-len(rows) // max_rows))
    sel = rows[::step][:max_rows]
    tr, ro = pool.buffers(len(sel), case.V, case.dtype)
    for a in range(0, len(sel), 1024):
        part = sel[a:a + 1024]
        tr[a:a + len(part)] = synth.rows_to_host(case.train, part)
        ro[a:a + len(part)] = synth.rows_to_host(case.rollout, part)
    return {"rows": len(sel), "every": step, "of": len(rows), "V": case.V,
            "dtype": case.dtype, "ids": case.ids[sel]}


def cpu_baseline(pool, sample, budget_s):
    """The fp64 oracle (textbook two-pass log-sum-exp, both sides, dlogp) on a pool of host
    worker processes over the sampled rows, repeated until `budget_s` seconds of wall time
    are spent; rows scored per second of the pool's wall time."""
    n, V, dt = sample["rows"], sample["V"], sample["dtype"]
    done, spent, passes = 0, 0.0, 0
    while spent < budget_s or passes == 0:
        _, _, _, wall = pool.score(n, V, dt, sample["ids"])
        spent += wall
        done += n
        passes += 1
    return {"value": done / spent, "unit": "active tokens/s", "cores": pool.workers,
            "kind": "oracle",
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} active rows of the main batch (every {sample['every']}th of "
                      f"{sample['of']}, both sides, V={V}, {dt}), scored {passes} times by "
                      f"numpy fp64 two-pass log-sum-exp in {pool.workers} worker processes; "
                      f"{spent:.1f} s of pool wall time"}


def lmhead_leg(steps=5, warmup=2):
    """Fused LM-head workload (hidden [16384, 4096] x W [4096, 151936], bf16): the whole
    drift_lmhead_logprob call timed with events on the launch stream, the [V, H] weight
    layout with and without a soft-cap on the logits; beside it, for context, the vendor
    library's plain GEMM of the same shape (logits written out)."""
    import torch

    from train_rollout_logprob_amd import binding as B
    from train_rollout_logprob_amd import synth

    case = synth.make_lmhead_case(device="cuda:0")
    ids = torch.as_tensor(case.ids, device="cuda:0")
    ws = B.workspace(B.DRIFT_OP_LMHEAD, case.T, case.V, B.DRIFT_BF16, "cuda:0",
                     hidden_dim=case.H)
    lp = torch.empty(case.T, dtype=torch.float32, device="cuda:0")
    for _ in range(warmup):
        B.lmhead_logprob(case.hidden, case.weight, ids, ws=ws, out=lp)
    st, _ = B.drift_get_status(ws)
    if st != B.DRIFT_OK:
        raise RuntimeError(f"lmhead status {B.STATUS_NAMES[st]}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        B.lmhead_logprob(case.hidden, case.weight, ids, ws=ws, out=lp)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 2.0 * case.T * case.H * case.V
    tflops = flop / (ms * 1e-3) / 1e12
    out = {"workload": f"fused LM-head: hidden [{case.T}, {case.H}] x W [{case.H}, {case.V}] "
                       f"bf16, fp32 accumulation", "ms_per_call": ms,
           "active_tokens_per_s": case.T / (ms * 1e-3), "tflops": tflops,
           "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
           "flop_per_call": flop}
    del ws
    torch.cuda.empty_cache()
    # the same call with the weight kept as [V, H] (a linear layer's layout; read in place,
    # no per-call transpose), bitwise the same outputs
    w_vh = case.weight.t().contiguous()
    ws = B.workspace(B.DRIFT_OP_LMHEAD_VH, case.T, case.V, B.DRIFT_BF16, "cuda:0",
                     hidden_dim=case.H)
    out_vh = torch.empty_like(lp)
    for _ in range(warmup):
        B.lmhead_logprob(case.hidden, w_vh, ids, ws=ws, out=out_vh, weight_layout="vh")
    e0.record()
    for _ in range(steps):
        B.lmhead_logprob(case.hidden, w_vh, ids, ws=ws, out=out_vh, weight_layout="vh")
    e1.record()
    torch.cuda.synchronize()
    vh_ms = e0.elapsed_time(e1) / steps
    out["weight_vh"] = {"what": "drift_lmhead_logprob_vh: W given as [V, H], read in place",
                        "ms_per_call": vh_ms, "tflops": flop / (vh_ms * 1e-3) / 1e12,
                        "frac": flop / (vh_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                        "bitwise_equal_to_hv": bool(torch.equal(out_vh.view(torch.int32),
                                                                lp.view(torch.int32)))}
    # the same [V, H] call with a soft-cap of 30 on the head's logits
    # (drift_lmhead_logprob_chain; the cap is folded into the epilogue)
    chain = [("softcap", 30.0)]
    for _ in range(warmup):
        B.lmhead_logprob(case.hidden, w_vh, ids, ws=ws, out=out_vh, weight_layout="vh",
                         transforms=chain)
    e0.record()
    for _ in range(steps):
        B.lmhead_logprob(case.hidden, w_vh, ids, ws=ws, out=out_vh, weight_layout="vh",
                         transforms=chain)
    e1.record()
    torch.cuda.synchronize()
    st, _ = B.drift_get_status(ws)
    if st != B.DRIFT_OK:
        raise RuntimeError(f"lmhead with a soft-cap: status {B.STATUS_NAMES[st]}")
    cap_ms = e0.elapsed_time(e1) / steps
    out["weight_vh_softcap"] = {"what": "drift_lmhead_logprob_chain, W as [V, H], soft-cap 30 "
                                        "on the logits", "ms_per_call": cap_ms,
                                "tflops": flop / (cap_ms * 1e-3) / 1e12,
                                "frac": flop / (cap_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    del ws, w_vh
    torch.cuda.empty_cache()
    # context, not the product path: the plain bf16 GEMM of the same shape through the
    # vendor library (torch.matmul -> hipBLASLt), which writes the logits instead of
    # reducing them, timed the same way on the same box
    z = torch.empty((case.T, case.V), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(warmup):
        torch.matmul(case.hidden, case.weight, out=z)
    e0.record()
    for _ in range(steps):
        torch.matmul(case.hidden, case.weight, out=z)
    e1.record()
    torch.cuda.synchronize()
    ref_ms = e0.elapsed_time(e1) / steps
    out["plain_gemm_reference"] = {"what": "torch.matmul bf16 of the same shape (hipBLASLt), "
                                           "logits written to HBM", "ms_per_call": ref_ms,
                                   "tflops": flop / (ref_ms * 1e-3) / 1e12}
    return out


def segments_leg(case, d, active, logprob_ws, steps=20):
    """Per-sequence statistics of the timed batch (drift_segment_diagnostics): one segment
    per sequence (batch row, or packed sequence by cu_seqlens); events around `steps`
    asynchronous calls on the launch stream."""
    import torch

    from train_rollout_logprob_amd import binding as B

    dev = d.device
    if case.cu_seqlens is not None:
        offs = torch.as_tensor(case.cu_seqlens, dtype=torch.int32, device=dev)
    else:
        offs = torch.arange(case.B + 1, dtype=torch.int32, device=dev) * case.L
    S = offs.numel() - 1
    out = torch.empty(S * ctypes.sizeof(B.drift_stats), dtype=torch.uint8, device=dev)
    call = (lambda: B.drift_segment_diagnostics(d, active, case.N, offs, S, case.eps_low,
                                                case.eps_high, logprob_ws, out))
    for _ in range(3):
        assert call() == B.DRIFT_OK
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    worst = max(B.segment_diagnostics(d, active, offs, case.eps_low, case.eps_high),
                key=lambda s_: s_["max_abs_dlogp"])
    return {"kernel": "diag_segments", "segments": S, "us_per_call": us,
            "rows_per_s": case.N / (us * 1e-6),
            "worst_segment": {"argmax_row": worst["argmax_row"],
                              "max_abs_dlogp": worst["max_abs_dlogp"]}}


def active_rows_leg(case, active, steps=20):
    """The ascending active-row list of the timed batch (drift_active_rows, two small
    launches): events around `steps` asynchronous calls on the launch stream."""
    import torch

    from train_rollout_logprob_amd import binding as B

    rows, n, ws = B.active_rows(active)
    call = (lambda: B.drift_active_rows(active, case.N, rows, n, ws, ws.numel()))
    for _ in range(3):
        assert call() == B.DRIFT_OK
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    return {"kernels": "compact_count + compact_scatter", "n_active": int(n.item()),
            "us_per_call": us, "rows_per_s": case.N / (us * 1e-6)}


def exact_leg(case, ids, att, act, cu, shards=8, steps=10, warmup=2):
    """Order-independent (exact) reduction on the same batch: the unsharded exact scoring
    kernel, then the batch split into `shards` vocabulary shards (column views, as
    tensor-parallel ranks hold them): per-shard partial kernels plus the shard-order merge,
    whose outputs are checked bitwise against the unsharded exact call."""
    import torch

    from train_rollout_logprob_amd import binding as B

    dev = case.train.device
    N, V, esz = case.N, case.V, case.elem_bytes
    n_active = case.n_active()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    out = None
    for i in range(warmup + steps):
        evs = (ev[2 * (i - warmup)].cuda_event, ev[2 * (i - warmup) + 1].cuda_event) \
            if i >= warmup else None
        out = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout, case.B,
                                 case.L, cu, ws=out[4] if out else None,
                                 out=out[:4] if out else None, events=evs, reduction="exact")
    torch.cuda.synchronize()
    st, _ = B.drift_get_status(out[4])
    if st != B.DRIFT_OK:
        raise RuntimeError(f"exact scoring: status {B.STATUS_NAMES[st]}")
    ex_all = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    ex_ms = sum(ex_all) / steps
    ex_bytes = n_active * V * esz * 2
    width = (V // shards) // 8 * 8
    bounds = [width * s for s in range(shards)] + [V]
    nb = N * ctypes.sizeof(B.drift_lse_partial)
    tparts = torch.empty(shards * nb, dtype=torch.uint8, device=dev)
    rparts = torch.empty(shards * nb, dtype=torch.uint8, device=dev)
    wss = [B.workspace(B.DRIFT_OP_SELECTED_LOGPROB, N, 1, B.DRIFT_BF16, dev) for _ in range(shards)]
    args = [B.make_args(case.train[:, bounds[s]:bounds[s + 1]],
                        case.rollout[:, bounds[s]:bounds[s + 1]], ids, att, act, case.layout,
                        case.B, case.L, cu) for s in range(shards)]

    def sharded():
        for s in range(shards):
            assert B.drift_shard_partials(args[s], bounds[s], V, tparts[s * nb:],
                                          rparts[s * nb:], wss[s], wss[s].numel()) == B.DRIFT_OK
        return B.merge_shards(tparts, rparts, bounds, ids, V, N, att, act, case.layout, case.B,
                              case.L, cu)

    for _ in range(warmup):
        res = sharded()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        res = sharded()
    e1.record()
    torch.cuda.synchronize()
    sh_ms = e0.elapsed_time(e1) / steps
    same = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
               for a, b in zip(res[:3], out[:3]))
    return {
        "workload": f"same batch; exact reduction unsharded, then {shards} vocabulary shards "
                    f"of {width} columns (column views) + shard-order merge",
        "exact": {"kernel": f"score_rows_exact<{case.dtype}>", "kernel_ms": ex_ms,
                  "kernel_ms_median": ex_all[steps // 2], "kernel_ms_min": ex_all[0],
                  "bytes_per_launch": ex_bytes,
                  "achieved_gbs": ex_bytes / (ex_ms * 1e-3) / 1e9,
                  "frac": ex_bytes / (ex_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "sharded": {"shards": shards, "ms_all_shards_and_merge": sh_ms,
                    "achieved_gbs": ex_bytes / (sh_ms * 1e-3) / 1e9,
                    "bitwise_equal_to_unsharded": bool(same)},
    }


def copy_ceiling(src, dst, active, reps=10, warmup=2):
    """Plain-copy rate (GB/s) of the gradient pass's traffic on the same tensors: every row of
    `dst` written, the rows of `src` whose `active` byte is set read, one block per row,
    16-byte nontemporal loads and stores (libdrift_ceiling.so, measurement only); the faster
    of 4 and 8 loads in flight per lane. HIP events on the launch stream, median."""
    import torch

    from train_rollout_logprob_amd import build as Bd

    if not os.path.exists(Bd.CEILING_LIB):
        raise RuntimeError(f"{Bd.CEILING_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(Bd.CEILING_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.drift_copy_ceiling.argtypes = [vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, vp]
    lib.drift_copy_ceiling.restype = ctypes.c_int
    rows = dst.shape[0]
    row_bytes = dst.shape[1] * dst.element_size()
    if src.shape[1] * src.element_size() != row_bytes:
        raise ValueError("copy ceiling: source and destination rows must have the same size")
    n_read = int(active.to(torch.bool).sum().item())
    stream = torch.cuda.current_stream()
    best = None
    for unroll in (4, 8):
        def call():
            st = lib.drift_copy_ceiling(src.data_ptr(), dst.data_ptr(), rows, row_bytes,
                                        src.stride(0) * src.element_size(),
                                        dst.stride(0) * dst.element_size(), active.data_ptr(),
                                        unroll, stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"drift_copy_ceiling: status {st}")

        for _ in range(warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
        gbs = (n_read + rows) * row_bytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, ms, unroll)
    return best


def training_leg(case, ids, att, act, cu, steps=10, warmup=2):
    """Training-only state on the same batch: the scoring kernel with per-row entropy and
    LSE written for both sides (kernel time from events on the launch stream), then
    drift_dlogits of the train side into bf16 with a per-row upstream gradient."""
    import torch

    from train_rollout_logprob_amd import binding as B

    dev = case.train.device
    N, V, esz = case.N, case.V, case.elem_bytes
    n_active = case.n_active()
    ent = tuple(torch.empty(N, dtype=torch.float32, device=dev) for _ in range(2))
    lse = tuple(torch.empty(N, dtype=torch.float64, device=dev) for _ in range(2))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    out = None
    for i in range(warmup + steps):
        evs = (ev[2 * (i - warmup)].cuda_event, ev[2 * (i - warmup) + 1].cuda_event) \
            if i >= warmup else None
        out = B.selected_logprob(case.train, case.rollout, ids, att, act, case.layout, case.B,
                                 case.L, cu, ws=out[4] if out else None,
                                 out=out[:4] if out else None, events=evs, entropy=ent,
                                 lse=lse)
    torch.cuda.synchronize()
    st, _ = B.drift_get_status(out[4])
    if st != B.DRIFT_OK:
        raise RuntimeError(f"scoring with entropy: status {B.STATUS_NAMES[st]}")
    ent_all = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    ent_ms = sum(ent_all) / steps
    ent_bytes = n_active * V * esz * 2
    active = out[3]
    g = torch.randn(N, dtype=torch.float32, device=dev, generator=torch.Generator(
        device=dev).manual_seed(11))
    grad = torch.empty((N, V), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        B.dlogits(case.train, case.rollout, ids, 0, lse[0], active, grad_logp=g,
                  out_dtype=torch.bfloat16, out=grad)
    # one event pair per call: a host stall between calls does not count while the GPU is
    # still busy with the previous call
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    for e0, e1 in dev_ev:
        e0.record()
        B.dlogits(case.train, case.rollout, ids, 0, lse[0], active, grad_logp=g,
                  out_dtype=torch.bfloat16, out=grad)
        e1.record()
    torch.cuda.synchronize()
    dl_all = sorted(e0.elapsed_time(e1) for e0, e1 in dev_ev)
    dl_ms = sum(dl_all) / steps
    dl_bytes = n_active * V * esz + N * V * 2
    dl_gbs = dl_bytes / (dl_ms * 1e-3) / 1e9
    ceiling = copy_ceiling(case.train, grad, active) if esz == 2 else None
    if ceiling:
        log(f"[bench] dlogits {dl_gbs:.0f} GB/s; plain copy of the same rows {ceiling[0]:.0f} GB/s "
            f"({ceiling[1]:.3f} ms, {ceiling[2]} loads in flight): {dl_gbs / ceiling[0]:.3f} of it")
    del grad
    return {
        "workload": "same batch; entropy + LSE of both sides from the scoring pass, then "
                    "dlogits of the train side (bf16 out, upstream gradient per row)",
        "score_with_entropy": {"kernel": f"score_rows<{case.dtype}, entropy>",
                               "kernel_ms": ent_ms, "kernel_ms_median": ent_all[steps // 2],
                               "kernel_ms_min": ent_all[0], "bytes_per_launch": ent_bytes,
                               "achieved_gbs": ent_bytes / (ent_ms * 1e-3) / 1e9,
                               "frac": ent_bytes / (ent_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "dlogits": {"kernel": f"dlogits_rows<{case.dtype}, bf16>", "kernel_ms": dl_ms,
                    "kernel_ms_median": dl_all[steps // 2], "kernel_ms_min": dl_all[0],
                    "bytes_per_launch": dl_bytes,
                    "achieved_gbs": dl_gbs,
                    "frac": dl_gbs / HBM_PEAK_GBS,
                    "ceiling_gbs": ceiling[0] if ceiling else None,
                    "frac_of_ceiling": dl_gbs / ceiling[0] if ceiling else None,
                    "ceiling_kernel": "copy_rows: the same rows of the train logits copied into "
                                      "the gradient buffer, inactive rows written as zeros, "
                                      "16-byte nontemporal loads and stores" if ceiling else None,
                    "traffic": recorded_traffic(DLOGITS_PROFILE, DLOGITS_SOURCES)
                    if case.name == "qwen8b" else None},
    }


def time_steps(runner, steps, warmup, name):
    """Runs `warmup` untimed and `steps` timed steps of a ScoringStep (scoring kernel
    bracketed by events on its launch stream, then drift_diagnostics_async on the step's
    diagnostics stream), pipelined two deep: step i + 1 is launched before the host waits
    for step i and checks its statistics (status and active count), so the GPU does not
    idle while the host reads them and step i's diagnostics overlap step i + 1's scoring;
    the last step is collected and the device synchronized before the clock stops.
    Returns the sorted kernel times (ms), the wall time of the timed steps (s) and the
    last step's statistics."""
    import torch

    from train_rollout_logprob_amd import binding as B

    n_ev = warmup + steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for e0, e1 in evs:          # create the underlying events
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    handles = [(e0.cuda_event, e1.cuda_event) for e0, e1 in evs]

    n_active = []

    def check(slot):
        st = runner.collect(slot)
        if st != B.DRIFT_OK:
            raise RuntimeError(f"{name}: status {B.STATUS_NAMES[st]}")
        n_active.append(runner.stats_of(slot).n_active)

    depth = runner.depth

    def run(lo, hi):
        q = collections.deque()
        last = None
        for i in range(lo, hi):
            if len(q) == depth:  # every slot holds a step: wait for the oldest
                check(q.popleft())
            runner.set_events(*handles[i])
            last = runner.submit()
            q.append(last)
        while q:
            check(q.popleft())
        return last

    run(0, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    last = run(warmup, n_ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if len(set(n_active)) != 1:
        raise RuntimeError(f"{name}: the steps disagree on the active count: {set(n_active)}")
    return (sorted(evs[i][0].elapsed_time(evs[i][1]) for i in range(warmup, n_ev)), elapsed,
            runner.stats_of(last))


def transforms_leg(case, ids, att, act, cu, steps=20, warmup=3):
    """The scoring step on the same batch with the same logit transform on both sides:
    temperature 0.7 (a multiplying chain) and soft-cap 30 (x -> 30 tanh(x / 30)); kernel
    time from events on the launch stream."""
    from train_rollout_logprob_amd import binding as B

    alg = case.n_active() * case.V * case.elem_bytes * 2
    out = {"workload": "same batch, the same chain on both sides"}
    for xf, chain in (("temperature", [("temperature", 0.7)]),
                      ("softcap", [("softcap", 30.0)])):
        runner = B.ScoringStep(case.train, case.rollout, ids, att, act, case.layout, case.B,
                               case.L, cu, case.eps_low, case.eps_high,
                               transforms=(chain, chain))
        kern, _, _ = time_steps(runner, steps, warmup, f"{case.name} {xf}")
        avg = sum(kern) / len(kern)
        out[xf] = {"chain": chain, "kernel": f"score_rows<{case.dtype}, folded chain>",
                   "kernel_ms": avg, "kernel_ms_median": kern[len(kern) // 2],
                   "kernel_ms_min": kern[0], "bytes_per_launch": alg,
                   "achieved_gbs": alg / (avg * 1e-3) / 1e9,
                   "frac": alg / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] {case.name} {xf}: scoring kernel {avg:.3f} ms "
            f"(median {kern[len(kern) // 2]:.3f}), {out[xf]['achieved_gbs']:.0f} GB/s")
        del runner
    return out


def score_leg(name, steps, warmup, xf="none", ceiling=True):
    """Generates one scoring workload on cuda:0 and times `steps` steps (scoring +
    diagnostics, pipelined two deep) after `warmup` untimed ones. Returns the measurement
    and what later legs reuse (the case, its device inputs and the step runner)."""
    import torch

    from train_rollout_logprob_amd import binding as B
    from train_rollout_logprob_amd import synth

    dev = "cuda:0"
    log(f"[bench] generating the {name} workload")
    case = synth.make_logits_case(name, device=dev)
    ids = torch.as_tensor(case.ids, device=dev)
    att = torch.as_tensor(case.attention, device=dev) if case.attention is not None else None
    act = torch.as_tensor(case.action, device=dev)
    cu = torch.as_tensor(case.cu_seqlens, device=dev) if case.cu_seqlens is not None else None
    n_active = case.n_active()
    chain = {"none": None, "temperature": [("temperature", 0.7)],
             "softcap": [("softcap", 30.0)]}[xf]
    runner = B.ScoringStep(case.train, case.rollout, ids, att, act, case.layout, case.B,
                           case.L, cu, case.eps_low, case.eps_high, transforms=(chain, chain))
    log(f"[bench] {name}: timing {steps} steps")
    kern, elapsed, stats = time_steps(runner, steps, warmup, name)
    kern_avg = sum(kern) / len(kern)
    if stats.n_active != n_active:
        raise RuntimeError(f"{name}: {stats.n_active} active rows, expected {n_active}")
    alg_bytes = n_active * case.V * case.elem_bytes * 2
    achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
    ms_per_step = elapsed * 1e3 / steps
    out = {
        "workload": WORKLOAD_TEXT[name], "V": case.V, "B": case.B, "L": case.L, "N": case.N,
        "n_active": n_active, "logits_dtype": case.dtype, "transforms": xf,
        "ms_per_step": ms_per_step, "active_tokens_per_s": n_active * steps / elapsed,
        "logits_gbs": alg_bytes * steps / elapsed / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(SCORE_PROFILES[name])
                     if name in SCORE_PROFILES and xf == "none" else None,
                     "kernel": f"score_rows<{case.dtype}>", "kernel_ms": kern_avg,
                     "kernel_ms_median": kern[len(kern) // 2], "kernel_ms_min": kern[0],
                     "bytes_per_launch": alg_bytes},
        "diagnostics": {k: getattr(stats, k) for k in (
            "ratio0", "clipfrac0", "approx_kl0", "mismatch_kl", "mean_abs_dlogp",
            "p95_abs_dlogp", "p99_abs_dlogp", "max_abs_dlogp", "argmax_row")},
    }
    log(f"[bench] {name}: step {ms_per_step:.3f} ms, scoring kernel {kern_avg:.3f} ms "
        f"(median {kern[len(kern) // 2]:.3f}, min {kern[0]:.3f}; {achieved:.0f} GB/s), "
        f"{out['active_tokens_per_s'] / 1e6:.3f} M active tok/s")
    if ceiling:
        ceiling_gbs, ceiling_ms = read_ceiling(case)
        out["roofline"].update({
            "ceiling_gbs": ceiling_gbs, "frac_of_ceiling": achieved / ceiling_gbs,
            "ceiling_kernel": "read_rows: pure 16-byte nontemporal reads of every row pair "
                              "of the same tensors, one block per pair"})
        log(f"[bench] {name}: pure-read ceiling {ceiling_gbs:.0f} GB/s ({ceiling_ms:.3f} ms); "
            f"scoring kernel at {achieved / ceiling_gbs:.3f} of it")
    if name == "tiny":
        out["roofline"]["note"] = ("0.65 MB per launch: launch-latency bound, a correctness "
                                   "case, not a bandwidth figure")
    return out, (case, ids, att, act, cu, runner)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="large", choices=["qwen8b", "large", "packed", "tiny",
                                                             "lmhead"],
                    help="the main line's scoring workload (default: large, the largest "
                         "single-GPU batch)")
    ap.add_argument("--legs", default="all",
                    help="legs beside the main line: all, none (for profiling runs), or a "
                         "comma list of " + ", ".join(LEGS))
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: a plain device copy of known size, to calibrate HBM counters")
    ap.add_argument("--copy-mib", type=int, default=4096)
    ap.add_argument("--xf", default="none", choices=["none", "temperature", "softcap"],
                    help="apply a logit transform on both sides (cost of the option)")
    args = ap.parse_args()
    args.legs = (set(LEGS) if args.legs == "all" else set() if args.legs == "none"
                 else set(args.legs.split(",")))
    if not args.legs <= set(LEGS):
        ap.error(f"--legs: unknown leg(s) {sorted(args.legs - set(LEGS))}")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library "
              f"has no multi-GPU path; the per-row work shards by rows with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    # the oracle's worker pool starts before this process touches the GPU
    pool = None
    if args.mode == "bench" and args.workload != "lmhead" and not args.no_cpu_baseline:
        from oracle.pool import OraclePool
        pool = OraclePool()
    try:
        run(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run(args, pool):
    import torch

    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.mode == "copy":
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        e0.record()
        for _ in range(5):
            dst.fill_(7)
        e1.record()
        torch.cuda.synchronize()
        ms_fill = e0.elapsed_time(e1) / 5
        log(f"[bench] copied {n} bytes 8 times (read {n} and write {n} per copy): "
            f"{ms:.3f} ms per copy = {2 * n / (ms * 1e-3) / 1e9:.0f} GB/s read+write; "
            f"fill {ms_fill:.3f} ms = {n / (ms_fill * 1e-3) / 1e9:.0f} GB/s write")
        return
    if args.workload == "lmhead":
        print(json.dumps(lmhead_leg(args.steps, args.warmup)), flush=True)
        return

    main_leg, (case, ids, att, act, cu, runner) = score_leg(args.workload, args.steps,
                                                            args.warmup, args.xf)
    rf = main_leg["roofline"]
    line = {
        "metric": METRIC,
        "value": main_leg["active_tokens_per_s"],
        "unit": "active tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": main_leg["workload"], "V": case.V, "B": case.B, "L": case.L,
                   "N": case.N, "n_active": main_leg["n_active"], "logits_dtype": case.dtype,
                   "arith": "logits widened to fp32; fp32 exp2 terms, fp64 sums and LSE",
                   "transforms": args.xf, "parallelism": "single GPU"},
        "logits_gbs": main_leg["logits_gbs"],
        "roofline": rf,
        "cpu_baseline": None,
        "diagnostics": main_leg["diagnostics"],
    }
    sample = None
    if pool is not None:
        log("[bench] copying the CPU baseline's sample rows to the host")
        sample = cpu_sample(pool, case)
    legs = args.legs if args.xf == "none" else set()

    def qwen8b_legs(case, ids, att, act, cu):
        if "training" in legs:
            torch.cuda.empty_cache()
            log("[bench] training-state leg (entropy, lse, dlogits)")
            line["training"] = training_leg(case, ids, att, act, cu)
        if "exact" in legs:
            torch.cuda.empty_cache()
            log("[bench] exact-reduction leg (unsharded and vocabulary shards)")
            line["exact"] = exact_leg(case, ids, att, act, cu)
        if "transforms" in legs:
            log("[bench] logit-transform leg (temperature, soft-cap)")
            line["transforms"] = transforms_leg(case, ids, att, act, cu)

    if "segments" in legs:
        line["segments"] = segments_leg(case, runner.out[2], runner.out[3], runner.ws)
        line["active_rows"] = active_rows_leg(case, runner.out[3])
        if line["active_rows"]["n_active"] != main_leg["n_active"]:
            raise RuntimeError("active-row list length differs from the active count")
    del runner
    if args.workload == "qwen8b":
        qwen8b_legs(case, ids, att, act, cu)
    del case, ids, att, act, cu
    torch.cuda.empty_cache()
    if "configs" in legs:
        line["configs"] = {}
        for name in OTHER_CONFIGS[args.workload]:
            leg, (case, ids, att, act, cu, runner) = score_leg(name, args.steps, args.warmup)
            line["configs"][name] = leg
            del runner
            if name == "qwen8b":
                qwen8b_legs(case, ids, att, act, cu)
            del case, ids, att, act, cu
            torch.cuda.empty_cache()
    if "lmhead" in legs:
        log("[bench] fused LM-head leg")
        line["lmhead"] = lmhead_leg()
        torch.cuda.empty_cache()
    # the CPU leg runs last, so the GPU legs above run at the clocks of a busy GPU
    if sample is not None:
        log(f"[bench] cpu baseline (oracle, {pool.workers} worker processes)")
        line["cpu_baseline"] = cpu_baseline(pool, sample, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Python binding of the drift library (C ABI of include/drift.h).

This module only marshals arguments into the C ABI declared in ``include/drift.h``; every
step of the computation runs in the HIP kernels of ``libdrift.so``. Loading fails loudly
if the library has not been built (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library shares with PyTorch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdrift.so")

DRIFT_OK = 0
DRIFT_EINVAL = -1
DRIFT_EDTYPE = -2
DRIFT_EWORKSPACE = -3
DRIFT_ETOKEN = -4
DRIFT_EMASK = -5
DRIFT_ENOACTIVE = -6
DRIFT_ENONFINITE = -7
DRIFT_EHIP = -8
STATUS_NAMES = {DRIFT_OK: "OK", DRIFT_EINVAL: "EINVAL", DRIFT_EDTYPE: "EDTYPE",
                DRIFT_EWORKSPACE: "EWORKSPACE", DRIFT_ETOKEN: "ETOKEN", DRIFT_EMASK: "EMASK",
                DRIFT_ENOACTIVE: "ENOACTIVE", DRIFT_ENONFINITE: "ENONFINITE",
                DRIFT_EHIP: "EHIP"}

DRIFT_F32, DRIFT_BF16, DRIFT_I32, DRIFT_I64 = 0, 1, 2, 3
DRIFT_PAD_RIGHT, DRIFT_PAD_LEFT, DRIFT_PACKED = 0, 1, 2
LAYOUTS = {"right": DRIFT_PAD_RIGHT, "left": DRIFT_PAD_LEFT, "packed": DRIFT_PACKED}
DRIFT_OP_SELECTED_LOGPROB, DRIFT_OP_DIAGNOSTICS, DRIFT_OP_LMHEAD, DRIFT_OP_ACTIVE_ROWS = 0, 1, 2, 3
DRIFT_OP_LMHEAD_VH = 4
DRIFT_WEIGHT_HV, DRIFT_WEIGHT_VH = 0, 1
DRIFT_XF_SCALE, DRIFT_XF_TEMPERATURE, DRIFT_XF_SOFTCAP = 1, 2, 3
DRIFT_MAX_TRANSFORMS = 4
DRIFT_REDUCE_TREE, DRIFT_REDUCE_EXACT = 0, 1
REDUCTIONS = {"tree": DRIFT_REDUCE_TREE, "exact": DRIFT_REDUCE_EXACT}
DRIFT_PART_SCORED, DRIFT_PART_OWNER, DRIFT_PART_BAD = 1, 2, 4
DRIFT_MAX_SHARDS = 64
XF_CODES = {"scale": DRIFT_XF_SCALE, "temperature": DRIFT_XF_TEMPERATURE,
            "softcap": DRIFT_XF_SOFTCAP}

EXPORTS = ("drift_workspace_size", "drift_selected_logprob", "drift_get_status",
           "drift_diagnostics", "drift_segment_diagnostics", "drift_lmhead_logprob",
           "drift_dlogits", "drift_shard_partials", "drift_merge_shards",
           "drift_active_rows", "drift_backend_descriptor", "drift_strerror",
           "drift_diagnostics_noalloc", "drift_lmhead_logprob_vh", "drift_lmhead_logprob_chain",
           "drift_diagnostics_async")
DRIFT_NOALLOC_MAX_ROWS = 1 << 22


class drift_transform(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("op", ctypes.c_int32 * DRIFT_MAX_TRANSFORMS),
                ("value", ctypes.c_float * DRIFT_MAX_TRANSFORMS)]


class drift_logprob_args(ctypes.Structure):
    _fields_ = [("logits_dtype", ctypes.c_int32), ("ids_dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("reduction", ctypes.c_int32),
                ("num_rows", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("train_logits", ctypes.c_void_p),
                ("rollout_logits", ctypes.c_void_p), ("target_ids", ctypes.c_void_p),
                ("attention_mask", ctypes.c_void_p), ("action_mask", ctypes.c_void_p),
                ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("cu_seqlens", ctypes.c_void_p), ("num_seqs", ctypes.c_int64),
                ("prof_events", ctypes.c_void_p * 2), ("vocab_real", ctypes.c_int64),
                ("transforms", drift_transform * 2), ("entropy", ctypes.c_void_p * 2),
                ("lse", ctypes.c_void_p * 2)]


class drift_lse_partial(ctypes.Structure):
    _fields_ = [("bin", ctypes.c_uint64 * 3), ("top", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("x_sel", ctypes.c_float), ("reserved", ctypes.c_float)]


class drift_stats(ctypes.Structure):
    _fields_ = [("n_active", ctypes.c_int64), ("n_clip_low", ctypes.c_int64),
                ("n_clip_high", ctypes.c_int64), ("n_nonfinite", ctypes.c_int64),
                ("argmax_row", ctypes.c_int64), ("ratio0", ctypes.c_double),
                ("clipfrac0", ctypes.c_double), ("approx_kl0", ctypes.c_double),
                ("mean_abs_dlogp", ctypes.c_double), ("mean_dlogp", ctypes.c_double),
                ("p95_abs_dlogp", ctypes.c_float), ("p99_abs_dlogp", ctypes.c_float),
                ("max_abs_dlogp", ctypes.c_float), ("status", ctypes.c_int32),
                ("mismatch_kl", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class drift_backend_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32)] + [
        (n, ctypes.c_char_p) for n in ("backend_id", "semantic_ops", "archs", "dtypes",
                                        "layouts", "determinism", "precision", "lse_domain",
                                        "fallback", "build_fingerprint")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import "
                          f"__graft_entry__ as g; g.build()'` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.drift_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int]
    lib.drift_workspace_size.restype = sz
    lib.drift_selected_logprob.argtypes = [ctypes.POINTER(drift_logprob_args), vp, vp, vp, vp,
                                           vp, sz, vp]
    lib.drift_selected_logprob.restype = ctypes.c_int
    lib.drift_get_status.argtypes = [vp, vp, ctypes.POINTER(i64)]
    lib.drift_get_status.restype = ctypes.c_int
    lib.drift_diagnostics.argtypes = [vp, vp, i64, ctypes.c_double, ctypes.c_double, vp,
                                      ctypes.POINTER(drift_stats), vp, sz, vp]
    lib.drift_diagnostics.restype = ctypes.c_int
    lib.drift_diagnostics_async.argtypes = [vp, vp, i64, ctypes.c_double, ctypes.c_double, vp,
                                            vp, vp, sz, vp]
    lib.drift_diagnostics_async.restype = ctypes.c_int
    lib.drift_diagnostics_noalloc.argtypes = [vp, vp, i64, ctypes.c_double, ctypes.c_double,
                                              vp, vp, vp]
    lib.drift_diagnostics_noalloc.restype = ctypes.c_int
    lib.drift_segment_diagnostics.argtypes = [vp, vp, i64, vp, i64, ctypes.c_double,
                                              ctypes.c_double, vp, vp, vp]
    lib.drift_segment_diagnostics.restype = ctypes.c_int
    lib.drift_active_rows.argtypes = [vp, i64, vp, vp, vp, sz, vp]
    lib.drift_active_rows.restype = ctypes.c_int
    lib.drift_lmhead_logprob.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.drift_lmhead_logprob.restype = ctypes.c_int
    lib.drift_lmhead_logprob_vh.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.drift_lmhead_logprob_vh.restype = ctypes.c_int
    lib.drift_lmhead_logprob_chain.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp, vp,
                                               ctypes.POINTER(drift_transform), vp, vp, sz, vp]
    lib.drift_lmhead_logprob_chain.restype = ctypes.c_int
    lib.drift_dlogits.argtypes = [ctypes.POINTER(drift_logprob_args), ctypes.c_int, vp, vp, vp,
                                  ctypes.c_int, vp, i64, vp]
    lib.drift_dlogits.restype = ctypes.c_int
    lib.drift_shard_partials.argtypes = [ctypes.POINTER(drift_logprob_args), i64, i64, vp, vp, vp,
                                         sz, vp]
    lib.drift_shard_partials.restype = ctypes.c_int
    lib.drift_merge_shards.argtypes = [ctypes.POINTER(drift_logprob_args), vp, vp, ctypes.c_int,
                                       ctypes.POINTER(i64), vp, vp, vp, vp, vp, sz, vp]
    lib.drift_merge_shards.restype = ctypes.c_int
    lib.drift_backend_descriptor.argtypes = []
    lib.drift_backend_descriptor.restype = ctypes.POINTER(drift_backend_desc)
    lib.drift_strerror.argtypes = [ctypes.c_int]
    lib.drift_strerror.restype = ctypes.c_char_p
    return lib


lib = _load()


# ----------------------------------------------------------------------------- C names

def drift_workspace_size(op: int, num_rows: int, vocab: int, hidden_dim: int, dtype: int) -> int:
    return int(lib.drift_workspace_size(op, num_rows, vocab, hidden_dim, dtype))


def drift_selected_logprob(args: drift_logprob_args, train_logp, rollout_logp, dlogp, active,
                           ws, ws_bytes: int, stream) -> int:
    return int(lib.drift_selected_logprob(ctypes.byref(args), _ptr(train_logp),
                                          _ptr(rollout_logp), _ptr(dlogp), _ptr(active),
                                          _ptr(ws), ws_bytes, _stream(stream)))


def drift_get_status(ws, stream=None):
    bad = ctypes.c_int64(-1)
    st = int(lib.drift_get_status(_ptr(ws), _stream(stream), ctypes.byref(bad)))
    return st, int(bad.value)


def drift_diagnostics(dlogp, active, num_rows: int, eps_low: float, eps_high: float,
                      logprob_ws, ws, ws_bytes: int, stream=None):
    out = drift_stats()
    st = int(lib.drift_diagnostics(_ptr(dlogp), _ptr(active), num_rows, eps_low, eps_high,
                                   _ptr(logprob_ws), ctypes.byref(out), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    return st, out


def drift_segment_diagnostics(dlogp, active, num_rows: int, seg_offsets, num_segments: int,
                              eps_low: float, eps_high: float, logprob_ws, out_dev,
                              stream=None) -> int:
    return int(lib.drift_segment_diagnostics(_ptr(dlogp), _ptr(active), num_rows,
                                             _ptr(seg_offsets), num_segments, eps_low,
                                             eps_high, _ptr(logprob_ws), _ptr(out_dev),
                                             _stream(stream)))


def drift_diagnostics_async(dlogp, active, num_rows: int, eps_low: float, eps_high: float,
                            logprob_ws, out, ws, ws_bytes: int, stream=None) -> int:
    return int(lib.drift_diagnostics_async(_ptr(dlogp), _ptr(active), num_rows, eps_low,
                                           eps_high, _ptr(logprob_ws), _ptr(out), _ptr(ws),
                                           ws_bytes, _stream(stream)))


def drift_diagnostics_noalloc(dlogp, active, num_rows: int, eps_low: float, eps_high: float,
                              logprob_ws, out_dev, stream=None) -> int:
    return int(lib.drift_diagnostics_noalloc(_ptr(dlogp), _ptr(active), num_rows, eps_low,
                                             eps_high, _ptr(logprob_ws), _ptr(out_dev),
                                             _stream(stream)))


def drift_active_rows(active, num_rows: int, rows, n_dev, ws, ws_bytes: int,
                      stream=None) -> int:
    return int(lib.drift_active_rows(_ptr(active), num_rows, _ptr(rows), _ptr(n_dev), _ptr(ws),
                                     ws_bytes, _stream(stream)))


def drift_lmhead_logprob(hidden, weight, T: int, H: int, V: int, target_ids, active, logp, ws,
                         ws_bytes: int, stream=None) -> int:
    return int(lib.drift_lmhead_logprob(_ptr(hidden), _ptr(weight), T, H, V, _ptr(target_ids),
                                        _ptr(active), _ptr(logp), _ptr(ws), ws_bytes,
                                        _stream(stream)))


def drift_lmhead_logprob_vh(hidden, weight_vh, T: int, H: int, V: int, target_ids, active, logp,
                            ws, ws_bytes: int, stream=None) -> int:
    return int(lib.drift_lmhead_logprob_vh(_ptr(hidden), _ptr(weight_vh), T, H, V,
                                           _ptr(target_ids), _ptr(active), _ptr(logp), _ptr(ws),
                                           ws_bytes, _stream(stream)))


def drift_lmhead_logprob_chain(hidden, weight, weight_layout: int, T: int, H: int, V: int,
                               target_ids, active, transform, logp, ws, ws_bytes: int,
                               stream=None) -> int:
    """`transform`: a drift_transform, or None."""
    return int(lib.drift_lmhead_logprob_chain(
        _ptr(hidden), _ptr(weight), weight_layout, T, H, V, _ptr(target_ids), _ptr(active),
        ctypes.byref(transform) if transform is not None else None, _ptr(logp), _ptr(ws),
        ws_bytes, _stream(stream)))


def drift_dlogits(args: drift_logprob_args, side: int, lse, active, grad_logp, out_dtype: int,
                  grad_logits, out_stride: int, stream=None) -> int:
    return int(lib.drift_dlogits(ctypes.byref(args), side, _ptr(lse), _ptr(active),
                                 _ptr(grad_logp), out_dtype, _ptr(grad_logits), out_stride,
                                 _stream(stream)))


def drift_shard_partials(local: drift_logprob_args, vocab_start: int, vocab_global: int,
                         train_part, rollout_part, ws, ws_bytes: int, stream=None) -> int:
    return int(lib.drift_shard_partials(ctypes.byref(local), vocab_start, vocab_global,
                                        _ptr(train_part), _ptr(rollout_part), _ptr(ws),
                                        ws_bytes, _stream(stream)))


def drift_merge_shards(glob: drift_logprob_args, train_parts, rollout_parts, num_shards: int,
                       shard_bounds, train_logp, rollout_logp, dlogp, active, ws,
                       ws_bytes: int, stream=None) -> int:
    b = (ctypes.c_int64 * (num_shards + 1))(*[int(x) for x in shard_bounds])
    return int(lib.drift_merge_shards(ctypes.byref(glob), _ptr(train_parts),
                                      _ptr(rollout_parts), num_shards, b, _ptr(train_logp),
                                      _ptr(rollout_logp), _ptr(dlogp), _ptr(active), _ptr(ws),
                                      ws_bytes, _stream(stream)))


def drift_backend_descriptor() -> dict:
    d = lib.drift_backend_descriptor().contents
    out = {"abi_version": d.abi_version}
    for n, _ in drift_backend_desc._fields_[1:]:
        v = getattr(d, n)
        out[n] = v.decode() if v is not None else None
    return out


def drift_strerror(status: int) -> str:
    return lib.drift_strerror(status).decode()


# ----------------------------------------------------------------------------- helpers

def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


class DriftError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({drift_strerror(status)})")


def workspace(op: int, num_rows: int, vocab: int, dtype: int, device, hidden_dim: int = 0
              ) -> torch.Tensor:
    n = drift_workspace_size(op, num_rows, vocab, hidden_dim, dtype)
    if n == 0:
        raise DriftError(DRIFT_EINVAL, "drift_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def set_chain(t: drift_transform, chain):
    """Fill a drift_transform from [(kind, value), ...] with kind in XF_CODES."""
    chain = list(chain or ())
    if len(chain) > DRIFT_MAX_TRANSFORMS:
        raise ValueError("at most 4 transform steps")
    t.count = len(chain)
    for i, (kind, value) in enumerate(chain):
        t.op[i] = XF_CODES[kind]
        t.value[i] = float(value)


def make_args(train, rollout, ids, attention=None, action=None, layout="right", batch=0,
              seq_len=0, cu_seqlens=None, vocab=None, events=None, vocab_real=None,
              transforms=(None, None), entropy=(None, None), lse=(None, None),
              reduction="tree") -> drift_logprob_args:
    """Describe torch tensors to the C ABI (no copies, no conversions). `vocab_real`:
    leading columns that enter the log-sum-exp (None = all); `transforms`: (train chain,
    rollout chain), each [(kind, value), ...]; `entropy` / `lse`: optional per-side
    output tensors (fp32 / fp64 [N]); `reduction`: "tree" or "exact"."""
    if train.dtype != rollout.dtype or train.shape != rollout.shape:
        raise ValueError("train and rollout logits must share dtype and shape")
    if train.stride(1) != 1 or rollout.stride(0) != train.stride(0):
        raise ValueError("logits rows must be contiguous with a common row stride")
    a = drift_logprob_args()
    a.logits_dtype = {torch.float32: DRIFT_F32, torch.bfloat16: DRIFT_BF16}.get(train.dtype, 99)
    a.ids_dtype = {torch.int32: DRIFT_I32, torch.int64: DRIFT_I64}.get(ids.dtype, 99)
    a.layout = LAYOUTS[layout]
    a.reduction = REDUCTIONS[reduction]
    a.num_rows = train.shape[0]
    a.vocab = vocab if vocab is not None else train.shape[1]
    a.row_stride = train.stride(0)
    a.train_logits = train.data_ptr()
    a.rollout_logits = rollout.data_ptr()
    a.target_ids = ids.data_ptr()
    a.attention_mask = attention.data_ptr() if attention is not None else None
    a.action_mask = action.data_ptr() if action is not None else None
    a.batch = batch
    a.seq_len = seq_len
    a.cu_seqlens = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    a.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else 0
    if events is not None:
        a.prof_events[0] = events[0]
        a.prof_events[1] = events[1]
    a.vocab_real = 0 if vocab_real is None else int(vocab_real)
    set_chain(a.transforms[0], transforms[0])
    set_chain(a.transforms[1], transforms[1])
    for side in (0, 1):
        e, l = entropy[side], lse[side]
        if e is not None and (e.dtype != torch.float32 or e.numel() < a.num_rows):
            raise ValueError("entropy outputs are fp32 [N]")
        if l is not None and (l.dtype != torch.float64 or l.numel() < a.num_rows):
            raise ValueError("lse outputs are fp64 [N]")
        a.entropy[side] = e.data_ptr() if e is not None else None
        a.lse[side] = l.data_ptr() if l is not None else None
    return a


def selected_logprob(train, rollout, ids, attention=None, action=None, layout="right",
                     batch=0, seq_len=0, cu_seqlens=None, ws=None, out=None, stream=None,
                     events=None, check=False, vocab_real=None, transforms=(None, None),
                     entropy=(None, None), lse=(None, None), reduction="tree"):
    """Allocate outputs (and a workspace unless given) and call drift_selected_logprob.
    Returns (train_logp, rollout_logp, dlogp, active, ws). With check=True, synchronizes
    and raises DriftError on a data-dependent status. `entropy` / `lse`: optional output
    tensors per side, filled by the same call."""
    N = train.shape[0]
    dev = train.device
    args = make_args(train, rollout, ids, attention, action, layout, batch, seq_len,
                     cu_seqlens, events=events, vocab_real=vocab_real, transforms=transforms,
                     entropy=entropy, lse=lse, reduction=reduction)
    if ws is None:
        ws = workspace(DRIFT_OP_SELECTED_LOGPROB, N, args.vocab, args.logits_dtype, dev)
    if out is None:
        out = (torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty(N, dtype=torch.float32, device=dev),
               torch.empty(N, dtype=torch.uint8, device=dev))
    st = drift_selected_logprob(args, *out, ws, ws.numel(), stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_selected_logprob")
    if check:
        st, _ = drift_get_status(ws, stream)
        if st != DRIFT_OK:
            raise DriftError(st, "drift_selected_logprob (device)")
    return (*out, ws)


def diagnostics(dlogp, active, eps_low=0.2, eps_high=0.2, logprob_ws=None, ws=None,
                stream=None):
    """Call drift_diagnostics; returns (status, stats dict)."""
    N = dlogp.shape[0]
    if ws is None:
        ws = workspace(DRIFT_OP_DIAGNOSTICS, N, 1, DRIFT_F32, dlogp.device)
    st, s = drift_diagnostics(dlogp, active, N, eps_low, eps_high, logprob_ws, ws, ws.numel(),
                              stream)
    return st, s.as_dict()


def shard_partials(train_local, rollout_local, ids, vocab_start, vocab_global, attention=None,
                   action=None, layout="right", batch=0, seq_len=0, cu_seqlens=None,
                   vocab_real=None, transforms=(None, None), out=None, ws=None, stream=None,
                   events=None):
    """Call drift_shard_partials on one shard's logits (the [N, width] columns
    [vocab_start, vocab_start + width) of the global vocabulary). Returns
    (train_partials, rollout_partials, ws): uint8 tensors holding [N] drift_lse_partial."""
    args = make_args(train_local, rollout_local, ids, attention, action, layout, batch, seq_len,
                     cu_seqlens, events=events, vocab_real=vocab_real, transforms=transforms)
    N = int(args.num_rows)
    dev = train_local.device
    if ws is None:
        ws = workspace(DRIFT_OP_SELECTED_LOGPROB, N, max(int(args.vocab), 1), args.logits_dtype,
                       dev)
    if out is None:
        nb = max(N, 1) * ctypes.sizeof(drift_lse_partial)
        out = (torch.empty(nb, dtype=torch.uint8, device=dev),
               torch.empty(nb, dtype=torch.uint8, device=dev))
    st = drift_shard_partials(args, vocab_start, vocab_global, out[0], out[1], ws, ws.numel(),
                              stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_shard_partials")
    return out[0], out[1], ws


def merge_shards(train_parts, rollout_parts, shard_bounds, ids, vocab, num_rows,
                 attention=None, action=None, layout="right", batch=0, seq_len=0,
                 cu_seqlens=None, vocab_real=None, lse=(None, None), out=None, ws=None,
                 stream=None):
    """Call drift_merge_shards on gathered partials (uint8 tensors holding
    [S][N] drift_lse_partial). Returns (train_logp, rollout_logp, dlogp, active, ws)."""
    dev = train_parts.device
    S = len(shard_bounds) - 1
    a = drift_logprob_args()
    a.logits_dtype, a.layout = DRIFT_F32, LAYOUTS[layout]
    a.ids_dtype = {torch.int32: DRIFT_I32, torch.int64: DRIFT_I64}.get(ids.dtype, 99)
    a.reduction = DRIFT_REDUCE_EXACT
    a.num_rows, a.vocab, a.row_stride = num_rows, vocab, vocab
    a.target_ids = ids.data_ptr()
    a.attention_mask = attention.data_ptr() if attention is not None else None
    a.action_mask = action.data_ptr() if action is not None else None
    a.batch, a.seq_len = batch, seq_len
    a.cu_seqlens = cu_seqlens.data_ptr() if cu_seqlens is not None else None
    a.num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else 0
    a.vocab_real = 0 if vocab_real is None else int(vocab_real)
    for side in (0, 1):
        a.lse[side] = lse[side].data_ptr() if lse[side] is not None else None
    if ws is None:
        ws = workspace(DRIFT_OP_SELECTED_LOGPROB, num_rows, vocab, DRIFT_F32, dev)
    if out is None:
        out = (torch.empty(num_rows, dtype=torch.float32, device=dev),
               torch.empty(num_rows, dtype=torch.float32, device=dev),
               torch.empty(num_rows, dtype=torch.float32, device=dev),
               torch.empty(num_rows, dtype=torch.uint8, device=dev))
    st = drift_merge_shards(a, train_parts, rollout_parts, S, shard_bounds, *out, ws, ws.numel(),
                            stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_merge_shards")
    return (*out, ws)


def dlogits(train, rollout, ids, side, lse, active, grad_logp=None, out_dtype=torch.float32,
            out=None, vocab_real=None, transforms=(None, None), stream=None):
    """Call drift_dlogits for one side (0 = train, 1 = rollout): the gradient of that side's
    selected logprob with respect to its logits, given the forward pass's `lse[side]` and
    `active`. Returns the [N, V] gradient tensor (out_dtype float32 or bfloat16)."""
    args = make_args(train, rollout, ids, vocab_real=vocab_real, transforms=transforms)
    N, V = int(args.num_rows), int(args.vocab)
    code = {torch.float32: DRIFT_F32, torch.bfloat16: DRIFT_BF16}.get(out_dtype, 99)
    if out is None:
        out = torch.empty(N, V, dtype=out_dtype, device=train.device)
    if out.dim() != 2 or out.shape[0] != N or out.stride(1) != 1:
        raise ValueError("out must be [N, >= V] with contiguous rows")
    if lse.dtype != torch.float64 or active.dtype != torch.uint8:
        raise ValueError("lse must be float64 and active uint8")
    if grad_logp is not None and grad_logp.dtype != torch.float32:
        raise ValueError("grad_logp must be float32")
    st = drift_dlogits(args, side, lse, active, grad_logp, code, out, out.stride(0), stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_dlogits")
    return out


def active_rows(active, rows=None, n=None, ws=None, stream=None):
    """Call drift_active_rows on a uint8 device tensor [N]. Returns (rows, n, ws): rows is an
    int32 tensor [N] whose first n entries are the active row indices in ascending order,
    n an int64 device tensor [1] (read it with .item(), which synchronizes)."""
    N = active.shape[0]
    dev = active.device
    if active.dtype != torch.uint8 or active.dim() != 1:
        raise ValueError("active must be a uint8 vector")
    if ws is None:
        ws = workspace(DRIFT_OP_ACTIVE_ROWS, N, 1, DRIFT_F32, dev)
    if rows is None:
        rows = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    if n is None:
        n = torch.empty(1, dtype=torch.int64, device=dev)
    st = drift_active_rows(active, N, rows, n, ws, ws.numel(), stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_active_rows")
    return rows, n, ws


def segment_diagnostics(dlogp, active, seg_offsets, eps_low=0.2, eps_high=0.2, logprob_ws=None,
                        stream=None):
    """Call drift_segment_diagnostics; seg_offsets is an int32 device tensor [S + 1].
    Returns a list of S stats dicts (one synchronizing copy of the device results)."""
    N = dlogp.shape[0]
    if seg_offsets.dtype != torch.int32 or seg_offsets.dim() != 1 or seg_offsets.numel() < 1:
        raise ValueError("seg_offsets must be an int32 vector [S + 1]")
    S = seg_offsets.numel() - 1
    out = torch.empty(max(S, 1) * ctypes.sizeof(drift_stats), dtype=torch.uint8,
                      device=dlogp.device)
    st = drift_segment_diagnostics(dlogp, active, N, seg_offsets, S, eps_low, eps_high,
                                   logprob_ws, out, stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_segment_diagnostics")
    host = bytearray(out.cpu().numpy().tobytes())
    arr = (drift_stats * max(S, 1)).from_buffer(host)
    return [arr[i].as_dict() for i in range(S)]


def diagnostics_noalloc(dlogp, active, eps_low=0.2, eps_high=0.2, logprob_ws=None, out=None,
                        stream=None):
    """Call drift_diagnostics_noalloc (no workspace; statistics written to the device
    buffer `out`, a uint8 tensor of sizeof(drift_stats) bytes, allocated here if None).
    Returns (stats dict, out); the dict comes from one synchronizing copy of `out`."""
    N = dlogp.shape[0]
    if out is None:
        out = torch.empty(ctypes.sizeof(drift_stats), dtype=torch.uint8, device=dlogp.device)
    st = drift_diagnostics_noalloc(dlogp, active, N, eps_low, eps_high, logprob_ws, out, stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_diagnostics_noalloc")
    host = bytearray(out.cpu().numpy().tobytes())
    return drift_stats.from_buffer(host).as_dict(), out


def diagnostics_async(dlogp, active, out, eps_low=0.2, eps_high=0.2, logprob_ws=None,
                      ws=None, stream=None):
    """Call drift_diagnostics_async: the statistics go to `out`, a uint8 tensor of
    sizeof(drift_stats) bytes in device memory or pinned host memory, once the stream
    passes the call; nothing is synchronized here. Returns the workspace, which stays in
    use until then."""
    N = dlogp.shape[0]
    if out.numel() < ctypes.sizeof(drift_stats) or out.dtype != torch.uint8:
        raise ValueError("out must be a uint8 tensor of at least sizeof(drift_stats) bytes")
    if not out.is_cuda and not out.is_pinned():
        raise ValueError("out must be device memory or pinned host memory")
    if ws is None:
        ws = workspace(DRIFT_OP_DIAGNOSTICS, N, 1, DRIFT_F32, dlogp.device)
    st = drift_diagnostics_async(dlogp, active, N, eps_low, eps_high, logprob_ws, out, ws,
                                 ws.numel(), stream)
    if st != DRIFT_OK:
        raise DriftError(st, "drift_diagnostics_async")
    return ws


def stats_from(buf) -> dict:
    """The statistics held in a uint8 tensor written by drift_diagnostics_async or
    drift_diagnostics_noalloc (copied to the host first if it is device memory; the caller
    has already waited for the call)."""
    host = bytearray(buf[:ctypes.sizeof(drift_stats)].cpu().numpy().tobytes())
    return drift_stats.from_buffer(host).as_dict()


def report(stats: dict, segments=None, **metadata) -> dict:
    """One JSON-ready report of a comparison ("Diagnostics" table, report layout): the
    statistics, optional per-segment versions, and metadata (the backend descriptor plus
    whatever the caller records: dtype, padding side, parallelism, cache mode, ...)."""
    desc = drift_backend_descriptor()
    out = {"metrics": {k: stats[k] for k in ("max_abs_dlogp", "mean_abs_dlogp",
                                             "p95_abs_dlogp", "p99_abs_dlogp", "ratio0",
                                             "clipfrac0", "approx_kl0", "mismatch_kl")},
           "mismatch_k3_kl": stats["approx_kl0"],
           "worst_token": {"row": stats["argmax_row"], "abs_dlogp": stats["max_abs_dlogp"]},
           "counts": {k: stats[k] for k in ("n_active", "n_clip_low", "n_clip_high",
                                            "n_nonfinite")},
           "status": STATUS_NAMES.get(stats["status"], stats["status"]),
           "metadata": dict(metadata, backend=desc)}
    if segments is not None:
        out["segments"] = [{"metrics": {k: s[k] for k in out["metrics"]},
                            "n_active": s["n_active"], "worst_row": s["argmax_row"],
                            "status": STATUS_NAMES.get(s["status"], s["status"])}
                           for s in segments]
    return out


class ScoringStep:
    """Repeated drift_selected_logprob + drift_diagnostics on fixed tensors.

    All marshalling (argument struct, output tensors, workspaces, pinned host buffers for
    the statistics) is done once here, so a call to `run` is two C calls.

    `run` waits for each step's statistics. `submit` / `collect` pipeline the steps instead:
    `submit` scores a step into one of `depth` slots (per-row outputs and a logprob
    workspace per slot) on the step's stream, then launches drift_diagnostics_async on a
    second stream once the scoring is done, with the statistics landing in the slot's
    pinned host record, and returns the slot. `collect(slot)` waits for that step's
    diagnostics and returns its status, the statistics then in `stats_of(slot)` and the
    per-row outputs in `out_of(slot)`. A loop that submits step i + 1 before collecting
    step i keeps the GPU busy while the host reads and checks the previous step, and the
    diagnostics of step i run beside the scoring of step i + 1 instead of between the two
    scoring passes. At most `depth` steps are outstanding: `submit` raises when the next
    slot has not been collected (collecting waits for the slot's diagnostics, so the slot's
    buffers are free again), and `collect` raises for a slot with no outstanding step.
    `run` uses slot 0 and raises while steps are outstanding; `out` and `ws` are slot 0's
    buffers.

    `overlap`: True puts the submitted steps' diagnostics on the second stream, False on
    the step's own stream after its scoring; None (default) chooses True when a step
    reads at least OVERLAP_MIN_BYTES of logits. On small batches the hand-over between
    the streams costs more than the diagnostics it hides (a 128-row fp32 batch: 57 µs
    per step against 37 µs on one stream)."""

    OVERLAP_MIN_BYTES = 512 << 20

    def __init__(self, train, rollout, ids, attention=None, action=None, layout="right",
                 batch=0, seq_len=0, cu_seqlens=None, eps_low=0.2, eps_high=0.2,
                 stream=None, vocab_real=None, transforms=(None, None), depth=2,
                 overlap=None):
        if depth < 1:
            raise ValueError("depth >= 1")
        dev = train.device
        self.args = make_args(train, rollout, ids, attention, action, layout, batch, seq_len,
                              cu_seqlens, vocab_real=vocab_real, transforms=transforms)
        self.N = int(self.args.num_rows)
        self.depth = depth
        self.eps = (float(eps_low), float(eps_high))
        self._ws = [workspace(DRIFT_OP_SELECTED_LOGPROB, self.N, self.args.vocab,
                              self.args.logits_dtype, dev) for _ in range(depth)]
        self.dws = workspace(DRIFT_OP_DIAGNOSTICS, self.N, 1, DRIFT_F32, dev)
        self._out = [(torch.empty(self.N, dtype=torch.float32, device=dev),
                      torch.empty(self.N, dtype=torch.float32, device=dev),
                      torch.empty(self.N, dtype=torch.float32, device=dev),
                      torch.empty(self.N, dtype=torch.uint8, device=dev))
                     for _ in range(depth)]
        self.ws, self.out = self._ws[0], self._out[0]
        sz = ctypes.sizeof(drift_stats)
        self._pinned = torch.empty(sz * (1 + depth), dtype=torch.uint8, pin_memory=True)
        self.stats = drift_stats.from_address(self._pinned.data_ptr())
        self._slot_ptr = [self._pinned.data_ptr() + sz * (1 + k) for k in range(depth)]
        self._slots = [drift_stats.from_address(q) for q in self._slot_ptr]
        # the stream every scoring call of this step launches into, fixed here (None = the
        # stream current now); submitted steps' diagnostics go to a stream of their own
        if stream is None:
            self._stream_obj = torch.cuda.current_stream()
        elif isinstance(stream, int):
            self._stream_obj = torch.cuda.ExternalStream(stream)
        else:
            self._stream_obj = stream
        self._stream = self._stream_obj.cuda_stream
        if overlap is None:
            esz = 2 if self.args.logits_dtype == DRIFT_BF16 else 4
            overlap = 2 * self.N * int(self.args.vocab) * esz >= self.OVERLAP_MIN_BYTES
        self.overlap = bool(overlap)
        self._diag_obj = torch.cuda.Stream(device=dev) if self.overlap else self._stream_obj
        self._diag = self._diag_obj.cuda_stream
        self._scored = [torch.cuda.Event() for _ in range(depth)]
        self._done = [torch.cuda.Event() for _ in range(depth)]
        self._pending = [False] * depth
        self._next = 0
        self._args_ref = ctypes.byref(self.args)
        self._stats_ref = ctypes.byref(self.stats)
        self._lp = []
        for k in range(depth):
            t, r, d, a = (x.data_ptr() for x in self._out[k])
            self._lp.append((self._args_ref, t, r, d, a, self._ws[k].data_ptr(),
                             self._ws[k].numel(), self._stream))
        self._lp_args = self._lp[0]
        d, a = self._lp[0][3], self._lp[0][4]
        self._dg_args = (d, a, self.N, self.eps[0], self.eps[1], self.ws.data_ptr(),
                         self._stats_ref, self.dws.data_ptr(), self.dws.numel(), self._stream)

    def set_events(self, ev0, ev1):
        """hipEvent_t handles recorded around the scoring kernel (0 to disable)."""
        self.args.prof_events[0] = ev0
        self.args.prof_events[1] = ev1

    def run(self) -> int:
        if any(self._pending):
            raise RuntimeError("run() with submitted steps not yet collected")
        st = lib.drift_selected_logprob(*self._lp_args)
        if st != DRIFT_OK:
            raise DriftError(st, "drift_selected_logprob")
        return lib.drift_diagnostics(*self._dg_args)

    def submit(self) -> int:
        """Launches one step; returns its slot."""
        k = self._next
        if self._pending[k]:
            raise RuntimeError(f"slot {k} still holds an uncollected step (depth "
                               f"{len(self._slots)})")
        self._next = (k + 1) % len(self._slots)
        lp = self._lp[k]
        st = lib.drift_selected_logprob(*lp)
        if st != DRIFT_OK:
            raise DriftError(st, "drift_selected_logprob")
        if self.overlap:
            self._scored[k].record(self._stream_obj)
            self._diag_obj.wait_event(self._scored[k])
        st = lib.drift_diagnostics_async(lp[3], lp[4], self.N, self.eps[0], self.eps[1],
                                         lp[5], self._slot_ptr[k], self.dws.data_ptr(),
                                         self.dws.numel(), self._diag)
        if st != DRIFT_OK:
            raise DriftError(st, "drift_diagnostics_async")
        self._done[k].record(self._diag_obj)
        self._pending[k] = True
        return k

    def collect(self, slot) -> int:
        """Waits for the step of `slot` (its diagnostics included); returns their status."""
        if not self._pending[slot]:
            raise RuntimeError(f"slot {slot} has no outstanding step")
        self._done[slot].synchronize()
        self._pending[slot] = False
        return self._slots[slot].status

    def stats_of(self, slot):
        return self._slots[slot]

    def out_of(self, slot):
        """(train_logp, rollout_logp, dlogp, active) of the step last submitted to `slot`."""
        return self._out[slot]

    def ws_of(self, slot):
        """The logprob workspace (device status) of the step last submitted to `slot`."""
        return self._ws[slot]


class ScoringGraph:
    """One step of a ScoringStep (drift_selected_logprob + drift_diagnostics_async) captured
    once as a HIP graph (torch.cuda.CUDAGraph) and replayed as a single launch, for batches
    small enough that launching the step's kernels one by one costs more than running them.

    The graph keeps the step's pointers: every replay reads the step's input tensors as they
    are then (overwrite them in place to score new data) and writes the step's outputs
    (`step.out`) and this graph's pinned statistics record (`stats()` once the replay has
    completed). The capture launches kernels only: neither entry point copies, sets memory
    or synchronizes. Profiling events are off inside the graph. A replay uses the step's
    slot-0 buffers and diagnostics workspace: it must not overlap the step's own `run` or
    submitted steps (wait for the replay, or collect every submitted step, in between)."""

    def __init__(self, step):
        self.step = step
        self._pinned = torch.empty(ctypes.sizeof(drift_stats), dtype=torch.uint8,
                                   pin_memory=True)
        self._stats = drift_stats.from_address(self._pinned.data_ptr())
        self.graph = torch.cuda.CUDAGraph()
        ev = (step.args.prof_events[0], step.args.prof_events[1])
        step.set_events(0, 0)
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):  # one uncaptured step first, as torch asks
                self._launch(side.cuda_stream)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(self.graph):
                self._launch(torch.cuda.current_stream().cuda_stream)
        finally:
            step.set_events(*ev)

    def _launch(self, stream):
        st = self.step
        t, r, d, a = st._lp_args[1:5]
        rc = lib.drift_selected_logprob(st._args_ref, t, r, d, a, st.ws.data_ptr(),
                                        st.ws.numel(), stream)
        if rc != DRIFT_OK:
            raise DriftError(rc, "drift_selected_logprob")
        rc = lib.drift_diagnostics_async(d, a, st.N, st.eps[0], st.eps[1], st.ws.data_ptr(),
                                         self._pinned.data_ptr(), st.dws.data_ptr(),
                                         st.dws.numel(), stream)
        if rc != DRIFT_OK:
            raise DriftError(rc, "drift_diagnostics_async")

    def replay(self):
        """Launches the captured step on the current stream (asynchronous)."""
        self.graph.replay()

    def stats(self):
        """The statistics of the last completed replay (the caller has waited for it)."""
        return self._stats


def lmhead_logprob(hidden, weight, ids, active=None, ws=None, out=None, stream=None,
                   check=False, weight_layout="hv", transforms=None):
    """Call drift_lmhead_logprob on torch tensors: hidden bf16 [T, H], weight bf16 [H, V]
    (weight_layout "hv") or [V, H] ("vh": drift_lmhead_logprob_vh, read in place), ids
    int32 [T], active uint8 [T] or None; `transforms`: an optional chain [(kind, value),
    ...] on the head's logits (drift_lmhead_logprob_chain). Returns (logp, ws)."""
    T, H = hidden.shape
    if weight_layout == "hv":
        H2, V = weight.shape
        op, fn, name = DRIFT_OP_LMHEAD, drift_lmhead_logprob, "drift_lmhead_logprob"
    elif weight_layout == "vh":
        V, H2 = weight.shape
        op, fn, name = DRIFT_OP_LMHEAD_VH, drift_lmhead_logprob_vh, "drift_lmhead_logprob_vh"
    else:
        raise ValueError("weight_layout is 'hv' or 'vh'")
    if H2 != H or hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise ValueError("hidden [T, H] and the weight must be bf16 with matching H")
    if not (hidden.is_contiguous() and weight.is_contiguous() and ids.is_contiguous()):
        raise ValueError("hidden, weight and ids must be contiguous")
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if ws is None:
        ws = workspace(op, T, V, DRIFT_BF16, hidden.device, hidden_dim=H)
    if out is None:
        out = torch.empty(T, dtype=torch.float32, device=hidden.device)
    if transforms:
        t = drift_transform()
        set_chain(t, transforms)
        layout = DRIFT_WEIGHT_VH if weight_layout == "vh" else DRIFT_WEIGHT_HV
        name = "drift_lmhead_logprob_chain"
        st = drift_lmhead_logprob_chain(hidden, weight, layout, T, H, V, ids, active, t, out,
                                        ws, ws.numel(), stream)
    else:
        st = fn(hidden, weight, T, H, V, ids, active, out, ws, ws.numel(), stream)
    if st != DRIFT_OK:
        raise DriftError(st, name)
    if check:
        st, _ = drift_get_status(ws, stream)
        if st != DRIFT_OK:
            raise DriftError(st, name + " (device)")
    return out, ws

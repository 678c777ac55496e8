"""The C-ABI library loads and exports every symbol the header declares; host-side
argument checks fail closed before any launch (CPU only; no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "drift.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(drift_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(["drift_workspace_size", "drift_selected_logprob",
                            "drift_get_status", "drift_diagnostics", "drift_lmhead_logprob",
                            "drift_dlogits", "drift_segment_diagnostics",
                            "drift_shard_partials", "drift_merge_shards",
                            "drift_active_rows", "drift_backend_descriptor",
                            "drift_strerror", "drift_diagnostics_noalloc",
                            "drift_lmhead_logprob_vh", "drift_lmhead_logprob_chain",
                            "drift_diagnostics_async"])


def test_library_exports_every_declared_symbol():
    from train_rollout_logprob_amd import binding as B
    raw = ctypes.CDLL(B.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(B.EXPORTS) == set(_declared_functions())


def test_struct_layouts_match_header():
    from train_rollout_logprob_amd import binding as B
    # drift_logprob_args: 4 x i32, 3 x i64, 5 pointers, 2 x i64, pointer, i64, 2 pointers,
    # i64 vocab_real, 2 x drift_transform (i32 count, 4 x i32 op, 4 x f32 value),
    # 2 entropy pointers, 2 lse pointers (offsets 208 and 224, as gcc lays out the header)
    assert ctypes.sizeof(B.drift_transform) == 36
    assert ctypes.sizeof(B.drift_logprob_args) == 16 + 24 + 40 + 16 + 8 + 8 + 16 + 8 + 72 + 32
    assert B.drift_logprob_args.entropy.offset == 208 and B.drift_logprob_args.lse.offset == 224
    assert ctypes.sizeof(B.drift_stats) == 5 * 8 + 5 * 8 + 3 * 4 + 4 + 8
    assert B.drift_stats.mismatch_kl.offset == 96
    assert ctypes.sizeof(B.drift_lse_partial) == 40


def test_descriptor_and_strerror():
    from train_rollout_logprob_amd import binding as B
    d = B.drift_backend_descriptor()
    assert d["abi_version"] == 10 and d["archs"] == "gfx950"
    assert "batch composition" in d["determinism"]
    assert d["lse_domain"] == "natural log"
    assert d["build_fingerprint"].startswith("src:")
    for code in B.STATUS_NAMES:
        assert B.drift_strerror(code) != "unknown status"
    assert B.drift_strerror(12345) == "unknown status"


def test_workspace_sizes():
    from train_rollout_logprob_amd import binding as B
    f = lambda op, n, v, dt, h=0: B.drift_workspace_size(op, n, v, h, dt)
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, 16384, 151936, B.DRIFT_BF16) == 256   # header only
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, 0, 1, B.DRIFT_F32) >= 256
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, 10, 0, B.DRIFT_F32) == 0      # V < 1
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, -1, 5, B.DRIFT_F32) == 0
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, 1 << 31, 5, B.DRIFT_F32) == 0
    assert f(B.DRIFT_OP_SELECTED_LOGPROB, 10, 5, 7) == 0                # bad dtype
    assert f(B.DRIFT_OP_DIAGNOSTICS, 270000, 1, B.DRIFT_F32) > 0
    assert f(B.DRIFT_OP_LMHEAD, 16384, 151936, B.DRIFT_F32, 4096) == 0  # bf16 only
    assert f(B.DRIFT_OP_LMHEAD, 16384, 151936, B.DRIFT_BF16, 4100) == 0 # H % 8
    # transposed W + partials: at least H*V*2 bytes
    assert f(B.DRIFT_OP_LMHEAD, 16384, 151936, B.DRIFT_BF16, 4096) >= 4096 * 151936 * 2
    # [V, H] weight read in place when H % 64 == 0: partials, z and one 256-row tail panel
    # of W (V % 256 != 0), no transposed copy
    vh = f(B.DRIFT_OP_LMHEAD_VH, 16384, 151936, B.DRIFT_BF16, 4096)
    assert 0 < vh < 4096 * 151936 * 2
    assert vh == f(B.DRIFT_OP_LMHEAD, 16384, 151936, B.DRIFT_BF16, 4096) - \
        (151936 + 128) * 4096 * 2 + 256 * 4096 * 2
    # H not a multiple of 64: the weight is copied with K padding as for [H, V]
    assert f(B.DRIFT_OP_LMHEAD_VH, 300, 1000, B.DRIFT_BF16, 264) == \
        f(B.DRIFT_OP_LMHEAD, 300, 1000, B.DRIFT_BF16, 264)
    assert f(B.DRIFT_OP_LMHEAD_VH, 16384, 151936, B.DRIFT_BF16, 4100) == 0
    assert f(9, 10, 10, B.DRIFT_F32) == 0


def test_host_checks_fail_closed_without_launching():
    from train_rollout_logprob_amd import binding as B
    lib = B.lib
    assert lib.drift_selected_logprob(None, None, None, None, None, None, 0, None) == B.DRIFT_EINVAL
    a = B.drift_logprob_args()
    a.logits_dtype = 5
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EDTYPE
    a.logits_dtype, a.ids_dtype, a.layout = B.DRIFT_F32, B.DRIFT_I32, B.DRIFT_PAD_RIGHT
    a.num_rows, a.vocab, a.row_stride = 0, 10, 5                        # stride < V
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL
    a.row_stride, a.batch, a.seq_len = 10, 0, 1
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EWORKSPACE        # no workspace
    a.layout = 7
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL
    a.layout, a.num_rows, a.batch, a.seq_len = B.DRIFT_PAD_LEFT, 6, 2, 4  # B*L != N
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL
    a.num_rows, a.batch, a.seq_len = 0, 1 << 32, 1 << 32       # B*L wraps to 0 in 64 bits
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL
    st = B.drift_stats()
    assert lib.drift_diagnostics(None, None, 5, 0.2, 0.2, None, ctypes.byref(st), None, 0,
                                 None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics(None, None, 0, 1.5, 0.2, None, ctypes.byref(st), None, 0,
                                 None) == B.DRIFT_EINVAL                # eps out of range
    assert lib.drift_lmhead_logprob(None, None, 4, 4100, 16, None, None, None, None, 0,
                                    None) == B.DRIFT_EINVAL             # H % 8 != 0
    big = 1 << 20                                     # aligned addresses, never dereferenced
    assert lib.drift_lmhead_logprob(big, big, 4, (1 << 22) + 8, 16, big, None, big, big, 1 << 40,
                                    None) == B.DRIFT_EINVAL             # H above 2^22
    for fn in (lib.drift_lmhead_logprob, lib.drift_lmhead_logprob_vh):
        assert fn(None, None, 4, 4100, 16, None, None, None, None, 0, None) == B.DRIFT_EINVAL
        assert fn(big, big, 4, 64, 12, big, None, big, big, 1 << 40, None) == B.DRIFT_EINVAL
        assert fn(big + 8, big, 4, 64, 16, big, None, big, big, 1 << 40,
                  None) == B.DRIFT_EINVAL                               # hidden not 16-aligned
        assert fn(big, big, 4, 64, 16, big, None, big, big, 64,
                  None) == B.DRIFT_EWORKSPACE                           # workspace too small
        # one dispatch of 512-thread blocks over padded 256 x 256 tiles: T <= 3,530,752 at
        # V = 151936 (the workspace check comes after the shape check)
        assert fn(big, big, 3530752, 4096, 151936, big, None, big, big, 64,
                  None) == B.DRIFT_EWORKSPACE
        assert fn(big, big, 3530753, 4096, 151936, big, None, big, big, 1 << 40,
                  None) == B.DRIFT_EINVAL
    # the chain entry point: layout and chain checked before the workspace; chains that
    # do not fold (two soft-caps, a cap above 40) are refused
    fc = lambda layout, chain, ws_bytes: lib.drift_lmhead_logprob_chain(
        big, big, layout, 4, 64, 16, big, None,
        ctypes.byref(chain) if chain is not None else None, big, big, ws_bytes, None)
    for chain, want in (([("softcap", 30.0)], B.DRIFT_EWORKSPACE),
                        ([("temperature", 0.7), ("scale", -2.0)], B.DRIFT_EWORKSPACE),
                        ([], B.DRIFT_EWORKSPACE),
                        ([("softcap", 30.0), ("softcap", 20.0)], B.DRIFT_EINVAL),
                        ([("softcap", 60.0)], B.DRIFT_EINVAL),
                        ([("softcap", 30.0), ("scale", 2.0)], B.DRIFT_EINVAL),
                        ([("temperature", 0.0)], B.DRIFT_EINVAL)):
        t = B.drift_transform()
        B.set_chain(t, chain)
        for layout in (B.DRIFT_WEIGHT_HV, B.DRIFT_WEIGHT_VH):
            assert fc(layout, t, 64) == want, (chain, layout)
    assert fc(2, None, 1 << 40) == B.DRIFT_EINVAL                      # unknown layout
    assert fc(B.DRIFT_WEIGHT_HV, None, 64) == B.DRIFT_EWORKSPACE       # no chain
    for op in (B.DRIFT_OP_LMHEAD, B.DRIFT_OP_LMHEAD_VH):
        assert B.drift_workspace_size(op, 3530752, 151936, 4096, B.DRIFT_BF16) > 0
        assert B.drift_workspace_size(op, 3530753, 151936, 4096, B.DRIFT_BF16) == 0
    assert lib.drift_get_status(None, None, None) == B.DRIFT_EWORKSPACE
    # vocab_real and transform chains are checked before the workspace
    a.layout, a.num_rows, a.batch, a.seq_len, a.vocab, a.row_stride = B.DRIFT_PAD_RIGHT, 0, 0, 1, 10, 10
    a.vocab_real = 11                                                  # > V
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL
    a.vocab_real = 0
    for chain in ([("temperature", 0.0)], [("softcap", -1.0)], [("scale", float("nan"))],
                  [("scale", 1.0)] * 5):
        try:
            B.set_chain(a.transforms[1], chain)
        except ValueError:
            continue                                                   # more than 4 steps
        assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                          None) == B.DRIFT_EINVAL, chain
    B.set_chain(a.transforms[1], [])
    a.transforms[0].count = 1
    a.transforms[0].op[0] = 9                                          # unknown op
    a.transforms[0].value[0] = 1.0
    assert lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                      None) == B.DRIFT_EINVAL


def test_dlogits_host_checks_fail_closed_without_launching():
    from train_rollout_logprob_amd import binding as B
    f = B.lib.drift_dlogits
    a = B.drift_logprob_args()
    a.logits_dtype, a.ids_dtype, a.layout = B.DRIFT_BF16, B.DRIFT_I64, B.DRIFT_PAD_RIGHT
    a.num_rows, a.vocab, a.row_stride = 0, 10, 10
    assert f(None, 0, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_EINVAL
    assert f(ctypes.byref(a), 2, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_EINVAL
    assert f(ctypes.byref(a), 0, None, None, None, B.DRIFT_I32, None, 10, None) == B.DRIFT_EDTYPE
    assert f(ctypes.byref(a), 1, None, None, None, B.DRIFT_BF16, None, 9, None) == B.DRIFT_EINVAL
    assert f(ctypes.byref(a), 1, None, None, None, B.DRIFT_BF16, None, 10, None) == B.DRIFT_OK
    a.num_rows = 4                                                    # outputs required
    assert f(ctypes.byref(a), 0, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_EINVAL
    a.num_rows, a.vocab_real = 0, 11
    assert f(ctypes.byref(a), 0, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_EINVAL
    a.vocab_real = 0
    B.set_chain(a.transforms[0], [("temperature", -2.0)])
    assert f(ctypes.byref(a), 0, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_EINVAL
    assert f(ctypes.byref(a), 1, None, None, None, B.DRIFT_F32, None, 10, None) == B.DRIFT_OK


def test_segment_diagnostics_host_checks():
    from train_rollout_logprob_amd import binding as B
    f = B.lib.drift_segment_diagnostics
    assert f(None, None, 10, None, 0, 0.2, 0.2, None, None, None) == B.DRIFT_OK   # no segments
    assert f(None, None, 10, None, 2, 0.2, 0.2, None, None, None) == B.DRIFT_EINVAL
    assert f(None, None, -1, None, 0, 0.2, 0.2, None, None, None) == B.DRIFT_EINVAL
    assert f(None, None, 10, None, 0, 0.2, 1.0, None, None, None) == B.DRIFT_EINVAL


def test_shard_and_merge_host_checks():
    from train_rollout_logprob_amd import binding as B
    a = B.drift_logprob_args()
    a.logits_dtype, a.ids_dtype, a.layout = B.DRIFT_BF16, B.DRIFT_I32, B.DRIFT_PAD_RIGHT
    a.num_rows, a.vocab, a.row_stride, a.batch, a.seq_len = 0, 16, 16, 0, 1
    sp = B.lib.drift_shard_partials
    assert sp(ctypes.byref(a), 4, 64, None, None, None, 0, None) == B.DRIFT_EINVAL    # % 8
    assert sp(ctypes.byref(a), 56, 64, None, None, None, 0, None) == B.DRIFT_EINVAL   # past end
    assert sp(ctypes.byref(a), 48, 64, None, None, None, 0, None) == B.DRIFT_EWORKSPACE
    a.reduction = 3
    assert sp(ctypes.byref(a), 48, 64, None, None, None, 0, None) == B.DRIFT_EINVAL
    a.reduction = 0
    mg = B.lib.drift_merge_shards
    b = (ctypes.c_int64 * 3)(0, 8, 16)
    assert mg(ctypes.byref(a), None, None, 0, b, None, None, None, None, None, 0, None) == B.DRIFT_EINVAL
    assert mg(ctypes.byref(a), None, None, 65, b, None, None, None, None, None, 0, None) == B.DRIFT_EINVAL
    bad = (ctypes.c_int64 * 3)(0, 9, 15)                                    # does not end at V
    assert mg(ctypes.byref(a), None, None, 2, bad, None, None, None, None, None, 0, None) == B.DRIFT_EINVAL
    assert mg(ctypes.byref(a), None, None, 2, b, None, None, None, None, None, 0, None) == B.DRIFT_EWORKSPACE
    # exact reduction does not carry the entropy moment
    a.reduction = B.DRIFT_REDUCE_EXACT
    e = ctypes.c_void_p(256)
    a.entropy[0] = e
    assert B.lib.drift_selected_logprob(ctypes.byref(a), None, None, None, None, None, 0,
                                        None) == B.DRIFT_EINVAL


CEILING_HEADER = os.path.join(ROOT, "include", "drift_ceiling.h")


def _ceiling_lib():
    from train_rollout_logprob_amd import build as Bd
    if not os.path.exists(Bd.CEILING_LIB):
        pytest.skip("libdrift_ceiling.so is not built")
    lib = ctypes.CDLL(Bd.CEILING_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.drift_read_ceiling.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.drift_read_ceiling.restype = ctypes.c_int
    lib.drift_copy_ceiling.argtypes = [vp, vp, i64, i64, i64, i64, vp, ctypes.c_int, vp]
    lib.drift_copy_ceiling.restype = ctypes.c_int
    return lib


def test_ceiling_library_exports_its_declared_symbols():
    src = re.sub(r"/\*.*?\*/", "", open(CEILING_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(drift_[a-z_]+)\s*\(", src)))
    assert names == ["drift_copy_ceiling", "drift_read_ceiling"]
    lib = _ceiling_lib()
    for n in names:
        assert hasattr(lib, n), n


def test_ceiling_host_checks_fail_before_launch():
    lib = _ceiling_lib()
    good = 1 << 20                                     # an aligned address, never dereferenced
    EINVAL = -1
    assert lib.drift_read_ceiling(None, None, 0, 16, 16, None, None) == 0   # nothing to read
    cases = [
        (good, good, -1, 16, 16, good),                # negative rows
        (good, good, 1 << 31, 16, 16, good),           # rows beyond a grid
        (good, good, 1, 0, 16, good),                  # empty rows
        (good, good, 1, 24, 32, good),                 # row bytes not a multiple of 16
        (good, good, 1, 32, 16, good),                 # stride below the row
        (good, good, 1, 16, 24, good),                 # stride not a multiple of 16
        (None, good, 1, 16, 16, good),                 # null input
        (good, good, 1, 16, 16, None),                 # null sink
        (good + 8, good, 1, 16, 16, good),             # misaligned input
        (good, good, 1, 16, 16, good + 2),             # misaligned sink
    ]
    for a, b, rows, rb, st, sink in cases:
        assert lib.drift_read_ceiling(a, b, rows, rb, st, sink, None) == EINVAL, (rows, rb, st)
    assert lib.drift_copy_ceiling(None, None, 0, 16, 16, 16, None, 8, None) == 0  # no rows
    copy_cases = [
        (good, good, -1, 16, 16, 16, 8),               # negative rows
        (good, good, 1 << 31, 16, 16, 16, 8),          # rows beyond a grid
        (good, good, 1, 0, 16, 16, 8),                 # empty rows
        (good, good, 1, 24, 32, 32, 8),                # row bytes not a multiple of 16
        (good, good, 1, 32, 16, 32, 8),                # source stride below the row
        (good, good, 1, 32, 32, 16, 8),                # destination stride below the row
        (good, good, 1, 16, 24, 16, 8),                # stride not a multiple of 16
        (good, good, 1, 16, 16, 16, 2),                # unsupported unroll
        (None, good, 1, 16, 16, 16, 8),                # null source
        (good, None, 1, 16, 16, 16, 4),                # null destination
        (good + 8, good, 1, 16, 16, 16, 8),            # misaligned source
        (good, good + 4, 1, 16, 16, 16, 8),            # misaligned destination
    ]
    for src, dst, rows, rb, ss, ds, u in copy_cases:
        assert lib.drift_copy_ceiling(src, dst, rows, rb, ss, ds, None, u, None) == EINVAL, \
            (rows, rb, ss, ds, u)


def test_build_fingerprint_covers_every_source():
    """The descriptor's source hash must change with any kernel source or header the
    library is compiled from."""
    from train_rollout_logprob_amd import build as Bd
    on_disk = {f for f in os.listdir(Bd.CSRC) if f.endswith((".hip", ".h"))}
    assert on_disk - {Bd.CEILING_SOURCE} == set(Bd.SOURCES) | set(Bd.HEADERS)


def test_active_rows_host_checks():
    from train_rollout_logprob_amd import binding as B
    ok = ctypes.c_void_p(1 << 20)  # aligned stand-ins; no call below reaches a launch
    ws = 1 << 16
    need = B.drift_workspace_size(B.DRIFT_OP_ACTIVE_ROWS, 5000, 1, 0, B.DRIFT_F32)
    assert need == 256  # one int32 count per tile of 4096 rows, rounded up to 256 bytes
    f = B.lib.drift_active_rows
    assert f(ok, -1, ok, ok, ws, need, None) == B.DRIFT_EINVAL
    assert f(ok, 5000, ok, None, ws, need, None) == B.DRIFT_EINVAL          # no n
    assert f(None, 5000, ok, ok, ws, need, None) == B.DRIFT_EINVAL          # no mask
    assert f(ok, 5000, ctypes.c_void_p((1 << 20) + 2), ok, ws, need, None) == B.DRIFT_EINVAL
    assert f(ok, 5000, ok, ok, ws, need - 1, None) == B.DRIFT_EWORKSPACE
    assert f(ok, 5000, ok, ok, ws + 8, need, None) == B.DRIFT_EWORKSPACE
    # up to 1024 tiles: counts only; beyond, int64 offsets per tile after the counts
    size = lambda n: B.drift_workspace_size(B.DRIFT_OP_ACTIVE_ROWS, n, 1, 0, B.DRIFT_F32)
    assert size(4096 * 1024) == 4096
    assert size(4096 * 1024 + 1) == 4352 + 8448  # 1025 counts, then 1025 offsets
    big = 2 ** 31 - 1
    tiles = -(-big // 4096)
    assert size(big) == -(-4 * tiles // 256) * 256 + -(-8 * tiles // 256) * 256
    assert f(ok, 4096 * 1024 + 1, ok, ok, ws, size(4096 * 1024 + 1) - 1, None) == \
        B.DRIFT_EWORKSPACE


def test_diagnostics_async_host_checks():
    """Null or misaligned outputs, bad sizes and eps, and short or misaligned workspaces
    fail before any launch (fake device pointers are never dereferenced)."""
    from train_rollout_logprob_amd import binding as B
    lib = B.lib
    d, a, out, ws = 4096, 8192, 16384, 1 << 20
    need = lib.drift_workspace_size(B.DRIFT_OP_DIAGNOSTICS, 100000, 1, 0, B.DRIFT_F32)
    f = lib.drift_diagnostics_async
    assert f(d, a, 100000, 0.2, 0.2, None, None, ws, need, None) == B.DRIFT_EINVAL
    assert f(d, a, 100000, 0.2, 0.2, None, out + 4, ws, need, None) == B.DRIFT_EINVAL
    assert f(d, a, -1, 0.2, 0.2, None, out, ws, need, None) == B.DRIFT_EINVAL
    assert f(d, a, 1 << 31, 0.2, 0.2, None, out, ws, need, None) == B.DRIFT_EINVAL
    assert f(d, a, 100000, 0.2, 1.0, None, out, ws, need, None) == B.DRIFT_EINVAL
    assert f(None, a, 100000, 0.2, 0.2, None, out, ws, need, None) == B.DRIFT_EINVAL
    assert f(d + 2, a, 100000, 0.2, 0.2, None, out, ws, need, None) == B.DRIFT_EINVAL
    assert f(d, a, 100000, 0.2, 0.2, None, out, ws, need - 1, None) == B.DRIFT_EWORKSPACE
    assert f(d, a, 100000, 0.2, 0.2, None, out, ws + 8, need, None) == B.DRIFT_EWORKSPACE
    assert f(d, a, 100000, 0.2, 0.2, None, out, None, need, None) == B.DRIFT_EWORKSPACE


def test_diagnostics_noalloc_host_checks():
    """Sizes beyond the scratch, null or misaligned outputs and bad eps fail before any
    launch (fake device pointers are never dereferenced)."""
    from train_rollout_logprob_amd import binding as B
    lib = B.lib
    d, a, out = 4096, 8192, 16384
    big = B.DRIFT_NOALLOC_MAX_ROWS + 1
    assert lib.drift_diagnostics_noalloc(d, a, big, 0.2, 0.2, None, out, None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics_noalloc(d, a, 10, 0.2, 0.2, None, None, None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics_noalloc(d, a, 10, 0.2, 0.2, None, out + 4, None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics_noalloc(d, a, -1, 0.2, 0.2, None, out, None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics_noalloc(d, a, 10, 1.0, 0.2, None, out, None) == B.DRIFT_EINVAL
    assert lib.drift_diagnostics_noalloc(None, a, 10, 0.2, 0.2, None, out, None) == B.DRIFT_EINVAL

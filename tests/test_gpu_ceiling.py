"""The measurement-only read kernel (libdrift_ceiling.so) reads every 16-byte vector of each
row pair exactly once: its per-wave XOR fold equals the fold computed on the host."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from train_rollout_logprob_amd import build as Bd
    if not os.path.exists(Bd.CEILING_LIB):
        raise RuntimeError(f"{Bd.CEILING_LIB} is missing: build it first")
    lib = ctypes.CDLL(Bd.CEILING_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.drift_read_ceiling.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.drift_read_ceiling.restype = ctypes.c_int
    return lib


def host_fold(a_rows, b_rows):
    """sink word w of row r: XOR of every uint32 of the vectors v (16 bytes each) with
    v mod 256 in [64 w, 64 w + 64), over both arrays."""
    out = np.zeros((a_rows.shape[0], 4), np.uint32)
    for arr in (a_rows, b_rows):
        vec = arr.view(np.uint32).reshape(arr.shape[0], -1, 4)
        lane = np.arange(vec.shape[1]) % 256
        for w in range(4):
            sel = vec[:, (lane >= 64 * w) & (lane < 64 * w + 64), :]
            out[:, w] ^= np.bitwise_xor.reduce(sel.reshape(arr.shape[0], -1), axis=1) \
                if sel.shape[1] else np.uint32(0)
    return out


@pytest.mark.parametrize("rows,row_vecs,pad_vecs", [(1, 1, 0), (3, 255, 1), (5, 2048, 0),
                                                    (7, 2049, 3), (4, 18992, 0), (2, 5000, 16)])
def test_read_ceiling_reads_every_vector_once(lib, rows, row_vecs, pad_vecs):
    print(f"case rows={rows} row_vecs={row_vecs} pad_vecs={pad_vecs}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(rows * 100003 + row_vecs)
    stride_words = 4 * (row_vecs + pad_vecs)
    a = torch.randint(-2**31, 2**31 - 1, (rows, stride_words), generator=g, device="cuda",
                      dtype=torch.int32)
    b = torch.randint(-2**31, 2**31 - 1, (rows, stride_words), generator=g, device="cuda",
                      dtype=torch.int32)
    sink = torch.zeros(rows * 4, dtype=torch.int32, device="cuda")
    st = lib.drift_read_ceiling(a.data_ptr(), b.data_ptr(), rows, 16 * row_vecs,
                                4 * stride_words, sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    an = a.cpu().numpy()[:, :4 * row_vecs].view(np.uint32)
    bn = b.cpu().numpy()[:, :4 * row_vecs].view(np.uint32)
    want = host_fold(an, bn)
    got = sink.cpu().numpy().view(np.uint32).reshape(rows, 4)
    np.testing.assert_array_equal(got, want)

"""The measurement kernels of libspd_probe.so (include/spd_probe.h) that the
benchmark's floor legs time: they run through their C ABI on real slices (an
empty slice, a one-row slice, slices past the 2048 indices staged at a time)
in every decomposition the benchmark uses, and leave what they must: every
gather workgroup writes its word, the store leaves zeros, the empty launch
succeeds."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import dev, device_csr, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    lib_dir = os.environ.get("SPD_LIB_DIR") or os.path.join(ROOT, "sparse_paged_decode_ragged_amd", "_lib")
    L = ctypes.CDLL(os.path.join(lib_dir, "libspd_probe.so"))
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.spd_probe_gather.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
    L.spd_probe_null.argtypes = [i32, P]
    L.spd_probe_store.argtypes = [P, i64, i32, P]
    return L


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("D", [64, 512])
def test_gather_probe_runs_every_decomposition(probe, D):
    lengths = [0, 1, 17, 300, 2500, 0, 64]
    w = W.random_csr("probe", 5, len(lengths), 8, D, 4000, lengths)
    log("case probe gather D=%d" % D)
    kv = W.device_bits(w.kv_bits, dev())
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    for groups, parts in [(1, 1), (4, 1), (1, 4), (2, 3)]:
        words = torch.full((w.N * groups * parts,), 0x5A5A5A5A, dtype=torch.int32, device=dev())
        st = probe.spd_probe_gather(kv.data_ptr(), idx.data_ptr(), ptr.data_ptr(), w.N, D, groups,
                                    parts, words.data_ptr(), stream())
        assert st == 0
        torch.cuda.synchronize()
        got = words.cpu().numpy()
        assert not np.any(got == 0x5A5A5A5A), "a workgroup wrote no word"


def test_store_and_null_probes(probe):
    buf = torch.full((1 << 20,), 7, dtype=torch.int32, device=dev())
    assert probe.spd_probe_store(buf.data_ptr(), 4 << 20, 256, stream()) == 0
    assert probe.spd_probe_null(256, stream()) == 0
    torch.cuda.synchronize()
    assert torch.all(buf == 0)

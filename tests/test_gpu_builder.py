"""GPU decode index builder (HIP, through the C ABI) against the oracle's
builder: bit-exact kv_indptr and kv_indices, including padded tokens, empty
rings, full rings, all-sentinel rows and batches larger than one scan chunk."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import device_builder_inputs, log, random_builder_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def check(spd, b: W.BuilderInputs, what: str):
    log("case builder %s" % what)
    ss, sl, cp, bt = device_builder_inputs(b)
    ptr, idx = spd.build_decode_indices(ss, sl, cp, bt, b.win, b.k_per_block, b.swa_pages)
    torch.cuda.synchronize()
    optr, oidx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos, b.block_table,
                                             b.win, b.k_per_block, b.swa_pages)
    gptr = ptr.cpu().numpy()
    assert np.array_equal(gptr, optr), what
    assert np.array_equal(idx.cpu().numpy()[:optr[-1]], oidx), what


@pytest.mark.parametrize("seed,N,win,topk,k,mb,nb", [
    (0, 1, 4, 3, 1, 3, 5),
    (1, 7, 16, 10, 4, 3, 9),
    (2, 64, 128, 512, 1, 512, 4000),
    (3, 300, 32, 100, 8, 13, 50),
    (4, 3000, 8, 70, 16, 5, 40),      # several 1024-token scan chunks
    (5, 1025, 128, 64, 64, 1, 100),
    (6, 200, 64, 512, 8, 64, 100),    # N * topk above the one-launch limit, N <= 1024
    (7, 2, 8, 5000, 4, 1300, 500),    # one-launch kernel: a wave's part spans 3 batches
    (8, 3, 8, 2047, 2, 1100, 300),    # the same with rows of one entry per load
])
def test_random_bit_exact(spd, seed, N, win, topk, k, mb, nb):
    check(spd, random_builder_inputs(seed, N, win, topk, k, mb, nb), "random N=%d" % N)


def test_window_only(spd):
    b = W.BuilderInputs(np.array([3, 0, 1], dtype=np.int32), np.array([2, 0, 5], dtype=np.int32),
                        None, None, 5, 1, 20)
    log("case builder window only")
    ss, sl, _, _ = device_builder_inputs(b)
    ptr, idx = spd.build_decode_indices(ss, sl, None, None, 5, 1, 20)
    torch.cuda.synchronize()
    assert ptr.cpu().tolist() == [0, 2, 2, 7]
    assert idx.cpu().tolist()[:7] == [15, 16, 5, 6, 7, 8, 9]


def test_decode_base_config(spd):
    check(spd, W.decode_base().builder, "decode_base")


def test_hand_worked_example(spd):
    """The hand-derived fixture tests/golden/builder_worked_example.json."""
    import golden_cases
    c = golden_cases.builder_case()
    b = W.BuilderInputs(c["state_slot"], c["swa_len"], c["comp_pos"], c["block_table"], c["win"],
                        c["k_per_block"], c["swa_pages"])
    log("case builder hand example")
    ss, sl, cp, bt = device_builder_inputs(b)
    ptr, idx = spd.build_decode_indices(ss, sl, cp, bt, b.win, b.k_per_block, b.swa_pages)
    torch.cuda.synchronize()
    n = int(c["kv_indptr"][-1])
    assert ptr.cpu().tolist() == c["kv_indptr"].tolist()
    assert idx.cpu().tolist()[:n] == c["kv_indices"].tolist()


def test_defensive_rules_and_unaligned_rows(spd):
    """Out-of-contract metadata takes the documented device rule: swa_len is
    clamped to [0, win] and a comp_pos entry whose block lookup falls outside
    [0, max_blocks) (or any negative entry) is dropped.  Expected output: the
    oracle's builder under that rule (clamp=True).  The comp_pos rows are passed as a view one
    int32 past a 16-byte boundary with topk % 4 == 0, so the 4-entries-per-load
    path must not be taken."""
    rng = np.random.default_rng(77)
    N, win, topk, k, mb, nb = 40, 16, 64, 4, 6, 30
    b = random_builder_inputs(78, N, win, topk, k, mb, nb)
    cp = b.comp_pos.copy()
    cp[rng.random(cp.shape) < 0.1] = mb * k + rng.integers(0, 50)      # beyond the table
    cp[rng.random(cp.shape) < 0.05] = -7
    sl = b.swa_len.copy()
    sl[:3] = [-2, win + 5, win]
    optr, oidx = oracle.build_decode_indices(b.state_slot, sl, cp, b.block_table, win, k,
                                             b.swa_pages, clamp=True)
    log("case builder defensive rules")
    d = torch.device("cuda:0")
    flat = torch.zeros(cp.size + 1, dtype=torch.int32, device=d)
    flat[1:] = torch.from_numpy(cp.reshape(-1)).to(d)
    cp_view = flat[1:].view(N, topk)                 # data pointer 4 bytes past the allocation
    assert cp_view.data_ptr() % 16 != 0
    ss = torch.from_numpy(b.state_slot).to(d)
    sld = torch.from_numpy(sl.astype(np.int32)).to(d)
    bt = torch.from_numpy(b.block_table).to(d)
    ptr, idx = spd.build_decode_indices(ss, sld, cp_view, bt, win, k, b.swa_pages)
    torch.cuda.synchronize()
    assert np.array_equal(ptr.cpu().numpy(), optr)
    assert np.array_equal(idx.cpu().numpy()[:optr[-1]], oidx)

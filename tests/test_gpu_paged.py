"""GPU parity of sparse_decode_attn_paged, the attention call with the page
transform fused in (through the C ABI): its output must equal, bit for bit,
build_decode_indices followed by sparse_decode_attn in the same mode (same
rows, visited in the same order), and the oracle (the oracle's builder, then
its attention) within |d| <= 1e-2 + 1e-2|ref|.  Cases cover every kind of
token the builder handles -- window-only, compressed-only, sentinels, entries
outside the block table (dropped), padded tokens -- in both work
decompositions, several (H, D), block sizes 1..64 and the longest list the
call accepts (win + topk = 2048)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (assert_close, bf16_to_f64, dev, device_builder_inputs, log,
                         oracle_tokens, random_builder_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def workload_for(b: W.BuilderInputs, H: int, D: int, seed: int, n_blocks: int) -> W.Workload:
    """q, pool and sinks for builder inputs b; the pool holds every slot b can produce."""
    rng = np.random.Generator(np.random.PCG64(seed))
    N = b.state_slot.shape[0]
    P = b.swa_pages + n_blocks * b.k_per_block
    sink = rng.standard_normal(H).astype(np.float32)
    return W.Workload(name="paged", N=N, H=H, D=D, P=P, q_bits=W.normal_bf16(rng, (N, H, D)),
                      kv_bits=W.normal_bf16(rng, (P, D)), attn_sink=sink,
                      softmax_scale=float(np.float32(1.0 / np.sqrt(D))),
                      max_len=b.win + b.topk, builder=b)


def run_both(spd, w: W.Workload, mode: int):
    """(paged output, two-call output, oracle kv_indptr, oracle kv_indices)."""
    b = w.builder
    d = dev()
    ss, sl, cp, bt = device_builder_inputs(b)
    q = W.device_bits(w.q_bits, d)
    kv = W.device_bits(w.kv_bits, d)
    sink = torch.from_numpy(w.attn_sink).to(d)
    fused = spd.sparse_decode_attn_paged(q, kv, ss, sl, cp, bt, b.win, b.k_per_block, b.swa_pages,
                                         sink, w.softmax_scale, mode=mode)
    ptr, idx = spd.build_decode_indices(ss, sl, cp, bt, b.win, b.k_per_block, b.swa_pages)
    two = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, mode=mode)
    torch.cuda.synchronize()
    # the builder's device-side rule for metadata outside its preconditions
    # (swa_len clamped to [0, win], entries past the block table dropped) is
    # the oracle's clamping form
    optr, oidx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos, b.block_table,
                                             b.win, b.k_per_block, b.swa_pages, clamp=True)
    return fused, two, optr, oidx


def check(spd, w: W.Workload, mode: int, what: str, tokens=None):
    log("case paged %s mode=%d" % (what, mode))
    fused, two, optr, oidx = run_both(spd, w, mode)
    assert torch.equal(fused.view(torch.int16), two.view(torch.int16)), \
        "%s: paged call differs from build + attention" % what
    L = np.diff(optr)
    zero = np.nonzero(L == 0)[0]
    if len(zero):  # padded tokens: exactly +0.0
        assert torch.all(fused[torch.from_numpy(zero).to(fused.device)].view(torch.int16) == 0)
    ref = oracle_tokens(w, oidx, optr, tokens)
    got = fused if tokens is None else fused[torch.from_numpy(np.asarray(tokens)).to(fused.device)]
    assert_close(bf16_to_f64(got), ref, "%s mode=%d" % (what, mode))


@pytest.mark.parametrize("mode", [1, 2, 3])
@pytest.mark.parametrize("seed,N,H,D,win,topk,k,mb,nb", [
    (11, 9, 8, 64, 16, 24, 4, 3, 9),
    (12, 20, 64, 512, 128, 512, 1, 512, 3000),
    (13, 33, 16, 128, 32, 100, 8, 13, 50),
    (14, 6, 128, 256, 64, 300, 64, 5, 40),
    (15, 5, 64, 512, 128, 1920, 16, 120, 200),   # the longest list: win + topk = 2048
    (16, 12, 24, 64, 8, 70, 2, 40, 90),
])
def test_random_inputs(spd, mode, seed, N, H, D, win, topk, k, mb, nb):
    if mode == 3 and H % 64:
        pytest.skip("the 32-head-wave mode needs H % 64 == 0")
    b = random_builder_inputs(seed, N, win, topk, k, mb, nb)
    # a few entries past the block table: the builder drops them, so must the paged call
    b.comp_pos[0, : min(3, topk)] = mb * k + np.arange(min(3, topk), dtype=np.int32)
    check(spd, workload_for(b, H, D, seed + 1000, nb), mode, "random N=%d H=%d D=%d" % (N, H, D))


@pytest.mark.parametrize("mode", [1, 2])
def test_window_only(spd, mode):
    # swa_len 9 > win is clamped to the full ring, -2 to an empty one
    b = W.BuilderInputs(np.array([3, 0, 1, 2, 0], dtype=np.int32),
                        np.array([2, 0, 5, 9, -2], dtype=np.int32), None, None, 5, 1, 20)
    check(spd, workload_for(b, 8, 64, 7, 0), mode, "window only")


@pytest.mark.parametrize("mode", [1, 2])
def test_compressed_only_and_all_padded(spd, mode):
    rng = np.random.default_rng(3)
    N, win, topk, k, mb, nb = 6, 16, 40, 4, 10, 30
    cp = rng.integers(0, mb * k, size=(N, topk)).astype(np.int32)
    cp[2] = -1                                  # token 2: nothing at all
    b = W.BuilderInputs(np.arange(N, dtype=np.int32), np.zeros(N, dtype=np.int32), cp,
                        rng.integers(0, nb, size=(N, mb)).astype(np.int32), win, k, N * win)
    check(spd, workload_for(b, 16, 128, 8, nb), mode, "compressed only")
    b2 = W.BuilderInputs(np.arange(N, dtype=np.int32), np.zeros(N, dtype=np.int32),
                         np.full((N, topk), -1, dtype=np.int32), b.block_table, win, k, N * win)
    check(spd, workload_for(b2, 16, 128, 9, nb), mode, "all padded")


def test_decode_base_config(spd):
    w = W.decode_base()
    for mode in (0, 1, 2, 3):
        check(spd, w, mode, "decode_base")


def test_large_config(spd):
    W.set_data_mode("device", dev())
    try:
        w = W.large()
    finally:
        W.set_data_mode("host")
    log("case paged large")
    fused, two, optr, oidx = run_both(spd, w, 0)
    assert torch.equal(fused.view(torch.int16), two.view(torch.int16))
    tokens = np.array([0, 1, 511, 777, 1023])
    ref = oracle_tokens(w, oidx, optr, tokens)
    assert_close(bf16_to_f64(fused[torch.from_numpy(tokens).to(fused.device)]), ref, "large paged")


def test_graph_capture_and_replay(spd):
    """Capture the paged call once; replay with new window lengths and sentinel
    patterns copied into the same buffers; each replay equals the eager call."""
    N, H, D, P, win, topk = 24, 64, 512, 65536, 128, 512
    w = W.window_plus_compressed("paged graph", 22, N, H, D, P, win, topk, 1)
    b = w.builder
    ss, sl, cp, bt = device_builder_inputs(b)
    q = W.device_bits(w.q_bits, dev())
    kv = W.device_bits(w.kv_bits, dev())
    sink = torch.from_numpy(w.attn_sink).to(dev())
    out = torch.zeros((N, H, D), dtype=torch.bfloat16, device=dev())
    log("case paged graph capture")

    def step():
        spd.sparse_decode_attn_paged(q, kv, ss, sl, cp, bt, win, 1, b.swa_pages, sink,
                                     w.softmax_scale, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    for rep in range(3):
        new_sl = rng.integers(0, win + 1, size=N).astype(np.int32)
        new_cp = b.comp_pos.copy()
        new_cp[rng.random((N, topk)) < 0.25] = -1
        sl.copy_(torch.from_numpy(new_sl))
        cp.copy_(torch.from_numpy(new_cp))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(replayed.view(torch.int16), out.view(torch.int16)), "replay %d" % rep

"""GPU parity at the benchmark configurations' full sizes: every token of
decode_base, ragged, large and prefill against the fp64 oracle (in chunks of
tokens, to bound host memory), in the launch configuration the benchmark
times; the other plans on sampled tokens that always include the longest,
shortest and empty slices; a small batch of long slices on the split plan;
plus HIP-graph capture and replay of builder + attention with fixed-shape
buffers whose contents change between replays."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (assert_close, bf16_to_f64, dev, device_builder_inputs, device_csr,
                         device_inputs, log, oracle_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


@pytest.fixture
def device_data():
    W.set_data_mode("device", dev())
    yield
    W.set_data_mode("host")


def sample_tokens(indptr: np.ndarray, n: int, seed: int) -> np.ndarray:
    L = np.diff(indptr)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(len(L), size=min(n, len(L)), replace=False).tolist())
    pick |= {int(np.argmax(L)), int(np.argmin(L)), 0, len(L) - 1}
    nz = np.nonzero(L)[0]
    if len(nz):
        pick.add(int(nz[np.argmin(L[nz])]))
    return np.array(sorted(pick))


def check_all_tokens(w, indices, indptr, out, what, chunk=512):
    """Every token of `out` against the oracle, chunk tokens at a time."""
    N = len(indptr) - 1
    worst = 0.0
    for t0 in range(0, N, chunk):
        toks = np.arange(t0, min(N, t0 + chunk))
        ref = oracle_tokens(w, indices, indptr, toks)
        got = bf16_to_f64(out[t0:t0 + len(toks)])
        err = np.abs(got - ref)
        bound = 1e-2 + 1e-2 * np.abs(ref)
        assert_close(got, ref, "%s tokens %d..%d" % (what, t0, toks[-1]))
        worst = max(worst, float((err / bound).max()) if err.size else 0.0)
    log("  %s: all %d tokens, max err/bound %.3f" % (what, N, worst))


def build_on_gpu(spd, b):
    ss, sl, cp, bt = device_builder_inputs(b)
    ptr, idx = spd.build_decode_indices(ss, sl, cp, bt, b.win, b.k_per_block, b.swa_pages)
    torch.cuda.synchronize()
    optr, oidx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos, b.block_table,
                                             b.win, b.k_per_block, b.swa_pages)
    assert np.array_equal(ptr.cpu().numpy(), optr)
    assert np.array_equal(idx.cpu().numpy()[:optr[-1]], oidx)
    return ptr, idx, optr, oidx


def test_decode_base_end_to_end(spd):
    w = W.decode_base()
    log("case decode_base: builder + attention, all 64 tokens")
    ptr, idx, optr, oidx = build_on_gpu(spd, w.builder)
    ref = oracle_tokens(w, oidx, optr)
    q, kv, sink = device_inputs(w)
    for plan in [dict(max_len=640), dict(plain=True), dict(mode=1, max_len=640),
                 dict(max_len=640, split_rows=64), dict(max_len=640, split_rows=320),
                 dict(mode=4, max_len=640), dict(mode=4, max_len=640, split_rows=128)]:
        out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, **plan)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out), ref, "decode_base %s" % plan)


def test_ragged_config(spd, device_data):
    w = W.ragged()
    log("case ragged: N=256, L up to 2048, 25% padded")
    tokens = sample_tokens(w.kv_indptr, 40, 1)
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr, tokens)
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    # the launch the benchmark times: every token
    out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, max_len=w.max_len)
    torch.cuda.synchronize()
    check_all_tokens(w, w.kv_indices, w.kv_indptr, out, "ragged")
    # the split plans take the XCD-strided partition order (256 tokens, one head group)
    for plan in [dict(plain=True), dict(mode=2), dict(mode=1, max_len=w.max_len),
                 dict(max_len=w.max_len, split_rows=768), dict(max_len=w.max_len, split_rows=384),
                 dict(mode=4, max_len=w.max_len, split_rows=512)]:
        out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, **plan)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out[torch.from_numpy(tokens).cuda()]), ref, "ragged %s" % plan)
        assert torch.all(out[192:].view(torch.int16) == 0)


def test_large_config(spd, device_data):
    w = W.large()
    log("case large: N=1024, H=128, 4 GiB pool, K_PER_BLOCK=64")
    ptr, idx, optr, oidx = build_on_gpu(spd, w.builder)
    q, kv, sink = device_inputs(w)
    out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, max_len=w.max_len)
    torch.cuda.synchronize()
    check_all_tokens(w, oidx, optr, out, "large", chunk=256)


def test_prefill_config(spd, device_data):
    w = W.prefill()
    log("case prefill: N=8192, L up to 640, sliding reuse")
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, max_len=w.max_len)
    torch.cuda.synchronize()
    check_all_tokens(w, w.kv_indices, w.kv_indptr, out, "prefill", chunk=1024)


def test_long_slices_small_batch_split(spd):
    """A few long slices (the case the automatic plan splits): every token
    against the oracle, on the automatic (split) plan and on rows mode."""
    lengths = [2048, 4000, 0, 3333, 1, 4096, 2500, 129]
    w = W.random_csr("long_small", 41, len(lengths), 64, 512, 40000, lengths)
    log("case long slices, small batch")
    plan = spd.sparse_decode_attn_plan_info(w.N, w.H, w.D, 4096)
    assert plan["mode"] == "split" and plan["splits"] > 1
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    for p in [dict(max_len=4096), dict(mode=2)]:
        out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, **p)
        torch.cuda.synchronize()
        check_all_tokens(w, w.kv_indices, w.kv_indptr, out, "long small %s" % p)


@pytest.mark.parametrize("mode", [1, 2])
def test_graph_capture_and_replay(spd, mode):
    """Capture builder + attention once; replay with new window lengths and
    sentinel patterns copied into the same buffers; every replay must equal the
    eager result bit for bit and the oracle within tolerance."""
    N, H, D, P, win, topk = 24, 64, 512, 65536, 128, 512
    w = W.window_plus_compressed("graph", 21, N, H, D, P, win, topk, 1)
    b = w.builder
    ss, sl, cp, bt = device_builder_inputs(b)
    q, kv, sink = device_inputs(w)
    cap = N * (win + topk)
    ptr = torch.zeros(N + 1, dtype=torch.int32, device=dev())
    idx = torch.zeros(cap, dtype=torch.int32, device=dev())
    out = torch.zeros((N, H, D), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(max(16, spd.sparse_decode_attn_workspace_size(N, H, D, win + topk, 0, 1)),
                     dtype=torch.uint8, device=dev())
    log("case graph capture")

    def step():
        spd.build_decode_indices(ss, sl, cp, bt, win, 1, b.swa_pages, kv_indptr=ptr, kv_indices=idx)
        spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, out=out,
                               max_len=win + topk, workspace=ws, mode=mode)

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

    rng = np.random.default_rng(5)
    for rep in range(4):
        new_sl = rng.integers(0, win + 1, size=N).astype(np.int32)
        new_sl[rng.random(N) < 0.2] = 0
        new_cp = b.comp_pos.copy()
        new_cp[rng.random((N, topk)) < rng.random()] = -1
        new_cp[rng.random(N) < 0.2] = -1
        sl.copy_(torch.from_numpy(new_sl))
        cp.copy_(torch.from_numpy(new_cp))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        graph_out = out.clone()
        graph_ptr = ptr.clone()
        # eager, into fresh buffers, with some unrelated eager work in between
        _ = torch.randn(1 << 20, device=dev()).sum()
        eptr, eidx = spd.build_decode_indices(ss, sl, cp, bt, win, 1, b.swa_pages)
        eout = spd.sparse_decode_attn(q, kv, eidx, eptr, sink, w.softmax_scale, max_len=win + topk,
                                      mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(graph_ptr, eptr)
        assert torch.equal(graph_out.view(torch.int16), eout.view(torch.int16)), "replay %d" % rep
        optr, oidx = oracle.build_decode_indices(b.state_slot, new_sl, new_cp, b.block_table, win, 1,
                                                 b.swa_pages)
        assert np.array_equal(graph_ptr.cpu().numpy(), optr)
        toks = np.array([0, 5, 11, N - 1])
        ref = oracle_tokens(w, oidx, optr, toks)
        assert_close(bf16_to_f64(graph_out[torch.from_numpy(toks).cuda()]), ref, "graph replay %d" % rep)

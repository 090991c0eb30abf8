"""Graph capture of the calls added beside the decode attention (FP8 attention,
the quantising store, the producer, the shared-window prefill, the split
plan with its in-kernel merge on a reused workspace): each is
captured once into a HIP graph and replayed several times, with new inputs
copied into the captured buffers and eager work between replays; every replay
must equal the eager call on the same inputs bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def bits_tensor(rng, shape, std=1.0):
    return W.device_bits(W.normal_bf16(rng, shape, std=std), dev())


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_equals_eager(g, fn, outs, refresh, reps=3):
    for rep in range(reps):
        refresh(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        fn()
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d" % rep


def test_fp8_attention_and_store(spd):
    log("case graph fp8")
    rng = np.random.default_rng(31)
    N, H, D, P = 16, 64, 512, 4096
    src = bits_tensor(rng, (P, D))
    kv8 = torch.empty((P, D), dtype=torch.uint8, device=dev())
    ksc = torch.empty(P, dtype=torch.float32, device=dev())
    q = bits_tensor(rng, (N, H, D))
    idx, ptr = W.csr_from_lists([rng.integers(0, P, size=L) for L in rng.integers(0, 700, size=N)])
    idx_d = torch.from_numpy(idx).to(dev())
    ptr_d = torch.from_numpy(ptr).to(dev())
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(dev())
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev())

    def step():
        spd.quantize_kv_fp8(src, kv8, ksc)
        spd.sparse_decode_attn_fp8(q, kv8, ksc, idx_d, ptr_d, sink, 0.05, out=out)

    g = capture(step)

    def refresh(rep):
        r = np.random.default_rng(100 + rep)
        src.copy_(bits_tensor(r, (P, D), std=1.0 + rep))
        q.copy_(bits_tensor(r, (N, H, D)))

    replay_equals_eager(g, step, [out, kv8, ksc], refresh)


def test_producer(spd):
    log("case graph producer")
    rng = np.random.default_rng(32)
    N, H, D, win, max_pos = 24, 64, 512, 16, 256
    q = bits_tensor(rng, (N, H, D))
    kv = bits_tensor(rng, (N, D))
    qw = torch.from_numpy((1 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev())
    kw = torch.from_numpy((1 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev())
    ang = np.arange(max_pos)[:, None] * 10000.0 ** (-np.arange(32) / 32.0)
    cs = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).to(dev())
    pos = torch.from_numpy(rng.integers(0, max_pos, size=N).astype(np.int32)).to(dev())
    slot = torch.arange(N, dtype=torch.int32, device=dev())
    pool = torch.zeros((N * win, D), dtype=torch.bfloat16, device=dev())
    kv8 = torch.zeros((N * win, D), dtype=torch.uint8, device=dev())
    ksc = torch.zeros(N * win, dtype=torch.float32, device=dev())
    q_out = torch.empty_like(q)

    def step():
        spd.fused_qk_norm_rope_swa_store(q, kv, qw, kw, 1e-6, pos, cs, slot, win, unified_kv=pool,
                                         kv_fp8=kv8, kv_scale=ksc, q_out=q_out)

    g = capture(step)

    def refresh(rep):
        r = np.random.default_rng(200 + rep)
        q.copy_(bits_tensor(r, (N, H, D)))
        kv.copy_(bits_tensor(r, (N, D)))
        pos.copy_(torch.from_numpy(r.integers(0, max_pos, size=N).astype(np.int32)))

    replay_equals_eager(g, step, [q_out, pool, kv8, ksc], refresh)


@pytest.mark.parametrize("group", [1, 2])
def test_prefill(spd, group):
    log("case graph prefill group=%d" % group)
    rng = np.random.default_rng(33)
    N, H, D, P = 40, 64, 512, 6000
    L = rng.integers(1, 500, size=N)
    start = np.zeros(N, dtype=np.int64)
    for t in range(1, N):
        start[t] = start[t - 1] + -(-int(L[t - 1]) // 10)
    stream = torch.from_numpy(rng.integers(0, P, size=int((start + L).max())).astype(np.int32)).to(dev())
    ws = torch.from_numpy(start.astype(np.int32)).to(dev())
    wl = torch.from_numpy(L.astype(np.int32)).to(dev())
    q = bits_tensor(rng, (N, H, D))
    kv = bits_tensor(rng, (P, D))
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(dev())
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev())

    def step():
        spd.sparse_prefill_attn(q, kv, stream, ws, wl, sink, 0.05, out=out, tokens_per_group=group)

    g = capture(step)

    def refresh(rep):
        r = np.random.default_rng(300 + rep)
        q.copy_(bits_tensor(r, (N, H, D)))
        wl.copy_(torch.from_numpy(np.maximum(L - r.integers(0, 50, size=N), 0).astype(np.int32)))

    replay_equals_eager(g, step, [out], refresh)


def test_split_plan_reused_workspace(spd):
    """The split plan in a graph: 5 tokens x 5 partitions of 96 rows (25
    workgroups, so a token's partitions fall on different XCDs), one
    workspace for the eager calls and the replays (its arrival counters must
    come back to zero after every call)."""
    import math
    log("case graph split")
    rng = np.random.default_rng(33)
    N, H, D, P, max_len = 5, 64, 512, 3000, 400
    q = bits_tensor(rng, (N, H, D))
    kv = bits_tensor(rng, (P, D))
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(dev())
    lengths = np.array([400, 97, 0, 333, 250], dtype=np.int64)
    indptr = np.zeros(N + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(lengths)
    idx = torch.from_numpy(rng.integers(0, P, size=int(lengths.sum())).astype(np.int32)).to(dev())
    ptr = torch.from_numpy(indptr).to(dev())
    plan = spd.sparse_decode_attn_plan_info(N, H, D, max_len, 96, spd.MODE_SPLIT)
    assert plan["mode"] == "split" and plan["splits"] == 5
    ws = torch.zeros(spd.sparse_decode_attn_workspace_size(N, H, D, max_len, 96, spd.MODE_SPLIT),
                     dtype=torch.uint8, device=dev())
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev())

    def fn():
        spd.sparse_decode_attn(q, kv, idx, ptr, sink, 1 / math.sqrt(D), out=out, max_len=max_len,
                               split_rows=96, mode=spd.MODE_SPLIT, workspace=ws)

    g = capture(fn)

    def refresh(rep):
        idx.copy_(torch.from_numpy(rng.integers(0, P, size=idx.numel()).astype(np.int32)))
        q.copy_(bits_tensor(rng, (N, H, D)))

    replay_equals_eager(g, fn, [out], refresh, reps=4)
    torch.cuda.synchronize()
    nctr = N * 4
    assert torch.all(ws[-4 * nctr:].view(torch.int32) == 0), "arrival counters left nonzero"

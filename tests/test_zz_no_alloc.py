"""sparse_decode_attn_noalloc (the library's per-GPU workspace, no allocation)
against sparse_decode_attn_ex (a caller workspace) through the C ABI: the
same plan on the same inputs gives the same bits, on calls in a row whose
plans differ and shrink (so each call finds the array as the previous call
left it), with every token also checked against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, bf16_to_f64, device_csr, device_inputs, log, oracle_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def run_pair(spd, w, **plan):
    """One call of each entry point with the same plan; returns both outputs."""
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    info = spd.sparse_decode_attn_plan_info(w.N, w.H, w.D, plan.get("max_len", 0),
                                            plan.get("split_rows", 0), plan.get("mode", 0))
    log("  noalloc %s: N=%d plan %s" % (w.name, w.N, info))
    need = spd.sparse_decode_attn_workspace_size(w.N, w.H, w.D, plan.get("max_len", 0),
                                                 plan.get("split_rows", 0), plan.get("mode", 0))
    assert need <= spd.NOALLOC_WORKSPACE_BYTES
    out_na = torch.full((w.N, w.H, w.D), float("nan"), dtype=torch.bfloat16, device=q.device)
    spd.sparse_decode_attn_noalloc(q, kv, idx, ptr, sink, w.softmax_scale, out_na, **plan)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    out_ex = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, workspace=ws, **plan)
    torch.cuda.synchronize()
    return info, out_na, out_ex


def check(w, info, out_na, out_ex, what):
    assert torch.equal(out_na.view(torch.int16), out_ex.view(torch.int16)), \
        "%s: noalloc and ex differ (plan %s)" % (what, info)
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    assert_close(bf16_to_f64(out_na), ref, what)


def test_noalloc_matches_ex_on_calls_in_a_row(spd):
    MODE_HEADS, MODE_SPLIT = spd.MODE_HEADS, spd.MODE_SPLIT
    cases = [
        # heads-mode split-L first: its partials fill the array where the
        # split plans below keep their arrival counters
        # (64 tokens x 8 partitions x 64 heads x 514 floats: 67 MB, past the
        # 34 MB at which the next plan's counters start)
        ("heads_big", dict(N=64, lengths=None, max_len=2048),
         dict(max_len=2048, split_rows=256, mode=MODE_HEADS), "heads"),
        # the automatic plan of a small batch of long slices: split mode, 32 partitions
        ("split_big", dict(N=8, lengths=[4096, 0, 3000, 1, 4095, 2222, 4096, 777], max_len=4096),
         dict(max_len=4096), "split"),
        # the same entry point again, smaller: 3 tokens, 6 partitions of 256 rows
        ("split_small", dict(N=3, lengths=[1500, 64, 0], max_len=1500),
         dict(max_len=1500, split_rows=256, mode=MODE_SPLIT), "split"),
        # and heads-mode split-L, smaller
        ("heads_small", dict(N=5, lengths=None, max_len=600),
         dict(max_len=600, split_rows=128, mode=MODE_HEADS), "heads"),
        # a plan with no workspace at all
        ("rows", dict(N=4, lengths=[640, 0, 17, 300], max_len=640), dict(max_len=640), "rows"),
    ]
    for i, (name, shape, plan, mode_name) in enumerate(cases):
        rng = np.random.default_rng(100 + i)
        lengths = shape["lengths"]
        if lengths is None:
            lengths = rng.integers(0, shape["max_len"] + 1, size=shape["N"]).tolist()
            lengths[0] = shape["max_len"]
        w = W.random_csr(name, 200 + i, shape["N"], 64, 512, 50000, lengths)
        info, out_na, out_ex = run_pair(spd, w, **plan)
        assert info["mode"] == mode_name, info
        if mode_name != "rows":
            assert info["splits"] > 1, info
        check(w, info, out_na, out_ex, name)


def test_noalloc_split_plan_in_a_graph(spd):
    """The allocation-free call captured in a HIP graph (its use case): the
    split plan of 6 tokens of up to 3000 rows, whose counter-clearing kernel
    and attention kernel are both graph nodes, replayed four times on new
    inputs, each replay equal bit for bit to sparse_decode_attn_ex on the
    same inputs; an eager call of another plan between replays reuses the
    array in between."""
    rng = np.random.default_rng(77)
    N, H, D, P, max_len = 6, 64, 512, 20000, 3000
    lengths = np.array([3000, 17, 0, 2500, 1, 2999])
    indptr = np.zeros(N + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(lengths)
    dev = torch.device("cuda:0")
    bits = lambda shape: torch.from_numpy(
        W.normal_bf16(rng, shape).view(np.int16)).to(dev).view(torch.bfloat16)
    q, kv = bits((N, H, D)), bits((P, D))
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(dev)
    idx = torch.from_numpy(rng.integers(0, P, size=int(lengths.sum())).astype(np.int32)).to(dev)
    ptr = torch.from_numpy(indptr).to(dev)
    scale = 1.0 / np.sqrt(D)
    info = spd.sparse_decode_attn_plan_info(N, H, D, max_len)
    assert info["mode"] == "split" and info["splits"] > 1, info
    out = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)

    def call():
        spd.sparse_decode_attn_noalloc(q, kv, idx, ptr, sink, scale, out, max_len=max_len)

    # warm-up outside capture, then capture on a side stream
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    ws = torch.zeros(spd.sparse_decode_attn_workspace_size(N, H, D, max_len), dtype=torch.uint8,
                     device=dev)
    other = torch.empty((3, H, D), dtype=torch.bfloat16, device=dev)
    for rep in range(4):
        log("  noalloc graph replay %d" % rep)
        q.copy_(bits((N, H, D)))
        idx.copy_(torch.from_numpy(rng.integers(0, P, size=idx.numel()).astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = spd.sparse_decode_attn(q, kv, idx, ptr, sink, scale, max_len=max_len, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "replay %d" % rep
        # another plan through the same array between replays (heads-mode split-L)
        spd.sparse_decode_attn_noalloc(q[:3], kv, idx, ptr[:4], sink, scale, other, max_len=3000,
                                       split_rows=256, mode=spd.MODE_HEADS)
        torch.cuda.synchronize()

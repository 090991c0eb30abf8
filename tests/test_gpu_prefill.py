"""GPU parity of sparse_prefill_attn (through the C ABI): token t attends to the
window kv_stream[win_start[t] : + win_len[t]] of one index stream.  The oracle is
the decode oracle on the same lists written out as CSR (the lists, not the
method, are converted).  Acceptance |d| <= 1e-2 + 1e-2 |ref|; empty and invalid
windows give exactly +0.0.

Cases: sliding windows of the prefill workload's shape at small N for every
supported H and every grouping (1, 2 or 4 tokens a workgroup) and D; an odd batch (a
group with a missing token); empty, negative and out-of-stream windows; windows
that do not overlap; windows longer than the 2048 indices staged at a time;
a -inf sink; rows planted late in a window that force the second pass; and the
prefill workload at full size (N=8192), sampled."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, bf16_to_f64, dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def t32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def windows_as_csr(stream, start, length):
    """The windows' lists written out as CSR (an empty list where a window is
    empty or leaves the stream)."""
    lists = []
    for s, l in zip(start.tolist(), length.tolist()):
        ok = s >= 0 and l > 0 and s + l <= len(stream)
        lists.append(stream[s:s + l] if ok else np.zeros(0, dtype=np.int32))
    return W.csr_from_lists(lists)


def sliding(rng, N, max_len, P, reuse=10):
    L = rng.integers(1, max_len + 1, size=N)
    start = np.zeros(N, dtype=np.int64)
    for t in range(1, N):
        start[t] = start[t - 1] + -(-int(L[t - 1]) // reuse)
    stream = rng.integers(0, P, size=int((start + L).max())).astype(np.int32)
    return stream, start.astype(np.int32), L.astype(np.int32)


def run_case(spd, stream, start, length, H, D, P, seed, what, sink=None, kv_bits=None,
             q_bits=None, tokens=None, group=0):
    rng = np.random.default_rng(seed)
    N = len(start)
    q_bits = W.normal_bf16(rng, (N, H, D)) if q_bits is None else q_bits
    kv_bits = W.normal_bf16(rng, (P, D)) if kv_bits is None else kv_bits
    sink = rng.standard_normal(H).astype(np.float32) if sink is None else sink
    scale = float(np.float32(1.0 / np.sqrt(D)))
    dev_bits = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev()).view(torch.bfloat16)
    out = spd.sparse_prefill_attn(dev_bits(q_bits), dev_bits(kv_bits), t32(stream), t32(start),
                                  t32(length), torch.from_numpy(sink).to(dev()), scale,
                                  tokens_per_group=group)
    torch.cuda.synchronize()
    idx, ptr = windows_as_csr(stream, start, length)
    if tokens is None:
        ref = oracle.sparse_decode_attn(q_bits, kv_bits, idx, ptr, sink, scale)
        got = bf16_to_f64(out)
    else:
        ref = oracle.sparse_decode_attn(q_bits, kv_bits, idx, ptr, sink, scale, tokens=tokens)
        got = bf16_to_f64(out[torch.from_numpy(np.asarray(tokens)).to(dev())])
    assert_close(got, ref, what)
    empty = np.nonzero(np.diff(ptr) == 0)[0]
    if len(empty) and tokens is None:
        assert torch.all(out[torch.from_numpy(empty).to(dev())].view(torch.int16) == 0), what
    return out


@pytest.mark.parametrize("H,group", [(32, 0), (32, 2), (32, 4), (64, 0), (64, 1), (64, 2),
                                     (128, 0)])
@pytest.mark.parametrize("D", [64, 512])
def test_sliding_windows(spd, H, group, D):
    log("case prefill sliding H=%d D=%d group=%d" % (H, D, group))
    rng = np.random.default_rng(H + D)
    stream, start, length = sliding(rng, 23, 200, 3000)
    run_case(spd, stream, start, length, H, D, 3000, H * D, "sliding H=%d D=%d" % (H, D),
             group=group)


def test_empty_invalid_and_disjoint_windows(spd):
    log("case prefill empty / invalid / disjoint")
    rng = np.random.default_rng(3)
    P = 2000
    stream = rng.integers(0, P, size=5000).astype(np.int32)
    start = np.array([10, 12, 0, 100, 4000, 4990, -3, 100, 3000, 20, 7], dtype=np.int32)
    length = np.array([50, 0, 70, 0, 300, 11, 5, 40, 33, 1, 900], dtype=np.int32)
    # token 1, 3: empty; 5: leaves the stream (4990 + 11 > 5000); 6: negative start;
    # tokens 4 and 8 are far from their group partners (disjoint windows)
    sink = rng.standard_normal(64).astype(np.float32)
    sink[:5] = -np.inf
    for group in (1, 2):
        run_case(spd, stream, start, length, 64, 256, P, 4, "empty/invalid/disjoint", sink=sink,
                 group=group)


def test_long_windows_cross_the_staging_chunk(spd):
    log("case prefill long windows")
    rng = np.random.default_rng(5)
    P = 8000
    stream = rng.integers(0, P, size=6000).astype(np.int32)
    start = np.array([0, 300, 2500, 2600, 100], dtype=np.int32)
    length = np.array([2500, 2400, 3000, 1, 4500], dtype=np.int32)
    for group in (1, 2):
        run_case(spd, stream, start, length, 64, 512, P, 6, "long windows", group=group)


def test_second_pass(spd):
    """Rows parallel to a token's q for head 0, late in its window: their scores
    lie far above the first tile, which takes the second pass."""
    log("case prefill second pass")
    rng = np.random.default_rng(7)
    P, H, D = 4000, 64, 512
    stream, start, length = sliding(rng, 9, 600, P)
    q_bits = W.normal_bf16(rng, (9, H, D))
    kv_bits = W.normal_bf16(rng, (P, D))
    q = W.bf16_to_f32(q_bits)
    for t in (0, 3, 8):
        if length[t] > 100:
            kv_bits[stream[start[t] + length[t] - 5]] = W.bf16_bits(4.0 * q[t, 0])
            kv_bits[stream[start[t] + length[t] - 40]] = W.bf16_bits(3.9 * q[t, 0])
    for group in (1, 2):
        run_case(spd, stream, start, length, H, D, P, 8, "second pass", kv_bits=kv_bits,
                 q_bits=q_bits, group=group)


def test_prefill_config_sampled(spd):
    """The prefill workload at full size (N=8192, H=64, D=512, pool 2^20 rows),
    q and the pool drawn on the device; sampled tokens against the oracle."""
    W.set_data_mode("device", dev())
    try:
        w = W.prefill()
    finally:
        W.set_data_mode("host")
    log("case prefill config")
    m = w.meta
    tokens = np.array([0, 1, 2, 4095, 4096, 8190, 8191])
    from gpu_helpers import oracle_tokens
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr, tokens)
    for group in (0, 2):
        out = spd.sparse_prefill_attn(w.q_bits, w.kv_bits, t32(m["stream"]), t32(m["win_start"]),
                                      t32(m["win_len"]), torch.from_numpy(w.attn_sink).to(dev()),
                                      w.softmax_scale, tokens_per_group=group)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out[torch.from_numpy(tokens).to(dev())]), ref,
                     "prefill config, group %d" % group)

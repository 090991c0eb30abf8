"""A seeded sweep of random shapes and plans through the C ABI, every token
against the oracle (|d| <= 1e-2 + 1e-2 |ref|), bf16 and FP8 pools.

Each case draws N, H, D, the pool size, a length mix (empty slices, single
rows, lengths around the 16-, 32- and 64-row tiles, long slices past the
indices staged at a time), the sinks (some -inf) and the softmax scale, then
runs the automatic plan and every explicit mode that applies to the shape
(rows, heads with and without split-L, 32-head waves, split mode with a
drawn partition length).  The cases are fixed by their seeds, so a failure
names a reproducible input."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, bf16_to_f64, dev, device_csr, device_inputs, log, oracle_tokens

pytestmark = pytest.mark.gpu

AUTO, HEADS, ROWS, WIDE, SPLIT = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128, 256, 512]))
    H = int(rng.choice([1, 3, 16, 20, 32, 48, 64, 64, 96, 128, 128]))
    N = int(rng.integers(1, 24))
    kinds = rng.integers(0, 6, size=N)
    lengths = []
    for k in kinds:
        if k == 0:
            lengths.append(0)
        elif k == 1:
            lengths.append(int(rng.integers(1, 4)))
        elif k == 2:
            lengths.append(int(rng.choice([15, 16, 17, 31, 32, 33, 63, 64, 65])))
        elif k == 3:
            lengths.append(int(rng.integers(1, 400)))
        elif k == 4:
            lengths.append(int(rng.integers(400, 1500)))
        else:
            lengths.append(int(rng.integers(1500, 2600)))
    P = int(rng.choice([500, 5000, 40000]))
    scale = float(np.float32(rng.choice([1.0 / np.sqrt(D), 0.02, 0.3])))
    return rng, N, H, D, P, lengths, scale


def plans_for(rng, H, D, max_len):
    out = [dict(plain=True), dict(max_len=max_len), dict(mode=ROWS), dict(mode=HEADS),
           dict(mode=HEADS, max_len=max_len, split_rows=int(rng.choice([32, 96, 256])))]
    if H % 64 == 0:
        out.append(dict(mode=WIDE))
    rows = int(rng.choice([64, 128, 320]))
    if max_len <= 32 * rows:  # at most 32 partitions
        out.append(dict(mode=SPLIT, max_len=max_len, split_rows=rows))
    out.append(dict(mode=SPLIT, max_len=max_len))
    return out


@pytest.mark.parametrize("seed", range(24))
def test_sweep_bf16(spd, seed):
    rng, N, H, D, P, lengths, scale = draw_case(seed)
    w = W.random_csr("sweep%d" % seed, 2000 + seed, N, H, D, P, lengths, scale=scale)
    sink = w.attn_sink.copy()
    sink[rng.random(H) < 0.2] = -np.inf
    w.attn_sink = sink
    max_len = max(lengths)
    log("case sweep bf16 seed=%d N=%d H=%d D=%d P=%d max_len=%d" % (seed, N, H, D, P, max_len))
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    q, kv, s = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    empty = torch.from_numpy(np.nonzero(np.diff(w.kv_indptr) == 0)[0]).to(dev())
    for plan in plans_for(rng, H, D, max_len):
        out = spd.sparse_decode_attn(q, kv, idx, ptr, s, w.softmax_scale, **plan)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out), ref, "sweep %d %s" % (seed, plan))
        assert torch.all(out[empty].view(torch.int16) == 0)


@pytest.mark.parametrize("seed", range(12))
def test_sweep_fp8(spd, seed):
    rng, N, H, D, P, lengths, scale = draw_case(100 + seed)
    D = max(D, 128) if rng.random() < 0.7 else D  # most cases where every FP8 mode applies
    w = W.random_csr("sweep8_%d" % seed, 3000 + seed, N, H, D, P, lengths, scale=scale)
    sink = w.attn_sink.copy()
    sink[rng.random(H) < 0.2] = -np.inf
    max_len = max(lengths)
    codes, scales = oracle.quantize_fp8(w.kv_bits)
    log("case sweep fp8 seed=%d N=%d H=%d D=%d P=%d max_len=%d" % (seed, N, H, D, P, max_len))
    ref = oracle.sparse_decode_attn_fp8(w.q_bits, codes, scales, w.kv_indices, w.kv_indptr, sink,
                                        w.softmax_scale)
    q = W.device_bits(w.q_bits, dev())
    kv8 = torch.from_numpy(codes).to(dev())
    ksc = torch.from_numpy(scales).to(dev())
    sk = torch.from_numpy(sink).to(dev())
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    plans = [dict(plain=True), dict(max_len=max_len), dict(mode=ROWS)]
    if D >= 128:
        rows = int(rng.choice([64, 128, 320]))
        if max_len <= 32 * rows:
            plans.append(dict(mode=SPLIT, max_len=max_len, split_rows=rows))
        plans.append(dict(mode=SPLIT, max_len=max_len))
        if H % 64 == 0:
            plans.append(dict(mode=WIDE))
    for plan in plans:
        out = spd.sparse_decode_attn_fp8(q, kv8, ksc, idx, ptr, sk, w.softmax_scale, **plan)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out), ref, "sweep fp8 %d %s" % (seed, plan))

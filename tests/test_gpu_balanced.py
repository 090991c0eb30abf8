"""GPU parity of split plans whose partitions the kernel sizes from the slice
lengths (SPD_MODE_SPLIT, or SPD_MODE_AUTO with max_len >= 2048, with no
partition length given and at most 256 (token, head group) pairs): every token
against the oracle (|d| <= 1e-2 + 1e-2 |ref|), bf16 and FP8 pools.

The kernel reads kv_indptr, finds the least partition length (a multiple of
its 32- or 64-row super-tile) for which the partitions of all slices fit in
the 256 workgroups, and deals them out token by token; the empty slices get
their zeros from the workgroups of the same index.  Cases: the ragged length
mix with a quarter of the slices empty, one long slice among short ones, every
slice empty, a single slice, mostly short slices with long and empty ones
among them, slices long enough to take the 32-partition limit, two head
groups (H = 128), a partial one (H = 96), 16 (H = 1000), 32-head workgroups
(H <= 32), D = 64 .. 512, calls with different length mixes one
after another on one workspace (its arrival counters end every call at zero),
bit-for-bit repeatability, and seeded random batches (shapes, length
distributions and empty fractions drawn per seed; 24 over bf16 pools, 8 over
FP8 pools)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, bf16_to_f64, dev, device_csr, device_inputs, log, oracle_tokens

pytestmark = pytest.mark.gpu

AUTO, SPLIT = 0, 4


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def ragged_lengths(rng, N, hi, empty=0.25):
    L = rng.integers(1, hi + 1, size=N)
    L[rng.random(N) < empty] = 0
    return [int(x) for x in L]


def mixed_lengths(rng, N):
    # a quarter empty, 15 % of 2500-6000 rows, the rest of 1-300 rows
    u = rng.random(N)
    L = np.where(u < 0.25, 0, np.where(u < 0.4, rng.integers(2500, 6001, N), rng.integers(1, 301, N)))
    return [int(x) for x in L]


def run_case(spd, w, what, max_len=None, mode=SPLIT, ws=None):
    max_len = max_len or max(1, max(np.diff(w.kv_indptr)))
    plan = spd.sparse_decode_attn_plan_info(w.N, w.H, w.D, max_len, 0, mode)
    assert plan["mode"] == "split" and plan["balanced"], plan
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    out = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, max_len=max_len,
                                 mode=mode, workspace=ws)
    torch.cuda.synchronize()
    assert_close(bf16_to_f64(out), ref, what)
    empty = np.nonzero(np.diff(w.kv_indptr) == 0)[0]
    if len(empty):
        assert torch.all(out[torch.from_numpy(empty).to(dev())].view(torch.int16) == 0), what
    return out


CASES = [
    # name, N, H, D, pool rows, length rule
    ("ragged", 256, 64, 512, 200000, lambda r: ragged_lengths(r, 256, 2048)),
    ("skewed", 64, 64, 512, 100000, lambda r: [9000] + [int(x) for x in r.integers(1, 200, 63)]),
    ("one_slice", 1, 64, 512, 50000, lambda r: [3000]),
    ("limit", 3, 64, 512, 300000, lambda r: [70000, 5, 0]),
    ("heads128", 100, 128, 512, 100000, lambda r: ragged_lengths(r, 100, 3000)),
    ("heads96", 40, 96, 256, 100000, lambda r: ragged_lengths(r, 40, 2500)),
    ("heads20_d128", 200, 20, 128, 100000, lambda r: ragged_lengths(r, 200, 4000)),
    ("d64", 120, 64, 64, 100000, lambda r: ragged_lengths(r, 120, 3000)),
    ("short", 256, 64, 512, 50000, lambda r: ragged_lengths(r, 256, 40)),
    # mostly short slices with long and empty ones among them
    ("mixed", 256, 64, 512, 200000, lambda r: mixed_lengths(r, 256)),
    ("mixed_heads128", 128, 128, 256, 100000, lambda r: mixed_lengths(r, 128)),
    # 16 head groups (the last one partial): 16 slots a head group
    ("heads1000", 12, 1000, 128, 50000, lambda r: ragged_lengths(r, 12, 3000)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_balanced_split_matches_oracle(spd, case):
    name, N, H, D, P, rule = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lengths = rule(rng)
    log("case balanced %s N=%d H=%d D=%d max_len=%d" % (name, N, H, D, max(lengths)))
    w = W.random_csr("bal_" + name, 500 + N + H + D, N, H, D, P, lengths)
    out = run_case(spd, w, name)
    # the same call again: the same bits
    q, kv, sink = device_inputs(w)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    out2 = spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale,
                                  max_len=max(1, max(lengths)), mode=SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_every_slice_empty(spd):
    log("case balanced all empty")
    w = W.random_csr("bal_empty", 71, 30, 64, 512, 1000, [0] * 30)
    q, kv, sink = device_inputs(w)
    idx = torch.zeros(1, dtype=torch.int32, device=dev())
    ptr = torch.zeros(31, dtype=torch.int32, device=dev())
    out = torch.full((30, 64, 512), 7.0, dtype=torch.bfloat16, device=dev())
    spd.sparse_decode_attn(q, kv, idx, ptr, sink, w.softmax_scale, out, max_len=4096, mode=SPLIT)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)


def test_length_mixes_one_after_another_on_one_workspace(spd):
    """Three different batches of 64 tokens through one workspace, twice over:
    the partition lengths differ per call, the counters end every call at
    zero, and each output matches the oracle."""
    N, H, D, P, max_len = 64, 64, 512, 100000, 8192
    rng = np.random.default_rng(5)
    mixes = [[8192] * 8 + [0] * 56, ragged_lengths(rng, N, 8192, 0.5),
             [int(x) for x in rng.integers(1, 300, N)]]
    ws = torch.zeros(spd.sparse_decode_attn_workspace_size(N, H, D, max_len, 0, SPLIT),
                     dtype=torch.uint8, device=dev())
    ws_before = ws.clone()
    works = [W.random_csr("bal_mix%d" % k, 90 + k, N, H, D, P, m) for k, m in enumerate(mixes)]
    for rep in range(2):
        for k, w in enumerate(works):
            log("case balanced mix %d rep %d" % (k, rep))
            run_case(spd, w, "mix %d rep %d" % (k, rep), max_len=max_len, ws=ws)
    # the arrival counters (the workspace's tail) are zero again
    plan = spd.sparse_decode_attn_plan_info(N, H, D, max_len, 0, SPLIT)
    ctr_bytes = N * plan["head_groups"] * D // (2 * plan["parities"])
    assert torch.equal(ws[-ctr_bytes:], ws_before[-ctr_bytes:])


def test_ragged_config_and_automatic_plan(spd):
    """The ragged configuration (N = 256, H = 64, D = 512, max_len 2048) in
    the automatic plan (the balanced split) and in split mode asked for, and
    the automatic plan on its first 200 tokens; every token checked."""
    w = W.ragged()
    plan = spd.sparse_decode_attn_plan_info(w.N, w.H, w.D, w.max_len)
    assert plan["mode"] == "split" and plan["balanced"], plan
    log("case balanced ragged config, automatic plan and split mode")
    run_case(spd, w, "ragged auto", max_len=w.max_len, mode=AUTO)
    run_case(spd, w, "ragged split", max_len=w.max_len, mode=SPLIT)
    lengths = list(np.diff(w.kv_indptr)[:200])
    w2 = W.random_csr("bal_ragged200", 808, 200, 64, 512, 200000, lengths)
    plan = spd.sparse_decode_attn_plan_info(w2.N, w2.H, w2.D, 2048)
    assert plan["mode"] == "split" and plan["balanced"], plan
    log("case balanced 200 ragged slices, automatic plan")
    run_case(spd, w2, "ragged200 auto", max_len=2048, mode=AUTO)


@pytest.mark.parametrize("name,N,H,D,hi", [("fp8_ragged", 256, 64, 512, 2048),
                                           ("fp8_h32", 100, 32, 256, 3000)])
def test_balanced_split_fp8(spd, name, N, H, D, hi):
    rng = np.random.default_rng(17 + N)
    lengths = ragged_lengths(rng, N, hi)
    lengths[0] = hi
    w = W.random_csr("bal_" + name, 700 + N, N, H, D, 150000, lengths)
    plan = spd.sparse_decode_attn_fp8_plan_info(N, H, D, hi, 0, SPLIT)
    assert plan["mode"] == "split" and plan["balanced"], plan
    log("case balanced %s N=%d H=%d D=%d" % (name, N, H, D))
    codes, scales = oracle.quantize_fp8(w.kv_bits)
    ref = oracle.sparse_decode_attn_fp8(w.q_bits, codes, scales, w.kv_indices, w.kv_indptr,
                                        w.attn_sink, w.softmax_scale)
    q = W.device_bits(w.q_bits, dev())
    kv8 = torch.from_numpy(codes).to(dev())
    ksc = torch.from_numpy(scales).to(dev())
    sk = torch.from_numpy(w.attn_sink).to(dev())
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    for mode in (SPLIT, AUTO):
        out = spd.sparse_decode_attn_fp8(q, kv8, ksc, idx, ptr, sk, w.softmax_scale, max_len=hi,
                                         mode=mode)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out), ref, "%s mode %d" % (name, mode))


def test_slices_longer_than_max_len(spd):
    """max_len only sizes the plan: slices longer than it (up to 2.5 x) are
    still cut from their own lengths and match the oracle."""
    rng = np.random.default_rng(31)
    lengths = ragged_lengths(rng, 48, 5000)
    lengths[5] = 5000
    w = W.random_csr("bal_over", 931, 48, 64, 256, 100000, lengths)
    log("case balanced slices past max_len")
    run_case(spd, w, "past max_len", max_len=2048)


def random_mix(rng):
    """A seeded batch shape and length mix for the balanced plan: N tokens of
    H heads (at most 256 (token, head group) pairs), lengths drawn uniform,
    exponential, bimodal or equal, some slices empty, one of at least 129 rows."""
    H, D = [(64, 512), (64, 128), (128, 256), (16, 128), (96, 64)][int(rng.integers(0, 5))]
    groups = 1 if H <= 64 else (H + 63) // 64
    N = int(rng.integers(1, 256 // groups + 1))
    kind = int(rng.integers(0, 4))
    hi = int(rng.choice([300, 2048, 6000]))
    if kind == 0:
        L = rng.integers(1, hi + 1, size=N)
    elif kind == 1:
        L = np.minimum(rng.exponential(hi / 4, size=N).astype(np.int64) + 1, 4 * hi)
    elif kind == 2:
        L = np.where(rng.random(N) < 0.1, rng.integers(hi, 3 * hi + 1, size=N),
                     rng.integers(1, 65, size=N))
    else:
        L = np.full(N, hi)
    L[rng.random(N) < rng.choice([0.0, 0.25, 0.6])] = 0
    L[int(rng.integers(0, N))] = max(129, int(L.max()))
    return N, H, D, [int(x) for x in L]


@pytest.mark.parametrize("seed", range(24))
def test_random_length_mixes(spd, seed):
    """Seeded random batches: every token against the oracle, empty slices
    zero."""
    rng = np.random.default_rng(1000 + seed)
    N, H, D, lengths = random_mix(rng)
    log("case balanced random seed %d: N=%d H=%d D=%d rows=%d max=%d" %
        (seed, N, H, D, sum(lengths), max(lengths)))
    w = W.random_csr("bal_rand%d" % seed, 2000 + seed, N, H, D, 60000, lengths)
    run_case(spd, w, "random mix %d" % seed)


@pytest.mark.parametrize("seed", range(8))
def test_random_length_mixes_fp8(spd, seed):
    """Seeded random batches over an FP8 pool (D >= 128): every token against
    the oracle's FP8 attention."""
    rng = np.random.default_rng(3000 + seed)
    N, H, D, lengths = random_mix(rng)
    D = max(D, 128)
    max_len = max(lengths)
    plan = spd.sparse_decode_attn_fp8_plan_info(N, H, D, max_len, 0, SPLIT)
    assert plan["mode"] == "split" and plan["balanced"], plan
    log("case balanced fp8 random seed %d: N=%d H=%d D=%d rows=%d max=%d" %
        (seed, N, H, D, sum(lengths), max_len))
    w = W.random_csr("bal_rand8_%d" % seed, 4000 + seed, N, H, D, 60000, lengths)
    codes, scales = oracle.quantize_fp8(w.kv_bits)
    ref = oracle.sparse_decode_attn_fp8(w.q_bits, codes, scales, w.kv_indices, w.kv_indptr,
                                        w.attn_sink, w.softmax_scale)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    out = spd.sparse_decode_attn_fp8(W.device_bits(w.q_bits, dev()), torch.from_numpy(codes).to(dev()),
                                     torch.from_numpy(scales).to(dev()), idx, ptr,
                                     torch.from_numpy(w.attn_sink).to(dev()), w.softmax_scale,
                                     max_len=max_len, mode=SPLIT)
    torch.cuda.synchronize()
    assert_close(bf16_to_f64(out), ref, "fp8 random mix %d" % seed)
    empty = np.nonzero(np.diff(w.kv_indptr) == 0)[0]
    if len(empty):
        assert torch.all(out[torch.from_numpy(empty).to(dev())].view(torch.int16) == 0)

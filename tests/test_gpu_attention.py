"""GPU parity of sparse decode attention (HIP path through the C ABI) against
the fp64 oracle, at small sizes that span several tiles and ragged tails, over
every supported head width and a range of head counts, with and without the
split-L plan; plus the invariants the pages fix (empty slice, no sink, single
row, permutation, determinism)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (assert_close, bf16_to_f64, device_csr, device_inputs, log,
                         oracle_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def run(spd, w, idx_np, ptr_np, sink=None, **plan):
    q, kv, s = device_inputs(w)
    if sink is not None:
        s = torch.from_numpy(np.asarray(sink, dtype=np.float32)).cuda()
    idx, ptr = device_csr(idx_np, ptr_np)
    out = spd.sparse_decode_attn(q, kv, idx, ptr, s, w.softmax_scale, **plan)
    torch.cuda.synchronize()
    return out


ROWS, HEADS, WIDE, SPLIT = 2, 1, 3, 4
PLANS = [dict(plain=True), dict(mode=ROWS), dict(mode=HEADS),
         dict(mode=HEADS, max_len=200, split_rows=32), dict(mode=HEADS, max_len=200, split_rows=64),
         dict(max_len=200), dict(mode=SPLIT, max_len=200), dict(mode=SPLIT, max_len=200, split_rows=32),
         dict(mode=SPLIT, max_len=200, split_rows=64)]


def plans(H):
    """PLANS, plus the 32-head-wave heads mode where it applies (H % 64 == 0)."""
    return PLANS + ([dict(mode=WIDE)] if H % 64 == 0 else [])


def test_tiny_all_tokens(spd):
    w = W.tiny()
    log("case tiny")
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    for plan in PLANS:
        out = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert_close(bf16_to_f64(out), ref, "tiny %s" % plan)
        assert torch.all(out[0].view(torch.int16) == 0)  # empty slice: exactly +0.0


LENGTHS = [0, 1, 5, 31, 32, 33, 64, 97, 200]


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("H", [1, 8, 16, 24, 40, 64, 128, 256])
def test_shapes(spd, H, D):
    seed = 100 + H * 7 + D
    w = W.random_csr("shapes", seed, len(LENGTHS), H, D, 700, LENGTHS)
    log("case shapes H=%d D=%d" % (H, D))
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    for plan in plans(H):
        out = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert_close(bf16_to_f64(out), ref, "H=%d D=%d %s" % (H, D, plan))


def test_many_tiles_and_long_slices(spd):
    lengths = [640, 2048, 1, 0, 1000, 333]
    w = W.random_csr("long", 7, len(lengths), 64, 512, 5000, lengths)
    log("case long slices")
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    for plan in [dict(plain=True), dict(mode=ROWS), dict(mode=HEADS), dict(mode=WIDE), dict(max_len=2048),
                 dict(max_len=2048, split_rows=96),
                 dict(max_len=256, split_rows=128)]:   # slices longer than max_len
        out = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert_close(bf16_to_f64(out), ref, "long %s" % plan)


@pytest.mark.parametrize("H", [32, 64])
@pytest.mark.parametrize("kind", ["none", "dominant", "mixed"])
def test_sink_variants(spd, kind, H):
    lengths = [0, 3, 40, 129]
    w = W.random_csr("sinks", 11, len(lengths), H, 128, 300, lengths)
    if kind == "none":
        sink = np.full(H, -np.inf, dtype=np.float32)
    elif kind == "dominant":
        sink = np.full(H, 30.0, dtype=np.float32)
    else:
        sink = np.where(np.arange(H) % 2 == 0, -np.inf, 5.0).astype(np.float32)
    log("case sink %s H=%d" % (kind, H))
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr, sink=sink)
    for plan in plans(w.H):
        out = run(spd, w, w.kv_indices, w.kv_indptr, sink=sink, **plan)
        assert_close(bf16_to_f64(out), ref, "sink %s %s" % (kind, plan))
        assert torch.all(out[0].view(torch.int16) == 0)


@pytest.mark.parametrize("H", [16, 64])
def test_single_row_without_sink_is_bit_exact(spd, H):
    """One index and attn_sink = -inf: the weight is exactly 1, so the output
    equals the bf16 row bit for bit."""
    w = W.random_csr("single", 12, 5, H, 512, 50, [1, 1, 1, 1, 1])
    sink = np.full(H, -np.inf, dtype=np.float32)
    log("case single row H=%d" % H)
    extra = [dict(mode=WIDE)] if H % 64 == 0 else []
    for plan in [dict(mode=ROWS), dict(mode=HEADS), dict(max_len=32, split_rows=32),
                 dict(mode=SPLIT, max_len=32)] + extra:
        out = run(spd, w, w.kv_indices, w.kv_indptr, sink=sink, **plan)
        kv = W.device_bits(w.kv_bits, torch.device("cuda:0"))
        for t in range(5):
            row = kv[int(w.kv_indices[t])]
            assert torch.equal(out[t].view(torch.int16), row.view(torch.int16).expand(H, -1))


def test_all_empty_batch(spd):
    w = W.random_csr("empty", 13, 6, 64, 512, 10, [0] * 6)
    log("case all empty")
    for plan in plans(w.H):
        out = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert torch.all(out.view(torch.int16) == 0)


def test_permutation_and_duplicates(spd):
    rng = np.random.default_rng(14)
    lengths = [77, 130, 5]
    w = W.random_csr("perm", 14, 3, 64, 256, 90, lengths)  # 90 rows: many duplicates
    perm = w.kv_indices.copy()
    for t in range(3):
        a, b = w.kv_indptr[t], w.kv_indptr[t + 1]
        perm[a:b] = rng.permutation(perm[a:b])
    log("case permutation")
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    for plan in [dict(mode=ROWS), dict(mode=HEADS), dict(mode=WIDE), dict(mode=SPLIT, max_len=130)]:
        o1 = bf16_to_f64(run(spd, w, w.kv_indices, w.kv_indptr, **plan))
        o2 = bf16_to_f64(run(spd, w, perm, w.kv_indptr, **plan))
        assert_close(o1, ref, "original order %s" % plan)
        assert_close(o2, ref, "permuted order %s" % plan)


def test_repeated_rows_closed_form(spd):
    """L copies of one row: out = r * L e^s / (L e^s + e^sink)."""
    L = 300
    w = W.random_csr("repeat", 15, 1, 16, 512, 4, [L])
    w.kv_indices[:] = 2
    log("case repeated row")
    out = bf16_to_f64(run(spd, w, w.kv_indices, w.kv_indptr, max_len=L, split_rows=64))
    assert_close(out, ref_closed_form(w, L), "repeated row, split")
    out = bf16_to_f64(run(spd, w, w.kv_indices, w.kv_indptr, mode=ROWS))
    assert_close(out, ref_closed_form(w, L), "repeated row, rows mode")
    out = bf16_to_f64(run(spd, w, w.kv_indices, w.kv_indptr, mode=SPLIT, max_len=L, split_rows=64))
    assert_close(out, ref_closed_form(w, L), "repeated row, split mode")


def ref_closed_form(w, L):
    r = W.bf16_to_f32(W.host_bits(w.kv_bits)[2]).astype(np.float64)
    q = W.bf16_to_f32(W.host_bits(w.q_bits)[0]).astype(np.float64)
    ref = np.zeros((1, 16, 512))
    for h in range(16):
        s = w.softmax_scale * float(q[h] @ r)
        ref[0, h] = r * L * math.exp(s) / (L * math.exp(s) + math.exp(float(w.attn_sink[h])))
    return ref


def test_deterministic(spd):
    w = W.random_csr("det", 16, 8, 64, 512, 3000, [640, 1, 0, 333, 1000, 64, 65, 2000])
    log("case determinism")
    for plan in [dict(mode=ROWS), dict(mode=HEADS), dict(mode=WIDE), dict(max_len=2000, mode=HEADS),
                 dict(max_len=2000, mode=SPLIT)]:
        a = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        b = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("H,D", [(64, 512), (32, 512), (64, 128)])
def test_split_every_unit_width_without_waiting(spd, H, D):
    """Split mode on a grid larger than the chip (16 tokens x 32 partitions of
    64 rows), so no merging workgroup waits and the arrival that completes
    each count merges its unit alone; the lengths give 1 to 32 partitions, so
    units of every width (a piece cut into 1, 2, 4 or 8) are merged.  Every
    token against the oracle, and the same bits on a second call."""
    lengths = [1, 64, 65, 130, 256, 257, 400, 520, 700, 1000, 1030, 1500, 2000, 2048, 0, 33]
    w = W.random_csr("split_units", 23, len(lengths), H, D, 9000, lengths)
    log("case split units H=%d D=%d" % (H, D))
    plan = spd.sparse_decode_attn_plan_info(w.N, H, D, 2048, 64, SPLIT)
    assert plan["splits"] == 32 and w.N * plan["head_groups"] * 32 > 256
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    a = run(spd, w, w.kv_indices, w.kv_indptr, mode=SPLIT, max_len=2048, split_rows=64)
    b = run(spd, w, w.kv_indices, w.kv_indptr, mode=SPLIT, max_len=2048, split_rows=64)
    assert_close(bf16_to_f64(a), ref, "split units H=%d D=%d" % (H, D))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_validate_indices(spd):
    d = torch.device("cuda:0")
    ptr = torch.tensor([0, 2, 2, 5], dtype=torch.int32, device=d)
    idx = torch.tensor([0, 9, 3, 4, 1], dtype=torch.int32, device=d)
    assert spd.validate_indices(idx, ptr, 10) == -1
    assert spd.validate_indices(idx, ptr, 9) == 3 + 1 + 1      # kv_indices[1] == 9 out of range
    bad_ptr = torch.tensor([0, 3, 2, 5], dtype=torch.int32, device=d)
    assert spd.validate_indices(idx, bad_ptr, 10) == 2        # decreasing at t = 2


def test_late_large_scores_take_the_second_pass(spd):
    """Rows planted in later tiles whose score for head 0 lies far (> 64 in
    log2 units) above everything in the first tile of the state that reads
    them: the reference maximum fixed at that first tile is left behind, so the
    kernel must redo the state with the true maximum.  Two planted rows of
    nearby scores keep the expected output a genuine mix of rows.  The 2100-row
    token also crosses the 2048-index staging chunk."""
    lengths = [300, 700, 40, 2100, 0]
    w = W.random_csr("late", 17, len(lengths), 64, 512, 6000, lengths, replace=False)
    kv = w.kv_bits.copy()
    q = W.bf16_to_f32(w.q_bits).astype(np.float32)
    plants = {0: (100, 290), 1: (150, 650), 3: (1000, 2090)}
    for t, (p2, p1) in plants.items():
        a = int(w.kv_indptr[t])
        kv[int(w.kv_indices[a + p1])] = W.bf16_bits(4.0 * q[t, 0])   # score ~ 90
        kv[int(w.kv_indices[a + p2])] = W.bf16_bits(3.9 * q[t, 0])   # ~ 2 lower
    w.kv_bits = kv
    log("case late large scores")
    ref = oracle_tokens(w, w.kv_indices, w.kv_indptr)
    for plan in plans(w.H) + [dict(mode=HEADS, max_len=2100, split_rows=256),
                              dict(mode=SPLIT, max_len=2100, split_rows=512)]:
        out = run(spd, w, w.kv_indices, w.kv_indptr, **plan)
        assert_close(bf16_to_f64(out), ref, "late large %s" % plan)


@pytest.mark.parametrize("case", __import__("golden_cases").attention_cases(), ids=lambda c: c["name"])
def test_worked_examples_padded(spd, case):
    """The hand-worked fixtures of tests/golden/, with D zero-padded to 64 (the
    padding adds nothing to any score and yields zero output columns)."""
    N, H, Dg = case["q"].shape
    D = 64
    q = np.zeros((N, H, D), dtype=np.float32)
    q[:, :, :Dg] = case["q"]
    kv = np.zeros((case["kv"].shape[0], D), dtype=np.float32)
    kv[:, :Dg] = case["kv"]
    ref = np.zeros((N, H, D))
    ref[:, :, :Dg] = case["out"]
    d = torch.device("cuda:0")
    qd = torch.from_numpy(W.bf16_bits(q).view(np.int16)).to(d).view(torch.bfloat16)
    kvd = torch.from_numpy(W.bf16_bits(kv).view(np.int16)).to(d).view(torch.bfloat16)
    sink = torch.from_numpy(case["attn_sink"]).to(d)
    idx, ptr = device_csr(case["kv_indices"], case["kv_indptr"])
    log("case golden %s" % case["name"])
    for plan in PLANS:
        out = spd.sparse_decode_attn(qd, kvd, idx, ptr, sink, case["softmax_scale"], **plan)
        torch.cuda.synchronize()
        assert_close(bf16_to_f64(out), ref, "golden %s %s" % (case["name"], plan))

"""Pins for the oracle's decode index builder (CPU only, bit-exact).

Page facts pinned (sglang PR #28392 summary, "key source snippet", the
paged_decode.py module docstring): pool slots [0, swa_pages) hold window
entries at state_slot * win + ring; slots from swa_pages on hold compressed
entries at block_id * K_PER_BLOCK + slot_in_block; the production builder
emits ragged-packed indices without sentinels, and a padded token gets a zero
length slice (kv_indptr[t+1] == kv_indptr[t]).
"""
import numpy as np
import pytest

import brute
import golden_cases
import workloads as W


def _random_builder(seed, N, win, topk, k, max_blocks, n_blocks, sentinel_frac=0.3,
                    empty_ring_frac=0.2):
    rng = np.random.default_rng(seed)
    n_states = N + 2
    state_slot = rng.permutation(n_states)[:N].astype(np.int32)
    swa_len = rng.integers(0, win + 1, size=N).astype(np.int32)
    swa_len[rng.random(N) < empty_ring_frac] = 0
    comp_pos = rng.integers(0, max_blocks * k, size=(N, topk)).astype(np.int32)
    comp_pos[rng.random((N, topk)) < sentinel_frac] = -1
    block_table = rng.integers(0, n_blocks, size=(N, max_blocks)).astype(np.int32)
    swa_pages = n_states * win
    pool_rows = swa_pages + n_blocks * k
    return state_slot, swa_len, comp_pos, block_table, swa_pages, pool_rows


@pytest.mark.parametrize("seed", range(8))
def test_matches_membership_brute_force(oracle_mod, seed):
    """P10a: per token, the multiset of produced slots equals the slots that a
    brute-force scan of the whole pool assigns to that token."""
    N, win, topk, k, max_blocks, n_blocks = 5, 4, 6, [1, 2, 3, 4][seed % 4], 3, 5
    ss, sl, cp, bt, swa_pages, pool_rows = _random_builder(seed, N, win, topk, k, max_blocks, n_blocks)
    indptr, indices = oracle_mod.build_decode_indices(ss, sl, cp, bt, win, k, swa_pages)
    want = brute.builder_membership(ss, sl, cp, bt, win, k, swa_pages, pool_rows)
    for t in range(N):
        got = sorted(indices[indptr[t]:indptr[t + 1]].tolist())
        assert got == want[t], t


def test_hand_worked_example(oracle_mod):
    """The hand-derived fixture tests/golden/builder_worked_example.json."""
    c = golden_cases.builder_case()
    indptr, indices = oracle_mod.build_decode_indices(c["state_slot"], c["swa_len"], c["comp_pos"],
                                                      c["block_table"], c["win"], c["k_per_block"],
                                                      c["swa_pages"])
    assert indptr.tolist() == c["kv_indptr"].tolist()
    assert indices.tolist() == c["kv_indices"].tolist()


def test_order_window_then_compressed(oracle_mod):
    """Reading of the unstated order: window ring slots ascending, then the
    compressed entries in comp_pos row order with negative entries dropped."""
    ss, sl, cp, bt, swa_pages, _ = _random_builder(11, 6, 8, 10, 4, 4, 9)
    indptr, indices = oracle_mod.build_decode_indices(ss, sl, cp, bt, 8, 4, swa_pages)
    for t in range(6):
        seg = indices[indptr[t]:indptr[t + 1]]
        n_win = int(sl[t])
        assert np.array_equal(seg[:n_win] - ss[t] * 8, np.arange(n_win))
        valid = cp[t][cp[t] >= 0]
        comp = seg[n_win:]
        assert len(comp) == len(valid)
        # inverse map of each compressed slot recovers (block, slot-in-block) of its comp_pos
        rel = comp - swa_pages
        assert np.array_equal(rel // 4, bt[t][valid // 4])
        assert np.array_equal(rel % 4, valid % 4)


def test_invariants_and_padding(oracle_mod):
    """P10b: indptr starts at 0, ends at the total, window slots < swa_pages <=
    compressed slots, full rings give state_slot*win + [0, win), all-sentinel
    rows with an empty ring give zero-length slices."""
    ss, sl, cp, bt, swa_pages, _ = _random_builder(12, 40, 16, 32, 8, 4, 30)
    sl[:5] = 16                     # full rings
    sl[-7:] = 0                     # padded tokens ...
    cp[-7:] = -1                    # ... with no compressed entries
    indptr, indices = oracle_mod.build_decode_indices(ss, sl, cp, bt, 16, 8, swa_pages)
    assert indptr[0] == 0 and indptr[-1] == len(indices)
    assert np.all(np.diff(indptr) >= 0)
    counts = np.diff(indptr)
    assert np.array_equal(counts, sl + (cp >= 0).sum(axis=1))
    for t in range(40):
        seg = indices[indptr[t]:indptr[t + 1]]
        assert np.all(seg[:sl[t]] < swa_pages) and np.all(seg[sl[t]:] >= swa_pages)
    for t in range(5):
        assert np.array_equal(indices[indptr[t]:indptr[t] + 16], ss[t] * 16 + np.arange(16))
    assert np.all(counts[-7:] == 0)


def test_no_compressed_part(oracle_mod):
    ss = np.array([1, 0], dtype=np.int32)
    sl = np.array([2, 3], dtype=np.int32)
    indptr, indices = oracle_mod.build_decode_indices(ss, sl, None, None, 3, 1, 6)
    assert indptr.tolist() == [0, 2, 5] and indices.tolist() == [3, 4, 0, 1, 2]


@pytest.mark.parametrize("win,k", [(0, 1), (-1, 1), (4, 0), (4, -2)])
def test_rejects_bad_scalars(oracle_mod, win, k):
    """win <= 0 or K_PER_BLOCK <= 0 would divide by zero or index out of bounds."""
    ss = np.zeros(1, dtype=np.int32)
    sl = np.zeros(1, dtype=np.int32)
    cp = np.zeros((1, 1), dtype=np.int32)
    bt = np.zeros((1, 1), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle_mod.build_decode_indices(ss, sl, cp, bt, win, k, 0)


def test_decode_base_structure(oracle_mod):
    """The decode_base workload built by the oracle: 640 entries per token,
    128 contiguous ring slots t*128 + [0,128) then 512 distinct compressed slots."""
    w = W.decode_base()
    b = w.builder
    indptr, indices = oracle_mod.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos,
                                                      b.block_table, b.win, b.k_per_block,
                                                      b.swa_pages)
    assert np.array_equal(indptr, np.arange(65, dtype=np.int32) * 640)
    for t in range(64):
        seg = indices[t * 640:(t + 1) * 640]
        assert np.array_equal(seg[:128], t * 128 + np.arange(128))
        comp = seg[128:]
        assert len(np.unique(comp)) == 512 and comp.min() >= 8192 and comp.max() < 65536


def test_clamped_builder_hand_worked_example(oracle_mod):
    """Metadata outside the builder's preconditions (ring lengths below 0 and
    above win, entries whose block lies past the table): the hand-derived
    fixture tests/golden/builder_clamp_example.json (reading R27)."""
    c = golden_cases.builder_case("builder_clamp_example.json")
    args = (c["state_slot"], c["swa_len"], c["comp_pos"], c["block_table"], c["win"],
            c["k_per_block"], c["swa_pages"])
    indptr, indices = oracle_mod.build_decode_indices(*args, clamp=True)
    assert indptr.tolist() == c["kv_indptr"].tolist()
    assert indices.tolist() == c["kv_indices"].tolist()
    with pytest.raises(ValueError):  # the strict builder rejects the same input
        oracle_mod.build_decode_indices(*args)


def test_clamped_builder_equals_strict_on_valid_input(oracle_mod):
    """Within the preconditions the clamping form changes nothing."""
    for seed in range(5):
        ss, sl, cp, bt, swa_pages, _ = _random_builder(40 + seed, 7, 8, 12, 4, 5, 11)
        a = oracle_mod.build_decode_indices(ss, sl, cp, bt, 8, 4, swa_pages)
        b = oracle_mod.build_decode_indices(ss, sl, cp, bt, 8, 4, swa_pages, clamp=True)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_clamped_builder_counts(oracle_mod):
    """Each token gets min(max(swa_len, 0), win) window rows and one row per
    entry c with 0 <= c < max_blocks * K, and nothing else."""
    rng = np.random.default_rng(77)
    N, win, topk, K, mb = 9, 6, 7, 3, 4
    ss = rng.integers(0, 20, size=N).astype(np.int32)
    sl = rng.integers(-5, 12, size=N).astype(np.int32)
    cp = rng.integers(-3, 2 * mb * K, size=(N, topk)).astype(np.int32)
    bt = rng.integers(0, 50, size=(N, mb)).astype(np.int32)
    indptr, indices = oracle_mod.build_decode_indices(ss, sl, cp, bt, win, K, 200, clamp=True)
    for t in range(N):
        n_win = min(max(int(sl[t]), 0), win)
        n_comp = int(((cp[t] >= 0) & (cp[t] < mb * K)).sum())
        assert indptr[t + 1] - indptr[t] == n_win + n_comp
        rows = indices[indptr[t]:indptr[t + 1]]
        assert rows[:n_win].tolist() == [int(ss[t]) * win + r for r in range(n_win)]
        assert np.all(rows[n_win:] >= 200)

"""Pins for the fp64 attention oracle (CPU only).

Definition pinned (sglang PR #28392 summary, "key source snippet", the
paged_decode.py module docstring): token t attends to the ragged slice
kv_indices[kv_indptr[t]:kv_indptr[t+1]] of a [P, D] bf16 pool whose rows are
both keys and values; attn_sink[H] is a virtual key in the softmax denominator;
an empty slice is legal.  Each test below checks the oracle against something
other than its own formula: a brute-force restatement on tiny inputs, a library
routine for the special case that reduces to plain attention, closed forms and
invariants.
"""
import math

import numpy as np
import pytest
import torch

import brute
import golden_cases
import workloads as W

LN2 = math.log(2.0)


def _rand_case(seed, N, H, D, P, max_L, sink_std=1.0, scale=None, dup=True):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, max_L + 1, size=N)
    lists = [rng.integers(0, P, size=L) if dup else rng.choice(P, size=min(L, P), replace=False)
             for L in lengths]
    idx, indptr = W.csr_from_lists(lists)
    q = W.normal_bf16(rng, (N, H, D))
    kv = W.normal_bf16(rng, (P, D))
    sink = (rng.standard_normal(H) * sink_std).astype(np.float32)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return q, kv, idx, indptr, sink, scale


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_softmax(oracle_mod, seed):
    """P1: oracle == explicit [scores, sink] softmax with exact sums (duplicates included)."""
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    D = [1, 2, 8, 64][seed % 4]
    P = int(rng.integers(1, 40))
    q, kv, idx, indptr, sink, scale = _rand_case(seed, N, H, D, P, 20)
    got = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    ref = brute.attention(q, kv, idx, indptr, sink, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("case", golden_cases.attention_cases(), ids=lambda c: c["name"])
def test_worked_examples(oracle_mod, case):
    """Hand-worked fixtures (tests/golden/attention_worked_examples.json): exact
    fractions derived from the definition, covering the sink as a virtual key
    in natural-log units, a -inf sink and an empty slice."""
    q = W.bf16_bits(case["q"])
    kv = W.bf16_bits(case["kv"])
    out = oracle_mod.sparse_decode_attn(q, kv, case["kv_indices"], case["kv_indptr"],
                                        case["attn_sink"], case["softmax_scale"])
    # softmax_scale and the sink are fp32 values, so the weights match the
    # stated integers only to fp32 precision
    np.testing.assert_allclose(out, case["out"], rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("seed", range(6))
def test_no_sink_is_plain_attention(oracle_mod, seed):
    """P2: attn_sink = -inf reduces to plain softmax attention; checked against
    torch's scaled_dot_product_attention in fp64 with K = V = the gathered rows."""
    N, H, D, P = 3, 4, [8, 16, 64][seed % 3], 50
    q, kv, idx, indptr, _, scale = _rand_case(seed, N, H, D, P, 30)
    sink = np.full(H, -np.inf, dtype=np.float32)
    got = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    qf = torch.from_numpy(W.bf16_to_f32(q).astype(np.float64))
    kvf = torch.from_numpy(W.bf16_to_f32(kv).astype(np.float64))
    for t in range(N):
        sl = torch.from_numpy(idx[indptr[t]:indptr[t + 1]].astype(np.int64))
        if len(sl) == 0:
            assert np.all(got[t] == 0.0)
            continue
        rows = kvf[sl]                                   # [L, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[t][None, :, None, :], rows[None, None].expand(1, H, -1, -1).contiguous(),
            rows[None, None].expand(1, H, -1, -1).contiguous(), scale=float(np.float32(scale)))
        np.testing.assert_allclose(got[t], ref[0, :, 0, :].numpy(), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("sink_value", [0.0, -3.5, 2.0, 30.0, -np.inf])
def test_empty_slice_is_exact_zero(oracle_mod, sink_value):
    """P3: an empty slice gives exactly 0 for any sink (incl. -inf: 0/0 := 0)."""
    q, kv, _, _, _, scale = _rand_case(3, 3, 2, 8, 10, 0)
    idx = np.array([4, 5], dtype=np.int32)
    indptr = np.array([0, 0, 2, 2], dtype=np.int32)   # tokens 0 and 2 empty
    sink = np.full(2, sink_value, dtype=np.float32)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    assert np.all(out[0] == 0.0) and np.all(out[2] == 0.0)
    assert np.all(np.signbit(out[0]) == False)  # noqa: E712  (+0.0, not -0.0)
    assert np.any(out[1] != 0.0)


@pytest.mark.parametrize("seed", range(4))
def test_permutation_invariance(oracle_mod, seed):
    """P4: reordering a token's slice leaves its output unchanged."""
    q, kv, idx, indptr, sink, scale = _rand_case(seed, 4, 3, 32, 64, 40)
    rng = np.random.default_rng(seed)
    perm_idx = idx.copy()
    for t in range(4):
        a, b = indptr[t], indptr[t + 1]
        perm_idx[a:b] = rng.permutation(idx[a:b])
    o1 = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    o2 = oracle_mod.sparse_decode_attn(q, kv, perm_idx, indptr, sink, scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)


def test_single_index_no_sink_returns_row(oracle_mod):
    """P5: one index with attn_sink = -inf returns that row exactly."""
    q, kv, _, _, _, scale = _rand_case(5, 2, 3, 64, 16, 0)
    idx = np.array([7, 11], dtype=np.int32)
    indptr = np.array([0, 1, 2], dtype=np.int32)
    sink = np.full(3, -np.inf, dtype=np.float32)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    rows = W.bf16_to_f32(kv).astype(np.float64)
    for h in range(3):
        assert np.array_equal(out[0, h], rows[7])
        assert np.array_equal(out[1, h], rows[11])


def test_zero_scale_closed_form(oracle_mod):
    """P6: softmax_scale = 0 makes every score 0, so
    out = sum_j KV[J_j] / (L + exp(sink))."""
    q, kv, idx, indptr, sink, _ = _rand_case(6, 4, 3, 16, 20, 12)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, 0.0)
    rows = W.bf16_to_f32(kv).astype(np.float64)
    for t in range(4):
        sl = idx[indptr[t]:indptr[t + 1]]
        if len(sl) == 0:
            continue
        for h in range(3):
            ref = rows[sl].sum(axis=0) / (len(sl) + math.exp(float(sink[h])))
            np.testing.assert_allclose(out[t, h], ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("L", [1, 2, 5, 33])
def test_repeated_row_closed_form(oracle_mod, L):
    """P7: L copies of one row r give out = r * L e^s / (L e^s + e^sink), s = scale * q.r."""
    q, kv, _, _, sink, scale = _rand_case(7, 1, 4, 64, 9, 0)
    idx = np.full(L, 3, dtype=np.int32)
    indptr = np.array([0, L], dtype=np.int32)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, sink, scale)
    r = W.bf16_to_f32(kv[3]).astype(np.float64)
    qf = W.bf16_to_f32(q[0]).astype(np.float64)
    for h in range(4):
        s = float(np.float32(scale)) * float(qf[h] @ r)
        coef = L * math.exp(s) / (L * math.exp(s) + math.exp(float(sink[h])))
        np.testing.assert_allclose(out[0, h], coef * r, rtol=1e-12, atol=1e-14)


def test_sink_limits(oracle_mod):
    """P8: a dominant sink drives the output to 0 (bounded by e^(max s - sink) max|v|);
    with no sink and equal scores the output is the mean of the rows."""
    q, kv, idx, indptr, _, scale = _rand_case(8, 3, 2, 32, 30, 10)
    big = np.full(2, 60.0, dtype=np.float32)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, big, scale)
    rows = W.bf16_to_f32(kv).astype(np.float64)
    qf = W.bf16_to_f32(q).astype(np.float64)
    for t in range(3):
        sl = idx[indptr[t]:indptr[t + 1]]
        if len(sl) == 0:
            continue
        for h in range(2):
            smax = float(np.max(float(np.float32(scale)) * (rows[sl] @ qf[t, h])))
            bound = len(sl) * math.exp(smax - 60.0) * np.abs(rows[sl]).max()
            assert np.abs(out[t, h]).max() <= bound * (1 + 1e-9)
    none = np.full(2, -np.inf, dtype=np.float32)
    out = oracle_mod.sparse_decode_attn(q, kv, idx, indptr, none, 0.0)
    for t in range(3):
        sl = idx[indptr[t]:indptr[t + 1]]
        if len(sl):
            np.testing.assert_allclose(out[t, 0], rows[sl].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_token_subset_matches_full(oracle_mod):
    """Evaluating a sample of tokens gives the same values as evaluating all."""
    w = W.tiny()
    full = oracle_mod.sparse_decode_attn(w.q_bits, w.kv_bits, w.kv_indices, w.kv_indptr,
                                         w.attn_sink, w.softmax_scale)
    sub = oracle_mod.sparse_decode_attn(w.q_bits, w.kv_bits, w.kv_indices, w.kv_indptr,
                                        w.attn_sink, w.softmax_scale, tokens=np.array([3, 1]))
    assert np.array_equal(sub[0], full[3]) and np.array_equal(sub[1], full[1])


def test_rejects_out_of_range_index(oracle_mod):
    q, kv, _, _, sink, scale = _rand_case(9, 1, 1, 8, 4, 0)
    with pytest.raises(ValueError):
        oracle_mod.sparse_decode_attn(q, kv, np.array([4], dtype=np.int32),
                                      np.array([0, 1], dtype=np.int32), sink, scale)


def test_tiny_config_against_brute(oracle_mod):
    """The tiny benchmark configuration, all tokens, against the brute force."""
    w = W.tiny()
    got = oracle_mod.sparse_decode_attn(w.q_bits, w.kv_bits, w.kv_indices, w.kv_indptr,
                                        w.attn_sink, w.softmax_scale)
    ref = brute.attention(w.q_bits, w.kv_bits, w.kv_indices, w.kv_indptr, w.attn_sink,
                          w.softmax_scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)

"""Pins of the oracle's FP8 pool functions (CPU): the OCP e4m3 decode, the
quantiser (scale = amax / 448, round to nearest even, saturating) and
attention over an FP8 pool.  Each is checked against something other than its
own formula: PyTorch's float8_e4m3fn decode and cast, closed-form values of
the format, exact round trips and a bf16 reduction."""
import math

import numpy as np
import pytest
import torch

import oracle


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values that are exact bf16 -> their uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values must be exact bf16"
    return (u >> 16).astype(np.uint16)


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).float().numpy().astype(np.float64)


def test_decode_matches_torch_on_every_code():
    mine = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = torch_e4m3(np.arange(256))
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref))
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2


def test_decode_closed_forms():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0      # +0, -0
    assert v(0x01) == 2.0 ** -9                                           # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9                                       # largest subnormal
    assert v(0x08) == 2.0 ** -6                                           # smallest normal
    assert v(0x38) == 1.0 and v(0x3F) == 1.875 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0                         # largest finite
    finite = [v(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(finite, finite[1:]))                 # strictly increasing
    for c in range(0x7F):                                                 # every value is bf16-exact
        f = np.float32(finite[c])
        assert (np.array([f]).view(np.uint32)[0] & 0xFFFF) == 0


def test_quantiser_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 30.0], size=(64, 1))).astype(np.float32)
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)  # exact bf16
    codes, scales = oracle.quantize_fp8(bf16_bits(x))
    # the scaled values, in fp32 as the quantiser defines them, rounded by torch
    amax = np.abs(x).max(axis=1)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    y = np.clip((x * inv[:, None]).astype(np.float32), -448.0, 448.0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))


def test_quantiser_ties_go_to_even():
    # rows whose largest entry is 448 (scale 1, inv 1): the entries are used as is
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    lo, hi = grid[40:100:3], grid[41:101:3]          # consecutive pairs of finite values
    mid = ((lo + hi) / 2).astype(np.float32)          # exactly halfway (exact in fp32 and bf16)
    row = np.concatenate([[448.0], mid]).astype(np.float32)
    codes, scales = oracle.quantize_fp8(bf16_bits(row[None, :]))
    assert scales[0] == 1.0
    got = codes[0, 1:].astype(int)
    lo_code = np.arange(40, 100, 3)
    expect = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)  # even mantissa = even code
    assert np.array_equal(got, expect)


def test_quantiser_saturation_zero_row_and_exact_round_trip():
    # the largest magnitude maps to +-448; a zero row gives scale 0 and zero codes
    x = np.array([[0.0, -3.0, 1.5, 0.25], [0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    codes, scales = oracle.quantize_fp8(bf16_bits(x))
    assert codes[0, 1] == 0xFE and scales[0] == np.float32(3.0) / np.float32(448.0)
    assert scales[1] == 0.0 and np.all(codes[1] == 0)
    # values that are a power-of-two scale times e4m3 values, with 448 present:
    # the codes come back exactly
    rng = np.random.default_rng(2)
    for k in (-20, -3, 0, 5):
        c = rng.integers(0, 0x7F, size=63)
        c = np.where(rng.random(63) < 0.5, c, c | 0x80)
        vals = np.array([oracle.e4m3_value(int(v)) for v in c])
        row = np.concatenate([[448.0], vals]) * 2.0 ** k
        codes, scales = oracle.quantize_fp8(bf16_bits(row.astype(np.float32)[None, :]))
        assert scales[0] == np.float32(2.0 ** k)
        dec = np.array([oracle.e4m3_value(int(v)) for v in codes[0]])
        assert np.array_equal(dec * 2.0 ** k, row)  # (-0 == 0 here)


def test_quantiser_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    codes, scales = oracle.quantize_fp8(bf16_bits(x))
    dec = torch_e4m3(codes) * scales[:, None].astype(np.float64)
    # e4m3 spacing is 2^(e-3) for |v| in [2^e, 2^(e+1)), 2^-9 below 2^-6: half of it
    # (plus a few fp32 roundings of the scaling) bounds the error
    y = np.abs(x.astype(np.float64)) / scales[:, None]
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half = 0.5 * 2.0 ** (e - 3) * scales[:, None] * (1 + 1e-6)
    assert np.all(np.abs(dec - x) <= half + 1e-30)


def test_fp8_attention_equals_bf16_attention_on_the_decoded_rows():
    """With power-of-two scales the decoded rows are exact bf16 values, so the
    FP8 oracle must give the bf16 oracle's output on those rows, exactly."""
    rng = np.random.default_rng(4)
    N, H, D, P = 3, 4, 32, 40
    codes = rng.integers(0, 0x7F, size=(P, D)).astype(np.uint8)
    codes |= (rng.random((P, D)) < 0.5).astype(np.uint8) << 7
    scales = (2.0 ** rng.integers(-4, 3, size=P)).astype(np.float32)
    rows = torch_e4m3(codes) * scales[:, None].astype(np.float64)
    kv_bits = bf16_bits(rows.astype(np.float32))
    q = (rng.standard_normal((N, H, D)) * 0.1).astype(np.float32)
    q_bits = bf16_bits((q.view(np.uint32) & 0xFFFF0000).view(np.float32))
    lists = [rng.integers(0, P, size=L) for L in (0, 5, 23)]
    ptr = np.concatenate([[0], np.cumsum([len(l) for l in lists])]).astype(np.int32)
    idx = np.concatenate(lists).astype(np.int32)
    sink = rng.standard_normal(H).astype(np.float32)
    a = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, 0.17)
    b = oracle.sparse_decode_attn(q_bits, kv_bits, idx, ptr, sink, 0.17)
    assert np.array_equal(a, b)
    assert np.all(a[0] == 0)

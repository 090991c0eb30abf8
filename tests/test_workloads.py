"""The seeded input generators: shapes, reproducibility and the structure each
benchmark configuration asks for (CPU only; large pools are not materialised)."""
import math

import numpy as np

import workloads as W


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    bits = W.bf16_bits(x)
    back = W.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]


def test_tiny_is_reproducible_and_shaped():
    a, b = W.tiny(), W.tiny()
    assert np.array_equal(a.q_bits, b.q_bits) and np.array_equal(a.kv_bits, b.kv_bits)
    assert a.q_bits.shape == (4, 8, 64) and a.kv_bits.shape == (256, 64)
    assert np.diff(a.kv_indptr).tolist() == [0, 1, 17, 64]
    assert a.kv_indices.min() >= 0 and a.kv_indices.max() < 256
    assert a.softmax_scale == 0.125


def test_decode_base_builder_inputs():
    w = W.decode_base()
    b = w.builder
    assert (w.N, w.H, w.D, w.P) == (64, 64, 512, 65536)
    assert b.win == 128 and b.swa_pages == 8192 and b.k_per_block == 1
    assert np.all(b.swa_len == 128) and np.array_equal(b.state_slot, np.arange(64))
    assert b.block_table.shape == (64, 512) and b.block_table.max() < 65536 - 8192
    for t in range(64):
        assert len(np.unique(b.block_table[t])) == 512
    assert w.softmax_scale == float(np.float32(1 / math.sqrt(512)))
    assert w.max_len == 640


def test_ragged_shape_small():
    w = W.ragged(N=16, H=4, D=64, P=4096, max_len=100)
    L = np.diff(w.kv_indptr)
    assert len(L) == 16 and np.all(L[12:] == 0) and np.all(L[:12] >= 1) and L.max() <= 100
    assert w.kv_indices.max() < 4096


def test_prefill_sliding_reuse_small():
    w = W.prefill(N=64, H=2, D=64, P=1 << 16, max_len=640)
    L = np.diff(w.kv_indptr).astype(np.int64)
    assert L.min() >= 1 and L.max() <= 640
    # the lists are exactly the windows of the stream (none cut at its end)
    m = w.meta
    assert np.array_equal(L, m["win_len"])
    for t in range(64):
        s0 = m["win_start"][t]
        assert np.array_equal(w.kv_indices[w.kv_indptr[t]:w.kv_indptr[t + 1]],
                              m["stream"][s0:s0 + m["win_len"][t]])
    # consecutive tokens share all but ceil(L_t/10) leading entries of the stream
    for t in range(63):
        a = w.kv_indices[w.kv_indptr[t]:w.kv_indptr[t + 1]]
        b = w.kv_indices[w.kv_indptr[t + 1]:w.kv_indptr[t + 2]]
        shift = (int(L[t]) + 9) // 10
        n = min(len(a) - shift, len(b))
        if n > 0:
            assert np.array_equal(a[shift:shift + n], b[:n])

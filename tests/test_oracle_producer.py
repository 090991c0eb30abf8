"""Pins of the oracle's decode-step producer (CPU): per-head RMSNorm of q, RMSNorm
of the new KV row, GPT-J RoPE on the last rope_dim entries, and the window-ring
slot of the KV row.  Each check comes from somewhere other than the oracle's own
formula: closed forms of RMSNorm (unit mean square, constant rows, scale
invariance, the weight as a per-entry factor), RoPE as complex multiplication
of (even, odd) pairs done with numpy complex arithmetic, norm preservation,
a hand-worked row, and the ring's occupancy."""
import numpy as np
import pytest

import oracle
import workloads as W


def bits(x):
    return W.bf16_bits(np.asarray(x, dtype=np.float32))


def vals(b):
    return W.bf16_to_f32(b).astype(np.float64)


def run(q, kv, qw=None, kw=None, eps=0.0, pos=None, cs=None, slot=None, win=8):
    N, H, D = q.shape
    qw = np.ones(D, np.float32) if qw is None else qw
    kw = np.ones(D, np.float32) if kw is None else kw
    pos = np.zeros(N, np.int32) if pos is None else pos
    cs = np.zeros((1, 0), np.float32) if cs is None else cs
    slot = np.zeros(N, np.int32) if slot is None else slot
    return oracle.qk_norm_rope(q, kv, qw, kw, eps, pos, cs, slot, win)


def rope_table(max_pos, rope_dim, base=10000.0):
    i = np.arange(rope_dim // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * i / rope_dim)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def test_hand_worked_row():
    # D = 4, rope on the last 2 entries; x = [1, 1, 1, 1] has mean square 1, so with
    # eps = 0 and w = [1, 2, 3, 4] the normed row is [1, 2, 3, 4]; the table row
    # (cos, sin) = (0, 1) turns the pair (3, 4) into (3*0 - 4*1, 3*1 + 4*0) = (-4, 3)
    q = bits(np.ones((1, 1, 4)))
    kv = bits(np.ones((1, 4)))
    w = np.array([1, 2, 3, 4], np.float32)
    cs = np.array([[1.0, 0.0], [0.0, 1.0]], np.float32)   # [max_pos = 2][rope_dim = 2]
    qo, ko, slot = run(q, kv, qw=w, kw=w, pos=np.array([1], np.int32), cs=cs,
                       slot=np.array([5], np.int32), win=8)
    assert np.array_equal(qo[0, 0], [1, 2, -4, 3])
    assert np.array_equal(ko[0], [1, 2, -4, 3])
    assert slot[0] == 5 * 8 + 1


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    N, H, D = 3, 4, 64
    q = bits(rng.standard_normal((N, H, D)) * 3)
    kv = bits(rng.standard_normal((N, D)))
    qo, ko, _ = run(q, kv)
    # unit mean square with w = 1 and eps = 0
    assert np.allclose((qo ** 2).mean(axis=-1), 1.0, rtol=1e-13)
    assert np.allclose((ko ** 2).mean(axis=-1), 1.0, rtol=1e-13)
    # direction kept: the output is a positive multiple of the input
    x = vals(q)
    for t in range(N):
        for h in range(H):
            r = qo[t, h][x[t, h] != 0] / x[t, h][x[t, h] != 0]
            assert r[0] > 0 and np.allclose(r, r[0], rtol=1e-13)
    # a constant row gives sign(c) * w exactly (eps = 0)
    w = rng.standard_normal(D).astype(np.float32)
    c = bits(np.full((1, 1, D), -2.5))
    qo2, _, _ = run(c, bits(np.full((1, D), 7.0)), qw=w)
    assert np.allclose(qo2[0, 0], -w.astype(np.float64), rtol=1e-15, atol=0)


def test_rmsnorm_scale_invariance_weight_and_eps():
    rng = np.random.default_rng(1)
    D = 128
    x = rng.standard_normal((1, 2, D))
    w = rng.standard_normal(D).astype(np.float32)
    base, _, _ = run(bits(x), bits(x[0, :1]), qw=w)
    scaled, _, _ = run(bits(x * 2.0 ** 20), bits(x[0, :1]), qw=w)    # exact in bf16
    assert np.allclose(base, scaled, rtol=1e-13)
    unit, _, _ = run(bits(x), bits(x[0, :1]))
    assert np.allclose(base, unit * w.astype(np.float64)[None, None, :], rtol=1e-13)
    # eps: mean square becomes ms / (ms + eps)
    ms = (vals(bits(x)) ** 2).mean(axis=-1)
    with_eps, _, _ = run(bits(x), bits(x[0, :1]), eps=0.5)
    assert np.allclose((with_eps ** 2).mean(axis=-1), ms / (ms + 0.5), rtol=1e-12)


@pytest.mark.parametrize("D,rope_dim", [(64, 64), (128, 32), (512, 64)])
def test_rope_is_complex_multiplication(D, rope_dim):
    rng = np.random.default_rng(D + rope_dim)
    N, H, max_pos = 5, 3, 300
    q = bits(rng.standard_normal((N, H, D)))
    kv = bits(rng.standard_normal((N, D)))
    cs = rope_table(max_pos, rope_dim)
    pos = rng.integers(0, max_pos, size=N).astype(np.int32)
    qo, ko, _ = run(q, kv, pos=pos, cs=cs)
    # the same rows without rotation: rope_dim 0
    qn, kn, _ = run(q, kv, pos=np.zeros(N, np.int32), cs=np.zeros((1, 0), np.float32))
    o, half = D - rope_dim, rope_dim // 2
    rot = cs[pos, :half].astype(np.float64) + 1j * cs[pos, half:].astype(np.float64)   # [N, half]
    for out, src in ((qo, qn), (ko[:, None, :], kn[:, None, :])):
        z = src[..., o::2] + 1j * src[..., o + 1::2]                   # [N, *, half]
        zr = z * rot[:, None, :]
        assert np.allclose(out[..., o::2], zr.real, rtol=1e-13, atol=1e-15)
        assert np.allclose(out[..., o + 1::2], zr.imag, rtol=1e-13, atol=1e-15)
        assert np.array_equal(out[..., :o], src[..., :o])               # untouched entries
        # pair norms kept (the table rows are unit vectors up to fp32 rounding)
        assert np.allclose(np.abs(zr), np.abs(z), rtol=1e-6)


def test_position_zero_is_identity_and_out_of_table_positions():
    rng = np.random.default_rng(3)
    N, H, D = 3, 2, 64
    q = bits(rng.standard_normal((N, H, D)))
    kv = bits(rng.standard_normal((N, D)))
    cs = rope_table(16, 32)
    qo, ko, slot = run(q, kv, pos=np.array([0, 16, -1], np.int32), cs=cs,
                       slot=np.array([2, 3, 4], np.int32), win=8)
    qn, kn, _ = run(q, kv)
    assert np.array_equal(qo[0], qn[0]) and np.array_equal(ko[0], kn[0])   # cos 1, sin 0
    assert slot.tolist() == [16, -1, -1]
    assert np.all(qo[1:] == 0) and np.all(ko[1:] == 0)


def test_ring_occupancy():
    """Positions p - win + 1 .. p of one request fill every slot of its ring once,
    and the next position takes the slot of the oldest one."""
    win, s, P = 8, 3, 40
    N = P
    q = bits(np.ones((N, 1, 2)))
    kv = bits(np.ones((N, 2)))
    cs = np.zeros((P, 0), np.float32)   # no rotary part
    pos = np.arange(P, dtype=np.int32)
    _, _, slot = run(q, kv, pos=pos, cs=cs, slot=np.full(N, s, np.int32), win=win)
    for p in range(win - 1, P):
        window = slot[p - win + 1: p + 1]
        assert sorted(window.tolist()) == list(range(s * win, s * win + win))
        if p + 1 < P:
            assert slot[p + 1] == slot[p - win + 1]


def test_without_rotary_part_positions_have_no_table_bound():
    """rope_dim = 0 reads no table, so any position >= 0 is stored (slot p mod win)
    and only a negative one is skipped."""
    q = bits(np.ones((3, 1, 4)))
    kv = bits(np.ones((3, 4)))
    _, _, slot = run(q, kv, pos=np.array([0, 1000003, -5], np.int32),
                     cs=np.zeros((0, 0), np.float32), slot=np.array([1, 2, 3], np.int32), win=8)
    assert slot.tolist() == [8, 2 * 8 + 1000003 % 8, -1]

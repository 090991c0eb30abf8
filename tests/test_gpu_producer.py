"""GPU parity of fused_qk_norm_rope_swa_store (through the C ABI) against the
oracle's producer:

* q_out and the stored bf16 KV rows within |d| <= 1e-2 + 1e-2 |ref| of the
  oracle's fp64 values (in practice within one bf16 rounding);
* the KV rows land in exactly the oracle's ring slots, every other pool row is
  left as it was, tokens whose position is outside the table write nothing;
* the FP8 store quantises the kernel's bf16 row: on every stored row, codes
  and scale equal the oracle quantiser's applied to that bf16 row, bit for
  bit, and that bf16 row lies within one bf16 ulp of the oracle's fp64 row
  (when only the FP8 pool is written, the bf16 row comes from a second call
  on the same inputs that writes the bf16 pool); every row decodes to within
  half an e4m3 spacing (plus the bf16 rounding) of the oracle's values.

Cases: every supported D, rotary widths 0, part of the row and all of it,
positions that wrap the ring, in-place q, both pools at once, a decode-base
batch (N=64, H=64, D=512), a large batch (N=1024, H=128) and batches with
a ragged tail where a wave takes two rows."""
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


def rope_table(max_pos, rope_dim, base=10000.0):
    i = np.arange(rope_dim // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * i / rope_dim)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def bf16_ulp(x64: np.ndarray) -> np.ndarray:
    """The spacing of bf16 values at |x| (8 significant bits), for normal x."""
    _, e = np.frexp(np.abs(x64))  # |x| = m 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 8)


def make_case(seed, N, H, D, rope_dim, win, n_slots, max_pos=4096):
    rng = np.random.default_rng(seed)
    q = W.normal_bf16(rng, (N, H, D), std=2.0)
    kv = W.normal_bf16(rng, (N, D))
    qw = (1.0 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    kw = (1.0 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    pos = rng.integers(0, max_pos, size=N).astype(np.int32)
    slot = rng.permutation(n_slots)[:N].astype(np.int32)
    cs = rope_table(max_pos, rope_dim)
    return q, kv, qw, kw, pos, cs, slot


def run_and_check(spd, case, win, num_rows, eps=1e-6, fp8=True, bf16=True, in_place=False,
                  what=""):
    q, kv, qw, kw, pos, cs, slot = case
    N, H, D = q.shape
    qo_ref, kv_ref, slot_ref = oracle.qk_norm_rope(q, kv, qw, kw, eps, pos, cs, slot, win)
    dq = to_dev(q)
    pool = torch.full((num_rows, D), 0.5, dtype=torch.bfloat16, device=dev()) if bf16 else None
    kv8 = torch.full((num_rows, D), 0x5A, dtype=torch.uint8, device=dev()) if fp8 else None
    ksc = torch.full((num_rows,), -1.0, dtype=torch.float32, device=dev()) if fp8 else None
    q_out = dq if in_place else torch.full_like(dq, 3.0)
    spd.fused_qk_norm_rope_swa_store(dq, to_dev(kv), to_dev(qw), to_dev(kw), eps, to_dev(pos),
                                     to_dev(cs) if cs.shape[1] else None, to_dev(slot), win,
                                     unified_kv=pool, kv_fp8=kv8, kv_scale=ksc, q_out=q_out)
    torch.cuda.synchronize()
    live = slot_ref >= 0
    got_q = bf16_to_f64(q_out)
    assert_close(got_q[live], qo_ref[live], "q_out " + what)
    if not in_place and (~live).any():
        assert np.all(got_q[~live] == 3.0), "a token outside the table wrote q_out"
    stored = slot_ref[live]
    untouched = np.setdiff1d(np.arange(num_rows), stored)
    if bf16:
        p = bf16_to_f64(pool)
        assert_close(p[stored], kv_ref[live], "kv row " + what)
        assert np.all(p[untouched] == 0.5), "a pool row outside the ring slots changed"
    if fp8:
        codes = kv8.cpu().numpy()
        scales = ksc.cpu().numpy()
        assert np.all(codes[untouched] == 0x5A) and np.all(scales[untouched] == -1.0)
        # the kernel's own bf16 rows: from this call's bf16 pool, or from a
        # second call on the same inputs that writes only a bf16 pool
        if bf16:
            gpu_rows = pool[torch.from_numpy(stored.astype(np.int64)).to(dev())]
        else:
            pool2 = torch.full((num_rows, D), 0.5, dtype=torch.bfloat16, device=dev())
            spd.fused_qk_norm_rope_swa_store(to_dev(q), to_dev(kv), to_dev(qw), to_dev(kw), eps,
                                             to_dev(pos), to_dev(cs) if cs.shape[1] else None,
                                             to_dev(slot), win, unified_kv=pool2,
                                             q_out=torch.empty_like(dq))
            torch.cuda.synchronize()
            gpu_rows = pool2[torch.from_numpy(stored.astype(np.int64)).to(dev())]
        gpu_bits = gpu_rows.view(torch.int16).cpu().numpy().view(np.uint16)
        gpu64 = bf16_to_f64(gpu_rows)
        ref = kv_ref[live]
        ulp = bf16_ulp(np.maximum(np.abs(ref), np.abs(gpu64)))
        tiny = np.abs(ref) < 2.0 ** -120  # below the normal range no ulp applies
        assert np.all((np.abs(gpu64 - ref) <= ulp) | tiny), "a bf16 row is more than 1 ulp off"
        ref_codes, ref_scales = oracle.quantize_fp8(gpu_bits)
        assert np.array_equal(codes[stored], ref_codes), "FP8 codes differ from the oracle's"
        assert np.array_equal(scales[stored].view(np.uint32), ref_scales.view(np.uint32)), \
            "FP8 scales differ from the oracle's"
        table = np.array([oracle.e4m3_value(c) for c in range(256)])
        dec = table[codes[stored]] * scales[stored][:, None]
        # half a spacing of e4m3 (2^-4 of the value, or 2^-10 * scale below 2^-6 * scale)
        # plus the bf16 rounding of the row and of the amax
        s = scales[stored][:, None].astype(np.float64)
        bound = 0.5 * np.maximum(np.abs(kv_ref[live]) * 2.0 ** -3, s * 2.0 ** -9) + \
            np.abs(kv_ref[live]) * 2.0 ** -7 + 1e-6
        assert np.all(np.abs(dec - kv_ref[live]) <= bound)
    return q_out


@pytest.mark.parametrize("D,rope_dim", [(64, 64), (64, 0), (128, 32), (256, 64), (512, 64),
                                        (512, 512)])
def test_matches_oracle(spd, D, rope_dim):
    log("case producer D=%d rope_dim=%d" % (D, rope_dim))
    N, H, win = 37, 12, 16
    case = make_case(D + rope_dim, N, H, D, rope_dim, win, n_slots=60)
    run_and_check(spd, case, win, num_rows=60 * win + 7, what="D=%d rope=%d" % (D, rope_dim))


def test_in_place_wrapping_positions_and_skipped_tokens(spd):
    log("case producer in place, wrap, skipped tokens")
    N, H, D, win, max_pos = 24, 8, 512, 8, 100
    q, kv, qw, kw, pos, cs, slot = make_case(5, N, H, D, 64, win, n_slots=30, max_pos=max_pos)
    # tokens 0..7: one request at consecutive positions 13..20, which wrap its
    # ring of 8 (slots 5, 6, 7, 0, 1, 2, 3, 4 of ring 2); the others have rings
    # of their own
    pos[:8] = np.arange(8) + 13
    slot[:8] = 2
    slot[8:] = np.random.default_rng(6).permutation(np.arange(3, 30))[:N - 8]
    pos[8] = -1                          # outside the table: nothing written
    pos[9] = max_pos                     # outside the table
    run_and_check(spd, (q, kv, qw, kw, pos, cs, slot), win, num_rows=30 * win, in_place=True,
                  what="in place")


def test_fp8_pool_alone_and_bf16_pool_alone(spd):
    log("case producer single pools")
    case = make_case(9, 20, 4, 256, 64, 32, n_slots=25)
    run_and_check(spd, case, 32, num_rows=25 * 32, bf16=False, what="fp8 only")
    run_and_check(spd, case, 32, num_rows=25 * 32, fp8=False, what="bf16 only")


@pytest.mark.parametrize("N,H", [(64, 64), (1024, 128)])
def test_decode_batches(spd, N, H):
    """decode_base's batch shape and the large one's (D=512, a 64-wide rotary
    part, win=128, one ring per token as in those configurations)."""
    log("case producer N=%d H=%d" % (N, H))
    D, win = 512, 128
    q, kv, qw, kw, pos, cs, slot = make_case(11 + N, N, H, D, 64, win, n_slots=N)
    slot = np.arange(N, dtype=np.int32)
    run_and_check(spd, (q, kv, qw, kw, pos, cs, slot), win, num_rows=N * win, what="N=%d" % N)


@pytest.mark.parametrize("N,H,D", [(255, 128, 128), (257, 128, 64)])
def test_two_rows_a_wave_with_ragged_tail(spd, N, H, D):
    """Batches of at least 32768 rows, where a wave takes two consecutive rows:
    N * H + N odd and not a multiple of eight (waves of the last workgroup with
    one live row or none), tokens outside the table, in place."""
    rows = N * H + N
    assert rows >= 32768 and rows % 8 != 0 and rows % 2 == 1
    log("case producer two rows a wave N=%d H=%d D=%d" % (N, H, D))
    win = 16
    q, kv, qw, kw, pos, cs, slot = make_case(77 + N, N, H, D, 64 if D >= 128 else 32, win,
                                             n_slots=N + 3)
    pos[3] = -5
    pos[N - 1] = 4096
    run_and_check(spd, (q, kv, qw, kw, pos, cs, slot), win, num_rows=(N + 3) * win,
                  in_place=True, what="two rows N=%d" % N)

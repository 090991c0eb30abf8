"""Host logic of bench.py (no GPU): the algorithmic byte counts its roofline
records divide by, the stream coverage of the shared-window record, and the
refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_hand_count():
    # three tokens with 2, 0, 3 rows; H = 4 heads, D = 8
    indptr = np.array([0, 2, 2, 5])
    ab = bench.algorithmic_bytes(indptr, N=3, H=4, D=8)
    assert ab["sum_L"] == 5 and ab["nonempty"] == 2
    assert ab["kv_bytes"] == 5 * 8 * 2
    assert ab["qo_bytes"] == 2 * 4 * 8 * 2 + 3 * 4 * 8 * 2      # q of non-empty tokens, all of out
    assert ab["B_alg"] == 80 + 320 + 4 * 5 + 4 * 4 + 4 * 4


def test_covered_positions_matches_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(50):
        S = int(rng.integers(1, 200))
        n = int(rng.integers(0, 30))
        start = rng.integers(-20, S + 20, size=n)
        length = rng.integers(-5, 60, size=n)
        seen = set()
        for s0, l0 in zip(start.tolist(), length.tolist()):
            if s0 >= 0 and l0 > 0 and s0 + l0 <= S:
                seen.update(range(s0, s0 + l0))
        assert bench.covered_positions(S, start, length) == len(seen)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_fp8_kernel_name_follows_the_plan():
    import sparse_paged_decode_ragged_amd as spd

    def name(N, H, D, max_len=0):
        return bench.fp8_kernel(spd.sparse_decode_attn_fp8_plan_info(N, H, D, max_len), D)
    # decode_base (H = 64): rows kernel; large (N = 1024, H = 128): one
    # 128-head workgroup per token fills the chip
    assert name(64, 64, 512, 640) == "attn_rows_fp8_kernel<512>"
    assert name(1024, 128, 512, 640) == "attn_wide_fp8_kernel<512,4>"
    assert name(255, 128, 512) == "attn_rows_fp8_kernel<512>"
    assert name(256, 128, 64) == "attn_rows_fp8_kernel<64>"
    # H = 64: two 32-head waves a workgroup once there are two per CU; four
    # waves (two parities of each head block) when there is one per CU
    assert name(8192, 64, 512, 640) == "attn_wide_fp8_kernel<512,2>"
    assert name(511, 64, 512) == "attn_wide_fp8_kernel<512,4,2>"
    assert name(256, 64, 512, 640) == "attn_wide_fp8_kernel<512,4,2>"
    # at most one 64-head workgroup per CU and slices up to 2048 rows: split mode
    assert name(256, 64, 512, 2048) == "attn_split_kernel<512,2,2,true>"
    assert name(255, 64, 512) == "attn_rows_fp8_kernel<512>"
    assert name(256, 64, 64) == "attn_rows_fp8_kernel<64>"
    # a small batch of long slices: split mode over codes
    assert name(8, 64, 512, 8192) == "attn_split_kernel<512,2,2,true>"
    assert name(8, 32, 256, 8192) == "attn_split_kernel<256,1,4,true>"


def test_mfma_flops_hand_count():
    # two tokens with 3 and 2 rows, H = 4, D = 8: per row and head, q.k takes
    # D multiplies and D adds, and p.v the same again
    assert bench.mfma_flops(5, H=4, D=8) == 5 * 4 * (2 * 8 + 2 * 8)
    # decode_base: 40,960 rows, 64 heads, D = 512
    assert bench.mfma_flops(40960, 64, 512) == 5368709120


def test_touched_bytes_and_one_cu_parts():
    import bench
    idx = np.array([5, 7, 5, 9, 7, 7], dtype=np.int32)
    tb = bench.touched_bytes(idx, N=2, H=3, D=8)
    assert tb["unique_rows"] == 3 and tb["gathered_rows"] == 6
    assert tb["unique_row_fraction"] == 0.5
    # 3 rows of 16 bytes, q and out of 2*3*8 bf16 each, 6 indices, 3 indptr entries
    assert tb["bytes"] == 3 * 16 + 2 * 2 * 3 * 8 * 2 + 4 * 6 + 4 * 3
    assert bench.touched_bytes(np.zeros(0, np.int32), 1, 1, 8)["unique_rows"] == 0
    assert bench.one_cu_parts(64) == 4 and bench.one_cu_parts(1024) == 1
    assert bench.one_cu_parts(1) == 32 and bench.one_cu_parts(8) == 32

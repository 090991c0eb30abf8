"""GPU parity of the FP8 pool calls (through the C ABI):

* quantize_kv_fp8 against the oracle's quantiser, bit for bit (codes and
  scales): both take every rounding decision in fp32 with the same IEEE
  operations;
* sparse_decode_attn_fp8 against the oracle's attention over the same FP8 pool
  (made by the oracle's quantiser from seeded bf16 rows), within
  |d| <= 1e-2 + 1e-2 |ref|.

Cases: every supported D, head counts that are not a multiple of 16, empty and
ragged slices, a slice longer than the 2048 indices staged at a time, zero
rows (scale 0), a -inf sink, rows planted late in a slice whose scores lie
far above the first tile (the fixed reference maximum then takes the second
pass), slots that scatter, skip and leave rows untouched; the 32-head-wave
kernel (128- and 64-head workgroups) on ragged tile edges, a restaged slice,
every code and the second pass; and the decode-base, ragged, large and
prefill configurations at full size, every token."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import assert_close, bf16_to_f64, dev, device_csr, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spd():
    import sparse_paged_decode_ragged_amd as m
    return m


def to_dev_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def rows_with_magnitudes(rng, n, D):
    """bf16 rows of mixed scale: N(0, 1) times a per-row factor in [2^-30, 2^30],
    plus zero rows, rows below the 2^-64 zero-row threshold, rows with
    negative zeros and rows holding exact e4m3 ties."""
    x = rng.standard_normal((n, D)).astype(np.float32)
    x *= (2.0 ** rng.uniform(-30, 30, size=(n, 1))).astype(np.float32)
    bits = W.bf16_bits(x)
    bits[1] = 0                                   # a zero row
    bits[2] = W.bf16_bits(x[2] * np.float32(2.0 ** -70) / np.abs(x[2]).max())  # amax < 2^-64
    bits[3, ::2] = 0x8000                         # negative zeros in a nonzero row
    # row 4: amax 448 (scale 1) and midpoints between consecutive e4m3 values
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    row = rng.choice(mids, size=D).astype(np.float32) * np.where(rng.random(D) < 0.5, -1, 1)
    row[0] = 448.0
    bits[4] = W.bf16_bits(row)
    return bits


@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_quantize_matches_oracle_bit_for_bit(spd, D):
    log("case fp8 quantize D=%d" % D)
    rng = np.random.default_rng(100 + D)
    n, P = 300, 420
    bits = rows_with_magnitudes(rng, n, D)
    slots = rng.permutation(P)[:n].astype(np.int32)
    slots[7] = -1                                  # skipped
    slots[8] = P + 3                               # skipped
    codes_ref, scales_ref = oracle.quantize_fp8(bits)
    kv8 = torch.full((P, D), 0x5A, dtype=torch.uint8, device=dev())
    ksc = torch.full((P,), -1.0, dtype=torch.float32, device=dev())
    spd.quantize_kv_fp8(to_dev_bits(bits), kv8, ksc, torch.from_numpy(slots).to(dev()))
    torch.cuda.synchronize()
    got_codes, got_scales = kv8.cpu().numpy(), ksc.cpu().numpy()
    ok = (slots >= 0) & (slots < P)
    assert np.array_equal(got_codes[slots[ok]], codes_ref[ok])
    assert np.array_equal(got_scales[slots[ok]].view(np.uint32), scales_ref[ok].view(np.uint32))
    untouched = np.setdiff1d(np.arange(P), slots[ok])
    assert np.all(got_codes[untouched] == 0x5A) and np.all(got_scales[untouched] == -1.0)


def test_quantize_without_slots(spd):
    log("case fp8 quantize no slots")
    rng = np.random.default_rng(7)
    bits = rows_with_magnitudes(rng, 37, 512)
    kv8 = torch.zeros((40, 512), dtype=torch.uint8, device=dev())
    ksc = torch.zeros(40, dtype=torch.float32, device=dev())
    spd.quantize_kv_fp8(to_dev_bits(bits), kv8.view(torch.float8_e4m3fn), ksc)
    torch.cuda.synchronize()
    codes_ref, scales_ref = oracle.quantize_fp8(bits)
    assert np.array_equal(kv8.cpu().numpy()[:37], codes_ref)
    assert np.array_equal(ksc.cpu().numpy()[:37], scales_ref)


def fp8_pool(rng, P, D, zero_rows=None):
    """(bf16 bits, codes, scales): seeded N(0, 1) rows quantised by the oracle;
    zero_rows are zero."""
    x = rng.standard_normal((P, D)).astype(np.float32)
    if zero_rows is not None:
        x[zero_rows] = 0.0
    bits = W.bf16_bits(x)
    codes, scales = oracle.quantize_fp8(bits)
    return bits, codes, scales


def run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, scale):
    q = to_dev_bits(q_bits)
    kv8 = torch.from_numpy(codes).to(dev())
    ksc = torch.from_numpy(scales).to(dev())
    di, dp = device_csr(idx, ptr)
    out = spd.sparse_decode_attn_fp8(q, kv8, ksc, di, dp, torch.from_numpy(sink).to(dev()), scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("seed,H,D,lengths", [
    (1, 8, 64, [0, 1, 17, 64, 3]),
    (2, 24, 128, [5, 0, 130, 16, 33]),
    (3, 64, 256, [200, 1, 0, 64]),
    (4, 64, 512, [640, 0, 15, 16, 17, 300]),
    (5, 16, 512, [2500, 7]),                 # more than 2048 indices: staged twice
    (6, 128, 512, [48, 96]),
])
def test_attention_matches_oracle(spd, seed, H, D, lengths):
    log("case fp8 attention seed=%d H=%d D=%d L=%s" % (seed, H, D, lengths))
    rng = np.random.default_rng(seed)
    N, P = len(lengths), 3000
    _, codes, scales = fp8_pool(rng, P, D, zero_rows=rng.choice(P, size=20, replace=False))
    idx, ptr = W.csr_from_lists([rng.integers(0, P, size=L) for L in lengths])
    q_bits = W.normal_bf16(rng, (N, H, D))
    sink = rng.standard_normal(H).astype(np.float32)
    sink[0] = -np.inf
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, scale)
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, scale)
    assert_close(bf16_to_f64(out), ref, "fp8 H=%d D=%d" % (H, D))
    empty = np.nonzero(np.diff(ptr) == 0)[0]
    if len(empty):
        assert torch.all(out[torch.from_numpy(empty).to(dev())].view(torch.int16) == 0)


def test_every_code_decodes_exactly(spd):
    """Single-row slices and no sink: the output is the row itself,
    scale * e4m3(code), which bf16 holds exactly for a power-of-two scale.  The
    rows hold every finite code (subnormals and both zeros included), each code
    in several column positions, so every conversion path must be exact."""
    log("case fp8 every code")
    H, D, P = 16, 512, 8
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = np.stack([np.resize(np.roll(finite, 37 * r), D) for r in range(P)]).astype(np.uint8)
    scales = (2.0 ** np.arange(-4, 4)).astype(np.float32)
    idx, ptr = W.csr_from_lists([[r] for r in range(P)])
    q_bits = W.normal_bf16(np.random.default_rng(5), (P, H, D))
    sink = np.full(H, -np.inf, dtype=np.float32)
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, 0.05)
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, 0.05)
    assert np.array_equal(bf16_to_f64(out), ref)


def test_attention_second_pass(spd):
    """Rows planted late in a slice, parallel to q[t, 0], score far (> 64 in
    log2 units) above the first tile, so the reference maximum fixed there is
    left behind and the kernel redoes the state with the true maximum.  Two
    planted rows of nearby scores keep the output a genuine mix of rows."""
    log("case fp8 attention second pass")
    rng = np.random.default_rng(11)
    H, D, P = 32, 512, 4000
    lengths = [300, 700, 40, 2100]
    lists = [rng.choice(P, size=L, replace=False) for L in lengths]
    idx, ptr = W.csr_from_lists(lists)
    q_bits = W.normal_bf16(rng, (len(lengths), H, D))
    q = W.bf16_to_f32(q_bits)
    x = rng.standard_normal((P, D)).astype(np.float32)
    plants = {0: (100, 290), 1: (150, 650), 3: (1000, 2090)}
    for t, (p2, p1) in plants.items():
        x[lists[t][p1]] = 4.0 * q[t, 0]            # score ~ 90 in log2 units
        x[lists[t][p2]] = 3.9 * q[t, 0]            # about 2 lower
    codes, scales = oracle.quantize_fp8(W.bf16_bits(x))
    sink = rng.standard_normal(H).astype(np.float32)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, scale)
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, scale)
    assert_close(bf16_to_f64(out), ref, "fp8 second pass")


def test_decode_base_config(spd):
    """decode_base (N=64, H=64, D=512, 640 rows a token) with its pool
    quantised by the oracle; every token against the oracle."""
    log("case fp8 decode_base")
    w = W.decode_base()
    b = w.builder
    ptr, idx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos, b.block_table,
                                           b.win, b.k_per_block, b.swa_pages)
    codes, scales = oracle.quantize_fp8(w.kv_bits)
    out = run_fp8(spd, w.q_bits, codes, scales, idx, ptr, w.attn_sink, w.softmax_scale)
    ref = oracle.sparse_decode_attn_fp8(w.q_bits, codes, scales, idx, ptr, w.attn_sink,
                                        w.softmax_scale)
    assert_close(bf16_to_f64(out), ref, "fp8 decode_base")


# --- workgroups of 32-head waves: 128 heads (H % 128 == 0, N * H / 128 >= 256)
# or 64 heads (H % 64 == 0, N * H / 64 >= 512) ---

WIDE_N = 256  # the smallest batch that takes the 32-head-wave kernel at H = 128
# (H, N): 128-head workgroups on four waves, 64-head ones on two, four waves
# with two head groups a token, and 64-head workgroups on four waves (two
# parities of each head block: a batch of one workgroup per CU at H = 64)
WIDE_SHAPES = [(128, 256), (64, 512), (256, 128), (64, 256)]


def wide_lengths(rng, n, long=()):
    """Lengths of every kind: empty, 1, around the 32-row tile (31, 32, 33, 63,
    64, 65), random up to 200, and the given long ones."""
    L = rng.integers(0, 200, size=n)
    edge = [0, 1, 31, 32, 33, 63, 64, 65, 0, 2]
    L[:len(edge)] = edge
    for i, v in enumerate(long):
        L[len(edge) + i] = v
    return L


@pytest.mark.parametrize("H,N", WIDE_SHAPES)
@pytest.mark.parametrize("D", [128, 256, 512])
def test_wide_attention_matches_oracle(spd, D, H, N):
    log("case fp8 wide attention D=%d H=%d N=%d" % (D, H, N))
    rng = np.random.default_rng(40 + D + H)
    P = 5000
    lengths = wide_lengths(rng, N, long=(2300,) if D == 512 else ())
    _, codes, scales = fp8_pool(rng, P, D, zero_rows=rng.choice(P, size=20, replace=False))
    idx, ptr = W.csr_from_lists([rng.integers(0, P, size=L) for L in lengths])
    q_bits = W.normal_bf16(rng, (N, H, D))
    sink = rng.standard_normal(H).astype(np.float32)
    sink[5] = -np.inf
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, scale)
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, scale)
    assert_close(bf16_to_f64(out), ref, "fp8 wide D=%d H=%d" % (D, H))
    empty = np.nonzero(np.diff(ptr) == 0)[0]
    assert torch.all(out[torch.from_numpy(empty).to(dev())].view(torch.int16) == 0)


@pytest.mark.parametrize("H,N", WIDE_SHAPES)
def test_wide_every_code_decodes_exactly(spd, H, N):
    """As test_every_code_decodes_exactly, on the 32-head-wave kernel: each
    token's slice is one row and there is no sink, so the output is the row,
    scale * e4m3(code), exactly."""
    log("case fp8 wide every code H=%d" % H)
    D, P = 512, 8
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = np.stack([np.resize(np.roll(finite, 37 * r), D) for r in range(P)]).astype(np.uint8)
    scales = (2.0 ** np.arange(-4, 4)).astype(np.float32)
    idx, ptr = W.csr_from_lists([[t % P] for t in range(N)])
    q_bits = W.normal_bf16(np.random.default_rng(6), (N, H, D))
    sink = np.full(H, -np.inf, dtype=np.float32)
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, 0.05)
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, 0.05)
    assert np.array_equal(bf16_to_f64(out), ref)


@pytest.mark.parametrize("H,N", WIDE_SHAPES)
def test_wide_attention_second_pass(spd, H, N):
    """Rows planted late in some slices score far above their first tile, on
    the 32-head-wave kernel (as test_attention_second_pass)."""
    log("case fp8 wide second pass H=%d" % H)
    rng = np.random.default_rng(12)
    D, P = 512, 6000
    lengths = rng.integers(1, 120, size=N)
    lengths[[3, 77, 100]] = [300, 700, 2100]
    lists = [rng.choice(P, size=L, replace=False) for L in lengths]
    idx, ptr = W.csr_from_lists(lists)
    q_bits = W.normal_bf16(rng, (N, H, D))
    q = W.bf16_to_f32(q_bits)
    x = rng.standard_normal((P, D)).astype(np.float32)
    for t, (p2, p1) in {3: (100, 290), 77: (150, 650), 100: (1000, 2090)}.items():
        x[lists[t][p1]] = 4.0 * q[t, 0]            # score ~ 90 in log2 units
        x[lists[t][p2]] = 3.9 * q[t, 0]            # about 2 lower
    codes, scales = oracle.quantize_fp8(W.bf16_bits(x))
    sink = rng.standard_normal(H).astype(np.float32)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = run_fp8(spd, q_bits, codes, scales, idx, ptr, sink, scale)
    tokens = np.array([0, 3, 77, 100, N - 1])
    sidx, sptr = W.csr_from_lists([lists[t] for t in tokens])
    ref = oracle.sparse_decode_attn_fp8(q_bits[tokens], codes, scales, sidx, sptr, sink, scale)
    assert_close(bf16_to_f64(out[torch.from_numpy(tokens).to(dev())]), ref, "fp8 wide second pass")


# --- the ragged, large and prefill configurations at full size over FP8 pools,
# in the launch configuration the benchmark times (32-head waves: 128 heads a
# workgroup for large, 64 for prefill; rows mode for ragged), every token ---

@pytest.fixture
def device_data():
    W.set_data_mode("device", dev())
    yield
    W.set_data_mode("host")


def check_fp8_config(spd, w, idx_np, ptr_np, what, chunk=512):
    """Quantise the whole bf16 pool on the GPU, run the FP8 call over all
    tokens, then check every token, chunk tokens at a time: the codes and
    scales of the rows they read bit for bit against the oracle's quantiser,
    their outputs against the oracle's FP8 attention over those rows."""
    from gpu_helpers import device_inputs
    q, kv, sink = device_inputs(w)
    kv8 = torch.empty((w.P, w.D), dtype=torch.uint8, device=dev())
    ksc = torch.empty(w.P, dtype=torch.float32, device=dev())
    spd.quantize_kv_fp8(kv, kv8, ksc)
    idx, ptr = device_csr(idx_np, ptr_np)
    out = spd.sparse_decode_attn_fp8(q, kv8, ksc, idx, ptr, sink, w.softmax_scale)
    torch.cuda.synchronize()
    for t0 in range(0, w.N, chunk):
        tokens = np.arange(t0, min(w.N, t0 + chunk))
        lists = [idx_np[ptr_np[t]:ptr_np[t + 1]] for t in tokens]
        allidx = np.concatenate(lists) if lists else np.zeros(0, np.int32)
        uniq, inv = np.unique(allidx, return_inverse=True)
        if len(uniq) == 0:
            uniq, inv = np.zeros(1, np.int64), np.zeros(0, np.int64)
        u = torch.from_numpy(uniq.astype(np.int64)).to(dev())
        codes, scales = oracle.quantize_fp8(W.host_bits(kv[u]))
        assert np.array_equal(kv8[u].cpu().numpy(), codes), "%s: codes, tokens %d.." % (what, t0)
        assert np.array_equal(ksc[u].cpu().numpy().view(np.uint32), scales.view(np.uint32)), \
            "%s: scales, tokens %d.." % (what, t0)
        sub_ptr = np.zeros(len(tokens) + 1, dtype=np.int32)
        sub_ptr[1:] = np.cumsum([len(x) for x in lists])
        tok = torch.from_numpy(tokens.astype(np.int64)).to(dev())
        ref = oracle.sparse_decode_attn_fp8(W.host_bits(q[tok]), codes, scales,
                                            inv.astype(np.int32), sub_ptr, w.attn_sink,
                                            w.softmax_scale)
        assert_close(bf16_to_f64(out[tok]), ref, "%s tokens %d..%d" % (what, t0, tokens[-1]))
    log("  %s: all %d tokens" % (what, w.N))


def test_large_config_fp8(spd, device_data):
    w = W.large()
    log("case fp8 large: N=1024, H=128, 4 Mi rows quantised on the GPU")
    b = w.builder
    ptr, idx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos, b.block_table,
                                           b.win, b.k_per_block, b.swa_pages)
    check_fp8_config(spd, w, idx, ptr, "fp8 large", chunk=256)


def test_prefill_config_fp8(spd, device_data):
    w = W.prefill()
    log("case fp8 prefill: N=8192, H=64, L up to 640")
    check_fp8_config(spd, w, w.kv_indices, w.kv_indptr, "fp8 prefill", chunk=1024)


def test_ragged_config_fp8(spd, device_data):
    w = W.ragged()
    log("case fp8 ragged: N=256, H=64, L up to 2048, 25 % empty")
    check_fp8_config(spd, w, w.kv_indices, w.kv_indptr, "fp8 ragged", chunk=64)


# --- split mode over an FP8 pool: partitions of a slice merged inside the
# kernel (64-head workgroups on two parities of each 32-head block, or
# 32-head workgroups on four parities when H <= 32) ---

SPLIT = 4
# (H, D): 64 heads (one head group), 96 (two, the second half padding), 32
# and 24 heads (32-head workgroups, four parities)
SPLIT_SHAPES = [(64, 128), (64, 256), (64, 512), (96, 512), (32, 512), (24, 256), (32, 128)]


def split_lengths(rng, n):
    """Empty, one row, around the 32- and 64-row super-tiles and the
    partition length, random, one slice over the 1024 indices staged at a
    time, and slices of 1 to 24 partitions of 96 rows (units of every width)."""
    L = rng.integers(0, 700, size=n)
    L[:10] = [0, 1, 31, 32, 33, 95, 96, 97, 2300, 1000]
    return L


@pytest.mark.parametrize("H,D", SPLIT_SHAPES)
def test_split_attention_matches_oracle(spd, H, D):
    """Partitions of 96 rows (up to 24 of a slice) merged in-kernel: every
    token against the oracle; a second call on the same workspace gives the
    same bits (its arrival counters end every call at zero, and the merge
    sums in partition order whatever the arrival order)."""
    log("case fp8 split H=%d D=%d" % (H, D))
    rng = np.random.default_rng(60 + H + D)
    N, P = 12, 5000
    lengths = split_lengths(rng, N)
    _, codes, scales = fp8_pool(rng, P, D, zero_rows=rng.choice(P, size=20, replace=False))
    idx, ptr = W.csr_from_lists([rng.integers(0, P, size=L) for L in lengths])
    q_bits = W.normal_bf16(rng, (N, H, D))
    sink = rng.standard_normal(H).astype(np.float32)
    sink[3] = -np.inf
    scale = float(np.float32(1.0 / np.sqrt(D)))
    max_len = int(lengths.max())
    plan = spd.sparse_decode_attn_fp8_plan_info(N, H, D, max_len, 96, SPLIT)
    assert plan["mode"] == "split" and plan["splits"] == (max_len + 95) // 96
    assert plan["parities"] == (4 if H <= 32 else 2)
    q = to_dev_bits(q_bits)
    kv8 = torch.from_numpy(codes).to(dev())
    ksc = torch.from_numpy(scales).to(dev())
    di, dp = device_csr(idx, ptr)
    sk = torch.from_numpy(sink).to(dev())
    need = spd.sparse_decode_attn_fp8_workspace_size(N, H, D, max_len, 96, SPLIT)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    outs = []
    for _ in range(2):
        outs.append(spd.sparse_decode_attn_fp8(q, kv8, ksc, di, dp, sk, scale, max_len=max_len,
                                               split_rows=96, mode=SPLIT, workspace=ws))
        torch.cuda.synchronize()
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, scale)
    assert_close(bf16_to_f64(outs[0]), ref, "fp8 split H=%d D=%d" % (H, D))
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    empty = np.nonzero(np.diff(ptr) == 0)[0]
    assert torch.all(outs[0][torch.from_numpy(empty).to(dev())].view(torch.int16) == 0)


@pytest.mark.parametrize("H", [64, 32])
def test_split_every_code_decodes_exactly(spd, H):
    """Each slice is one row repeated 300 times (four partitions of 96 rows)
    and there is no sink: every weight is exactly 1, so each partition's state
    and their merge hold exact sums and the output is the row, scale *
    e4m3(code), bit for bit (the rows hold every finite code)."""
    log("case fp8 split every code H=%d" % H)
    D, P = 512, 8
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = np.stack([np.resize(np.roll(finite, 37 * r), D) for r in range(P)]).astype(np.uint8)
    scales = (2.0 ** np.arange(-4, 4)).astype(np.float32)
    idx, ptr = W.csr_from_lists([[r] * 300 for r in range(P)])
    q_bits = W.normal_bf16(np.random.default_rng(8), (P, H, D))
    sink = np.full(H, -np.inf, dtype=np.float32)
    q = to_dev_bits(q_bits)
    di, dp = device_csr(idx, ptr)
    out = spd.sparse_decode_attn_fp8(q, torch.from_numpy(codes).to(dev()),
                                     torch.from_numpy(scales).to(dev()), di, dp,
                                     torch.from_numpy(sink).to(dev()), 0.05, max_len=300,
                                     split_rows=96, mode=SPLIT)
    torch.cuda.synchronize()
    ref = np.stack([np.broadcast_to(np.array([oracle.e4m3_value(c) for c in codes[r]]) * scales[r],
                                    (H, D)) for r in range(P)])
    assert np.array_equal(bf16_to_f64(out), ref)


def test_split_attention_second_pass(spd):
    """Rows planted in late partitions of long slices score far above the
    partitions' first tiles, so those partitions take the second pass; their
    states then merge with partitions that did not."""
    log("case fp8 split second pass")
    rng = np.random.default_rng(13)
    H, D, P = 64, 512, 6000
    lengths = [300, 700, 40, 2100]
    lists = [rng.choice(P, size=L, replace=False) for L in lengths]
    idx, ptr = W.csr_from_lists(lists)
    q_bits = W.normal_bf16(rng, (len(lengths), H, D))
    q = W.bf16_to_f32(q_bits)
    x = rng.standard_normal((P, D)).astype(np.float32)
    for t, (p2, p1) in {0: (100, 290), 1: (150, 650), 3: (1000, 2090)}.items():
        x[lists[t][p1]] = 4.0 * q[t, 0]            # score ~ 90 in log2 units
        x[lists[t][p2]] = 3.9 * q[t, 0]            # about 2 lower
    codes, scales = oracle.quantize_fp8(W.bf16_bits(x))
    sink = rng.standard_normal(H).astype(np.float32)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q = to_dev_bits(q_bits)
    di, dp = device_csr(idx, ptr)
    out = spd.sparse_decode_attn_fp8(q, torch.from_numpy(codes).to(dev()),
                                     torch.from_numpy(scales).to(dev()), di, dp,
                                     torch.from_numpy(sink).to(dev()), scale, max_len=2100,
                                     split_rows=128, mode=SPLIT)
    torch.cuda.synchronize()
    ref = oracle.sparse_decode_attn_fp8(q_bits, codes, scales, idx, ptr, sink, scale)
    assert_close(bf16_to_f64(out), ref, "fp8 split second pass")


def test_long_context_config_fp8(spd, device_data):
    """The long-slice batch (N = 8 tokens of 8192 rows, H = 64, D = 512, a
    2^20-row pool) over an FP8 pool in the launch configuration the benchmark
    times: the automatic plan with max_len 8192 (split mode, 32 partitions),
    every token against the oracle."""
    w = W.long_context()
    log("case fp8 long_context: N=%d, L=%d, automatic split plan" % (w.N, w.max_len))
    plan = spd.sparse_decode_attn_fp8_plan_info(w.N, w.H, w.D, w.max_len)
    assert plan["mode"] == "split" and plan["splits"] == 32
    from gpu_helpers import device_inputs
    q, kv, sink = device_inputs(w)
    kv8 = torch.empty((w.P, w.D), dtype=torch.uint8, device=dev())
    ksc = torch.empty(w.P, dtype=torch.float32, device=dev())
    spd.quantize_kv_fp8(kv, kv8, ksc)
    idx, ptr = device_csr(w.kv_indices, w.kv_indptr)
    out = spd.sparse_decode_attn_fp8(q, kv8, ksc, idx, ptr, sink, w.softmax_scale,
                                     max_len=w.max_len)
    torch.cuda.synchronize()
    allidx = w.kv_indices
    uniq, inv = np.unique(allidx, return_inverse=True)
    u = torch.from_numpy(uniq.astype(np.int64)).to(dev())
    codes, scales = oracle.quantize_fp8(W.host_bits(kv[u]))
    assert np.array_equal(kv8[u].cpu().numpy(), codes)
    ref = oracle.sparse_decode_attn_fp8(W.host_bits(q), codes, scales, inv.astype(np.int32),
                                        w.kv_indptr, w.attn_sink, w.softmax_scale)
    assert_close(bf16_to_f64(out), ref, "fp8 long_context")

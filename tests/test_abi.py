"""The C ABI library: it loads, exports every entry point include/spd.h
declares, and rejects bad arguments on the host before any HIP call (so these
run without a GPU).  No case here passes all checks, so nothing is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.environ.get("SPD_LIB_DIR") or os.path.join(ROOT, "sparse_paged_decode_ragged_amd", "_lib")
LIB = os.path.join(LIB_DIR, "libspd.so")
HEADER = os.path.join(ROOT, "include", "spd.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # 64 KiB-aligned non-null pointer value; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspd.so not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.sparse_decode_attn.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32, P]
    L.sparse_decode_attn_ex.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32, i32,
                                        i32, i32, P, sz, P]
    L.sparse_decode_attn_noalloc.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32,
                                             i32, i32, i32, P]
    L.sparse_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.sparse_decode_attn_workspace_size.restype = sz
    L.sparse_decode_attn_can_use.argtypes = [i32, i32]
    L.build_decode_indices.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i32, P, P, i64, P]
    L.spd_validate_indices.argtypes = [P, i64, P, i32, i64, ctypes.POINTER(ctypes.c_int64), P]
    L.sparse_decode_attn_paged.argtypes = [P, P, i64, P, P, P, i32, P, i32, i32, i32, i32, P,
                                           ctypes.c_float, P, i32, i32, i32, i32, P]
    L.sparse_decode_attn_fp8.argtypes = [P, P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32, P]
    L.quantize_kv_fp8.argtypes = [P, P, i32, i32, P, P, i64, P]
    L.fused_qk_norm_rope_swa_store.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, i32, i32, P,
                                               i32, P, P, P, i64, i32, i32, i32, P]
    L.sparse_prefill_attn.argtypes = [P, P, i64, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32,
                                      i32, P]
    L.spd_status_string.argtypes = [ctypes.c_int]
    L.spd_status_string.restype = ctypes.c_char_p
    return L


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"SPD_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert set(names) >= {"sparse_decode_attn", "build_decode_indices", "sparse_decode_attn_ex",
                          "sparse_decode_attn_workspace_size", "sparse_decode_attn_can_use",
                          "spd_validate_indices", "spd_status_string", "spd_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_binding_lists_the_same_symbols():
    import ast
    src = open(os.path.join(ROOT, "sparse_paged_decode_ragged_amd", "__init__.py")).read()
    tree = ast.parse(src)
    exported = None
    for node in tree.body:
        if isinstance(node, ast.Assign) and getattr(node.targets[0], "id", "") == "EXPORTED_SYMBOLS":
            exported = ast.literal_eval(node.value)
    assert exported is not None and set(exported) == set(declared_symbols())


def test_status_strings(lib):
    assert lib.spd_status_string(0) == b"SPD_OK"
    assert lib.spd_status_string(3) == b"SPD_ERR_WORKSPACE"
    assert lib.spd_version() >= 300


@pytest.mark.parametrize("H,D,ok", [(64, 512, 1), (128, 512, 1), (8, 64, 1), (1, 128, 1),
                                    (64, 576, 0), (64, 100, 0), (0, 512, 0), (2048, 512, 0)])
def test_can_use(lib, H, D, ok):
    assert lib.sparse_decode_attn_can_use(H, D) == ok


def _attn(lib, q=FAKE, kv=FAKE, rows=100, idx=FAKE, ptr=FAKE, sink=FAKE, scale=0.1, out=FAKE * 4096,
          N=2, H=8, D=64):
    return lib.sparse_decode_attn(q, kv, rows, idx, ptr, sink, scale, out, N, H, D, None)


def test_attn_rejects_bad_arguments(lib):
    assert _attn(lib, q=None) == INVALID
    assert _attn(lib, kv=None) == INVALID
    assert _attn(lib, idx=None) == INVALID
    assert _attn(lib, ptr=None) == INVALID
    assert _attn(lib, sink=None) == INVALID
    assert _attn(lib, out=None) == INVALID
    assert _attn(lib, N=-1) == INVALID
    assert _attn(lib, H=0) == INVALID
    assert _attn(lib, rows=0) == INVALID
    assert _attn(lib, q=FAKE + 2) == INVALID           # q not 16-byte aligned
    assert _attn(lib, out=FAKE) == INVALID             # out overlaps q
    assert _attn(lib, scale=float("nan")) == INVALID
    assert _attn(lib, D=100) == UNSUPPORTED
    assert _attn(lib, N=0) == OK                       # empty batch: nothing to do


def test_attn_ex_workspace_checks(lib):
    AUTO, HEADS, ROWS, SPLIT = 0, 1, 2, 4
    # Split mode with no partition length and at most 256 (token, head group)
    # pairs: 256 workgroups in all (256 / head groups a head group), which the
    # kernel deals out as partitions sized from the lengths.  One piece slot
    # per (workgroup, wave) of 32 heads x 256 bf16 + 32 fp32 m + 32 fp32 l,
    # then 8 int32 arrival counters per (token, head group, wave): one per
    # unit of a piece cut into its 8 d-tiles
    piece = 32 * 256 * 2 + 2 * 32 * 4
    split_need = 256 * 4 * piece + 64 * 4 * 8 * 4
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, SPLIT) == split_need
    # the automatic plan keeps rows mode for 640-row slices (no workspace) and
    # splits batches of slices of 2048 rows and more
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, AUTO) == 0
    assert lib.sparse_decode_attn_workspace_size(16, 64, 512, 2048, 0, AUTO) == \
        256 * 4 * piece + 16 * 4 * 8 * 4
    # 256 tokens (one workgroup each without a split) still split: 256 slots
    assert lib.sparse_decode_attn_workspace_size(256, 64, 512, 2048, 0, AUTO) == \
        256 * 4 * piece + 256 * 4 * 8 * 4
    assert lib.sparse_decode_attn_workspace_size(256, 64, 512, 2048, 0, SPLIT) == \
        256 * 4 * piece + 256 * 4 * 8 * 4
    # two head groups (H = 128): 128 slots each; counters per (token, head group)
    assert lib.sparse_decode_attn_workspace_size(100, 128, 512, 4096, 0, AUTO) == \
        256 * 4 * piece + 100 * 2 * 4 * 8 * 4
    # past 256 pairs the automatic plan does not split (heads mode), and an
    # explicit split mode keeps one partition a slice (no workspace)
    assert lib.sparse_decode_attn_workspace_size(257, 64, 512, 2048, 0, AUTO) == 0
    assert lib.sparse_decode_attn_workspace_size(257, 64, 512, 2048, 0, SPLIT) == 0
    assert lib.sparse_decode_attn_workspace_size(2, 64, 512, 65536, 0, SPLIT) == \
        256 * 4 * piece + 2 * 4 * 8 * 4
    # a given partition length: fixed partitions, at most 32 a slice
    assert lib.sparse_decode_attn_workspace_size(2, 64, 512, 65536, 2048, SPLIT) == \
        2 * 32 * 4 * piece + 2 * 4 * 8 * 4
    assert lib.sparse_decode_attn_workspace_size(2, 64, 512, 65536, 1024, SPLIT) == 0
    # without a capacity bound the automatic plan cannot split: rows mode, no workspace
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 0, 0, AUTO) == 0
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, ROWS) == 0
    # heads mode splits a 640-row slice into 4 partitions of 160 rows:
    # 64 tokens x 1 head group x 4 partitions x 64 heads x (512 + 2) floats
    need = lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, HEADS)
    assert need == 64 * 1 * 4 * 64 * 514 * 4
    assert lib.sparse_decode_attn_workspace_size(1024, 128, 512, 640, 0, AUTO) == 0  # no split
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 64, AUTO) == 64 * 10 * 64 * 514 * 4
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 64, ROWS) == 0  # invalid plan
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, 7) == 0      # unknown mode

    def ex(max_len=640, split=0, mode=HEADS, ws=None, ws_bytes=0):
        return lib.sparse_decode_attn_ex(FAKE, FAKE, 100, FAKE, FAKE, FAKE, 0.1, FAKE * 4096, 64, 64,
                                         512, max_len, split, mode, ws, ws_bytes, None)
    assert ex() == WORKSPACE
    assert ex(ws=FAKE * 8192, ws_bytes=need - 1) == WORKSPACE
    assert ex(max_len=-1) == INVALID
    assert ex(mode=7) == INVALID
    assert ex(mode=ROWS, split=64) == UNSUPPORTED
    WIDE = 3
    assert ex(mode=WIDE, split=64) == UNSUPPORTED    # 32-head waves never split
    assert lib.sparse_decode_attn_ex(FAKE, FAKE, 100, FAKE, FAKE, FAKE, 0.1, FAKE * 4096, 64, 40,
                                     512, 640, 0, WIDE, None, 0, None) == UNSUPPORTED  # H % 64
    assert lib.sparse_decode_attn_workspace_size(64, 64, 512, 640, 0, WIDE) == 0


def _build(lib, ss=FAKE, sl=FAKE, cp=FAKE, topk=4, bt=FAKE, mb=2, N=3, win=8, k=2, swa=24,
           ptr=FAKE, idx=FAKE, cap=None):
    if cap is None:
        cap = N * (win + topk)
    return lib.build_decode_indices(ss, sl, cp, topk, bt, mb, N, win, k, swa, ptr, idx, cap, None)


def test_builder_rejects_bad_arguments(lib):
    assert _build(lib, win=0) == INVALID        # would divide by zero / index out of range
    assert _build(lib, win=-3) == INVALID
    assert _build(lib, k=0) == INVALID
    assert _build(lib, N=-1) == INVALID
    assert _build(lib, cap=3 * 12 - 1) == INVALID   # capacity below N*(win+topk)
    assert _build(lib, cp=None) == INVALID          # topk > 0 without comp_pos
    assert _build(lib, bt=None) == INVALID
    assert _build(lib, mb=0) == INVALID
    assert _build(lib, ptr=None) == INVALID
    assert _build(lib, ss=None) == INVALID
    assert _build(lib, swa=-1) == INVALID
    assert _build(lib, N=1 << 20, win=1 << 12, topk=0, cp=None, cap=1 << 40) == INVALID  # > 2^31 entries


def test_validate_rejects_bad_arguments(lib):
    first = ctypes.c_int64(0)
    assert lib.spd_validate_indices(FAKE, 10, None, 2, 100, ctypes.byref(first), None) == INVALID
    assert lib.spd_validate_indices(None, 10, FAKE, 2, 100, ctypes.byref(first), None) == INVALID
    assert lib.spd_validate_indices(FAKE, 10, FAKE, -1, 100, ctypes.byref(first), None) == INVALID


def _paged(lib, q=FAKE, kv=FAKE, rows=100, ss=FAKE, sl=FAKE, cp=FAKE, topk=4, bt=FAKE, mb=2, win=8,
           k=2, swa=24, sink=FAKE, scale=0.1, out=FAKE * 4096, N=2, H=8, D=64, mode=0):
    return lib.sparse_decode_attn_paged(q, kv, rows, ss, sl, cp, topk, bt, mb, win, k, swa, sink,
                                        scale, out, N, H, D, mode, None)


def test_paged_attn_rejects_bad_arguments(lib):
    # the builder's argument rules
    assert _paged(lib, win=0) == INVALID
    assert _paged(lib, k=0) == INVALID
    assert _paged(lib, swa=-1) == INVALID
    assert _paged(lib, topk=-1) == INVALID
    assert _paged(lib, cp=None) == INVALID          # topk > 0 without comp_pos
    assert _paged(lib, bt=None) == INVALID
    assert _paged(lib, mb=0) == INVALID
    assert _paged(lib, ss=None) == INVALID
    assert _paged(lib, sl=None) == INVALID
    # the attention call's rules
    assert _paged(lib, q=None) == INVALID
    assert _paged(lib, kv=None) == INVALID
    assert _paged(lib, sink=None) == INVALID
    assert _paged(lib, out=None) == INVALID
    assert _paged(lib, rows=0) == INVALID
    assert _paged(lib, q=FAKE + 2) == INVALID       # q not 16-byte aligned
    assert _paged(lib, out=FAKE) == INVALID         # out overlaps q
    assert _paged(lib, scale=float("inf")) == INVALID
    assert _paged(lib, mode=5) == INVALID
    assert _paged(lib, D=100) == UNSUPPORTED
    # a token's list is built whole in LDS: win + topk <= 2048
    assert _paged(lib, win=1024, topk=1025) == UNSUPPORTED
    assert _paged(lib, N=0) == OK                   # empty batch: nothing to do
    assert _paged(lib, N=0, topk=0, cp=None, bt=None, mb=0) == OK


def _fp8(lib, q=FAKE, kv=FAKE, sc=FAKE * 8192, rows=100, idx=FAKE, ptr=FAKE, sink=FAKE, scale=0.1,
         out=FAKE * 4096, N=2, H=8, D=64):
    return lib.sparse_decode_attn_fp8(q, kv, sc, rows, idx, ptr, sink, scale, out, N, H, D, None)


def test_fp8_attn_rejects_bad_arguments(lib):
    assert _fp8(lib, N=0) == OK                          # nothing to do
    assert _fp8(lib, N=-1) == INVALID
    assert _fp8(lib, rows=0) == INVALID
    assert _fp8(lib, H=0) == INVALID
    assert _fp8(lib, D=100) == UNSUPPORTED
    assert _fp8(lib, H=2048) == UNSUPPORTED
    assert _fp8(lib, scale=float("nan")) == INVALID
    assert _fp8(lib, kv=None) == INVALID
    assert _fp8(lib, sc=None) == INVALID
    assert _fp8(lib, idx=None) == INVALID
    assert _fp8(lib, kv=FAKE + 8) == INVALID           # codes must be 16-byte aligned
    assert _fp8(lib, sc=FAKE * 8192 + 2) == INVALID    # scales 4-byte aligned
    assert _fp8(lib, q=FAKE + 4) == INVALID
    assert _fp8(lib, out=FAKE) == INVALID               # out overlaps q (both at FAKE)
    assert _fp8(lib, out=FAKE * 8192) == INVALID        # out overlaps the scales
    assert _fp8(lib, rows=1 << 41) == INVALID


def test_fp8_plans_and_ex_checks(lib):
    """The FP8 pool's plans (host only): split mode for small batches of long
    slices as for the bf16 pool, the 32-head-wave decompositions by batch
    size, and the mode, shape and workspace checks of sparse_decode_attn_fp8_ex."""
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.sparse_decode_attn_fp8_ex.argtypes = [P, P, P, ctypes.c_int64, P, P, P, ctypes.c_float, P,
                                              i32, i32, i32, i32, i32, i32, P, sz, P]
    lib.sparse_decode_attn_fp8_workspace_size.argtypes = [i32] * 6
    lib.sparse_decode_attn_fp8_workspace_size.restype = sz
    lib.sparse_decode_attn_fp8_plan_info.argtypes = [i32] * 6 + [ctypes.POINTER(ctypes.c_int32)]
    AUTO, HEADS, ROWS, WIDE, SPLIT = 0, 1, 2, 3, 4

    def info(N, H, D, max_len=0, split=0, mode=AUTO):
        out = (ctypes.c_int32 * 7)()
        st = lib.sparse_decode_attn_fp8_plan_info(N, H, D, max_len, split, mode, out)
        return st, list(out)

    # 8 tokens of 8192 rows: split mode, 64 heads a workgroup, up to 32
    # partitions a slice sized in the kernel (rows 0); the same workspace
    # layout as the bf16 pool's split mode: 256 workgroup slots
    st, i = info(8, 64, 512, 8192)
    assert st == OK and i == [SPLIT, 64, 1, 32, 0, 0, 2]
    assert lib.sparse_decode_attn_fp8_workspace_size(8, 64, 512, 8192, 0, AUTO) == \
        lib.sparse_decode_attn_workspace_size(8, 64, 512, 8192, 0, AUTO) == \
        256 * 4 * (32 * 256 * 2 + 2 * 32 * 4) + 8 * 4 * 8 * 4
    assert info(8, 32, 256, 8192)[1][:7] == [SPLIT, 32, 1, 32, 0, 0, 4]
    # no capacity bound, or slices under 2048 rows: no split
    assert info(8, 64, 512)[1][0] == ROWS
    assert info(64, 64, 512, 640)[1][0] == ROWS
    assert info(8, 64, 64, 8192)[1][0] == ROWS            # D = 64: no FP8 split kernel
    # the batch sizes of the 32-head-wave decompositions
    assert info(1024, 128, 512, 640)[1][:6] == [HEADS, 128, 1, 1, 1 << 30, 4]
    assert info(8192, 64, 512, 640)[1][:6] == [HEADS, 64, 1, 1, 1 << 30, 2]
    assert info(257, 64, 512, 2048)[1][:6] == [HEADS, 64, 1, 1, 1 << 30, 3]
    assert info(256, 64, 512, 2048)[1][:5] == [SPLIT, 64, 1, 32, 0]   # 256 slices: split
    assert info(255, 64, 512)[1][0] == ROWS
    # explicit modes
    assert info(8, 64, 512, 0, 0, WIDE)[1][5] == 2
    assert info(8, 128, 512, 0, 0, WIDE)[1][5] == 4
    assert info(64, 64, 512, 640, 0, ROWS)[1][0] == ROWS
    assert info(64, 64, 512, 640, 0, SPLIT)[1][:5] == [SPLIT, 64, 1, 20, 0]
    assert info(8, 64, 512, 8192, 1024, AUTO)[1][:5] == [SPLIT, 64, 1, 8, 1024]  # split_rows: split
    assert info(8, 64, 512, 0, 0, HEADS)[0] == UNSUPPORTED     # no FP8 heads kernel
    assert info(8, 64, 64, 0, 0, SPLIT)[0] == UNSUPPORTED
    assert info(8, 64, 64, 0, 0, WIDE)[0] == UNSUPPORTED
    assert info(8, 40, 512, 0, 0, WIDE)[0] == UNSUPPORTED      # H % 64
    assert info(8, 64, 512, 640, 64, ROWS)[0] == UNSUPPORTED
    assert info(8, 64, 64, 640, 64, AUTO)[0] == UNSUPPORTED
    assert info(8, 64, 512, 0, 0, 7)[0] == INVALID
    assert info(8, 64, 512, 65536, 1024, SPLIT)[0] == INVALID  # over 32 partitions
    assert lib.sparse_decode_attn_fp8_workspace_size(8, 64, 512, 0, 0, HEADS) == 0

    def ex(N=8, H=64, D=512, max_len=8192, split=0, mode=AUTO, ws=None, ws_bytes=0, scale=0.1):
        return lib.sparse_decode_attn_fp8_ex(FAKE, FAKE, FAKE * 8192, 100, FAKE, FAKE, FAKE, scale,
                                             FAKE * 4096, N, H, D, max_len, split, mode, ws,
                                             ws_bytes, None)
    need = lib.sparse_decode_attn_fp8_workspace_size(8, 64, 512, 8192, 0, AUTO)
    assert ex() == WORKSPACE
    assert ex(ws=FAKE * 16384, ws_bytes=need - 1) == WORKSPACE
    assert ex(ws=FAKE * 16384 + 8, ws_bytes=need) == INVALID    # workspace 16-byte aligned
    assert ex(max_len=-1) == INVALID
    assert ex(split=-1) == INVALID
    assert ex(mode=7) == INVALID
    assert ex(mode=HEADS) == UNSUPPORTED
    assert ex(D=64, mode=SPLIT) == UNSUPPORTED
    assert ex(mode=ROWS, split=64) == UNSUPPORTED
    assert ex(H=40, mode=WIDE, max_len=0) == UNSUPPORTED
    assert ex(scale=float("inf")) == INVALID
    assert ex(N=0) == OK


def _quant(lib, src=FAKE, slots=None, n=4, D=64, kv=FAKE * 4096, sc=FAKE * 8192, rows=100):
    return lib.quantize_kv_fp8(src, slots, n, D, kv, sc, rows, None)


def test_quantize_rejects_bad_arguments(lib):
    assert _quant(lib, n=0) == OK
    assert _quant(lib, n=-1) == INVALID
    assert _quant(lib, rows=0) == INVALID
    assert _quant(lib, D=0) == INVALID
    assert _quant(lib, D=96) == UNSUPPORTED
    assert _quant(lib, D=576) == UNSUPPORTED
    assert _quant(lib, src=None) == INVALID
    assert _quant(lib, kv=None) == INVALID
    assert _quant(lib, sc=None) == INVALID
    assert _quant(lib, src=FAKE + 8) == INVALID         # 16-byte alignment
    assert _quant(lib, kv=FAKE * 4096 + 4) == INVALID
    assert _quant(lib, sc=FAKE * 8192 + 1) == INVALID
    assert _quant(lib, slots=FAKE * 16 + 2) == INVALID
    assert _quant(lib, n=200, rows=100) == INVALID      # without slots, row i goes to row i
    assert _quant(lib, kv=FAKE) == INVALID              # pool overlaps the source
    assert _quant(lib, sc=FAKE * 4096 + 64 * 50) == INVALID   # scales inside the codes
    assert _quant(lib, slots=FAKE * 8192, n=4) == INVALID     # slots overlap the scales


def _prod(lib, q=FAKE, q_out=FAKE * 16, kv=FAKE * 32, qw=FAKE * 48, kw=FAKE * 48 + 4096,
          eps=1e-6, pos=FAKE * 64, cs=FAKE * 80, max_pos=16, rope_dim=64, slot=FAKE * 96, win=8,
          pool=FAKE * 4096, fp8=None, sc=None, rows=1000, N=4, H=8, D=512):
    return lib.fused_qk_norm_rope_swa_store(q, q_out, kv, qw, kw, eps, pos, cs, max_pos, rope_dim,
                                            slot, win, pool, fp8, sc, rows, N, H, D, None)


def test_producer_rejects_bad_arguments(lib):
    assert _prod(lib, N=0) == OK
    assert _prod(lib, N=-1) == INVALID
    assert _prod(lib, H=0) == INVALID
    assert _prod(lib, D=96) == UNSUPPORTED
    assert _prod(lib, D=1024) == UNSUPPORTED
    assert _prod(lib, win=0) == INVALID
    assert _prod(lib, rows=0) == INVALID
    assert _prod(lib, rope_dim=63) == INVALID            # odd
    assert _prod(lib, rope_dim=600) == INVALID           # > D
    assert _prod(lib, rope_dim=-2) == INVALID
    assert _prod(lib, eps=-1.0) == INVALID
    assert _prod(lib, eps=float("nan")) == INVALID
    assert _prod(lib, eps=float("inf")) == INVALID
    assert _prod(lib, pool=None) == INVALID              # no pool to store into
    assert _prod(lib, pool=None, fp8=FAKE * 4096) == INVALID   # FP8 pool without scales
    assert _prod(lib, cs=None) == INVALID                # rope_dim > 0 needs the table
    assert _prod(lib, max_pos=0) == INVALID
    assert _prod(lib, q=None) == INVALID
    assert _prod(lib, kv=None) == INVALID
    assert _prod(lib, pos=None) == INVALID
    assert _prod(lib, q=FAKE + 8) == INVALID             # 16-byte alignment
    assert _prod(lib, pool=FAKE * 4096 + 4) == INVALID
    assert _prod(lib, qw=FAKE * 48 + 2) == INVALID
    assert _prod(lib, q_out=FAKE + 1024) == INVALID      # partial overlap with q
    assert _prod(lib, pool=FAKE * 16) == INVALID         # pool over q_out
    assert _prod(lib, pool=FAKE * 32 - 4096) == INVALID  # pool over kv
    assert _prod(lib, fp8=FAKE * 8192, sc=FAKE * 8192 + 1000) == INVALID   # scales in the codes


def _pre(lib, q=FAKE, kv=FAKE * 64, rows=100, stream=FAKE * 128, slen=1000, ws=FAKE * 144,
         wl=FAKE * 160, sink=FAKE * 176, scale=0.1, out=FAKE * 4096, N=4, H=64, D=512, T=0):
    return lib.sparse_prefill_attn(q, kv, rows, stream, slen, ws, wl, sink, scale, out, N, H, D,
                                   T, None)


def test_prefill_rejects_bad_arguments(lib):
    assert _pre(lib, N=0) == OK
    assert _pre(lib, N=-1) == INVALID
    assert _pre(lib, rows=0) == INVALID
    assert _pre(lib, slen=-1) == INVALID
    assert _pre(lib, slen=1 << 31) == INVALID
    assert _pre(lib, H=48) == UNSUPPORTED       # 128 / H tokens per workgroup: H in {32, 64, 128}
    assert _pre(lib, H=256) == UNSUPPORTED
    assert _pre(lib, T=-1) == INVALID
    assert _pre(lib, T=3) == UNSUPPORTED         # 3 x 64 query rows fill no workgroup
    assert _pre(lib, H=128, T=2) == UNSUPPORTED
    assert _pre(lib, H=32, T=1) == UNSUPPORTED
    assert _pre(lib, D=96) == UNSUPPORTED
    assert _pre(lib, scale=float("inf")) == INVALID
    assert _pre(lib, stream=None) == INVALID     # a non-empty stream needs its pointer
    assert _pre(lib, ws=None) == INVALID
    assert _pre(lib, wl=None) == INVALID
    assert _pre(lib, kv=FAKE * 64 + 8) == INVALID
    assert _pre(lib, stream=FAKE * 128 + 2) == INVALID
    assert _pre(lib, out=FAKE) == INVALID         # over q
    assert _pre(lib, out=FAKE * 128 - 1024) == INVALID   # over the stream


def test_noalloc_rejects_plans_beyond_its_workspace(lib):
    """The allocation-free call checks every argument, then the plan's
    workspace against the 96 MiB it holds per GPU, before any HIP call."""
    AUTO, HEADS, SPLIT = 0, 1, 4
    limit = 96 << 20
    args = lambda N, max_len, split_rows, mode, scale=0.1, q=FAKE: (
        q, FAKE, 1 << 20, FAKE, FAKE, FAKE, scale, 1 << 40, N, 64, 512, max_len, split_rows,
        mode, None)
    # 4096 tokens of 64 heads in 8 partitions of 256 rows: 4096 * 8 * 64 * 514 * 4 bytes
    need = lib.sparse_decode_attn_workspace_size(4096, 64, 512, 2048, 256, HEADS)
    assert need > limit
    assert lib.sparse_decode_attn_noalloc(*args(4096, 2048, 256, HEADS)) == WORKSPACE
    # split mode past the limit too
    assert lib.sparse_decode_attn_workspace_size(1024, 64, 512, 4096, 256, SPLIT) > limit
    assert lib.sparse_decode_attn_noalloc(*args(1024, 4096, 256, SPLIT)) == WORKSPACE
    # argument errors come first, as in sparse_decode_attn_ex
    assert lib.sparse_decode_attn_noalloc(*args(4096, 2048, 256, HEADS, scale=float("nan"))) == INVALID
    assert lib.sparse_decode_attn_noalloc(*args(4096, 2048, 256, 7)) == INVALID
    assert lib.sparse_decode_attn_noalloc(*args(4096, 2048, 256, HEADS, q=None)) == INVALID
    # nothing to do
    assert lib.sparse_decode_attn_noalloc(*args(0, 2048, 256, HEADS)) == OK
    # the automatic plans fit: every batch of up to 255 heads-mode workgroups
    worst = max(lib.sparse_decode_attn_workspace_size(N, H, 512, L, 0, m)
                for N in (1, 2, 3, 5, 63, 64, 127, 255) for H in (64, 128, 256)
                for L in (2048, 8192, 65536) for m in (AUTO, HEADS, SPLIT))
    assert 0 < worst <= limit


PROBE_LIB = os.path.join(LIB_DIR, "libspd_probe.so")
PROBE_HEADER = os.path.join(ROOT, "include", "spd_probe.h")


def test_probe_library_exports_and_host_checks():
    """libspd_probe.so exports what include/spd_probe.h declares and rejects
    bad arguments before any HIP call."""
    if not os.path.exists(PROBE_LIB):
        pytest.fail("libspd_probe.so not built; run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE_LIB)
    names = re.findall(r"SPD_PROBE_API\s+[\w\s\*]+?\b(\w+)\s*\(", open(PROBE_HEADER).read())
    assert set(names) == {"spd_probe_gather", "spd_probe_null", "spd_probe_store"}
    for n in names:
        assert hasattr(L, n), n
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.spd_probe_gather.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
    L.spd_probe_null.argtypes = [i32, P]
    L.spd_probe_store.argtypes = [P, i64, i32, P]
    g = lambda **k: L.spd_probe_gather(k.get("kv", FAKE), FAKE, FAKE, k.get("N", 4), k.get("D", 512),
                                       k.get("groups", 1), k.get("parts", 1), FAKE, None)
    assert g(D=96) == 1 and g(groups=0) == 1 and g(parts=0) == 1 and g(N=-1) == 1
    assert g(kv=FAKE + 8) == 1 and g(kv=None) == 1
    assert g(N=1 << 20, groups=64, parts=64) == 1
    assert g(N=0) == 0
    assert L.spd_probe_null(0, None) == 1
    assert L.spd_probe_store(FAKE, 100, 256, None) == 1
    assert L.spd_probe_store(FAKE, 64, 0, None) == 1
    assert L.spd_probe_store(None, 64, 256, None) == 1
    assert L.spd_probe_store(FAKE, 0, 256, None) == 0


@pytest.mark.skipif(not os.environ.get("SPD_EXPECT_SANITIZED"),
                    reason="only in the sanitized run (tests/run_sanitized.sh)")
def test_sanitized_builds_are_the_ones_loaded(lib):
    """In the sanitized run the process has loaded the instrumented libspd and
    oracle (their sanitizer hooks are present), not the plain builds."""
    import oracle
    oracle.sparse_decode_attn  # noqa: B018  (module loaded)
    oracle._load()
    maps = open("/proc/self/maps").read()
    assert os.path.join(LIB_DIR, "libspd.so") in maps
    assert os.path.basename(os.path.normpath(LIB_DIR)) == "sanitize"
    assert os.environ["SPD_ORACLE_LIB"] in maps and "/sanitize/" in os.environ["SPD_ORACLE_LIB"]
    assert hasattr(ctypes.CDLL(None), "__asan_init")

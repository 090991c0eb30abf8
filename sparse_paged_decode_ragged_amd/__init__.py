"""Python binding of libspd: sparse decode attention over a unified paged KV
pool and its decode index builder, hand-written HIP for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/spd.h``.  PyTorch provides
device memory and the current stream.  There is no fallback: if the built
library is missing, importing this package raises.

Call names follow the C ABI:

* ``sparse_decode_attn(q, unified_kv, kv_indices, kv_indptr, attn_sink,
  softmax_scale, out=None, *, max_len=0, split_rows=0, workspace=None)``
* ``build_decode_indices(state_slot, swa_len, comp_pos, block_table, win,
  k_per_block, swa_pages, kv_indptr=None, kv_indices=None)``
* ``sparse_decode_attn_paged(q, unified_kv, state_slot, swa_len, comp_pos,
  block_table, win, k_per_block, swa_pages, attn_sink, softmax_scale,
  out=None)`` -- the two above in one kernel (the page transform fused into
  the attention call; no kv_indices in memory)
* ``sparse_prefill_attn(q, unified_kv, kv_stream, win_start, win_len, attn_sink,
  softmax_scale, out=None)`` -- the same attention for tokens whose row lists
  are windows of one index stream (consecutive tokens sharing rows)
* ``sparse_decode_attn_fp8(q, kv_fp8, kv_scale, kv_indices, kv_indptr,
  attn_sink, softmax_scale, out=None, *, max_len=0, split_rows=0, mode=0,
  workspace=None)`` -- the same attention over an FP8 pool (e4m3 codes times a
  per-row fp32 scale), with the plans of ``sparse_decode_attn_fp8_ex``
  (split mode included); ``sparse_decode_attn_fp8_workspace_size`` and
  ``sparse_decode_attn_fp8_plan_info`` as for the bf16 pool
* ``quantize_kv_fp8(src, kv_fp8, kv_scale, slots=None)`` -- the quantising
  store that fills such a pool
* ``fused_qk_norm_rope_swa_store(q, kv, q_weight, kv_weight, eps, positions,
  cos_sin, state_slot, win, unified_kv=None, kv_fp8=None, kv_scale=None,
  q_out=None)`` -- the decode-step producer that writes the rows the attention
  reads (RMSNorm + RoPE of q and the KV row, KV row into its window-ring slot)
* ``sparse_decode_attn_workspace_size``, ``sparse_decode_attn_can_use``,
  ``validate_indices``
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPD_LIB_DIR selects another build of the same library (build.py --sanitize
# writes a host-sanitized one to _lib/sanitize)
LIB_DIR = os.environ.get("SPD_LIB_DIR") or os.path.join(_PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libspd.so")

SPD_OK = 0
_STATUS = {0: "SPD_OK", 1: "SPD_ERR_INVALID_ARG", 2: "SPD_ERR_UNSUPPORTED", 3: "SPD_ERR_WORKSPACE",
           4: "SPD_ERR_HIP"}

EXPORTED_SYMBOLS = (
    "spd_status_string", "spd_version", "sparse_decode_attn_can_use", "sparse_decode_attn",
    "sparse_decode_attn_workspace_size", "sparse_decode_attn_ex", "build_decode_indices",
    "spd_validate_indices", "sparse_decode_attn_plan_info", "sparse_decode_attn_paged",
    "sparse_decode_attn_fp8", "quantize_kv_fp8", "fused_qk_norm_rope_swa_store",
    "sparse_prefill_attn", "sparse_decode_attn_noalloc", "sparse_decode_attn_fp8_ex",
    "sparse_decode_attn_fp8_workspace_size", "sparse_decode_attn_fp8_plan_info",
)


class SpdError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__("%s failed: %s" % (call, _STATUS.get(status, "status %d" % status)))
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libspd.so is not built (expected at %s); run "
                          "sparse_paged_decode_ragged_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.spd_status_string.argtypes = [ctypes.c_int]
    lib.spd_status_string.restype = ctypes.c_char_p
    lib.spd_version.argtypes = []
    lib.spd_version.restype = ctypes.c_int
    lib.sparse_decode_attn_can_use.argtypes = [i32, i32]
    lib.sparse_decode_attn_can_use.restype = ctypes.c_int
    lib.sparse_decode_attn.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32, P]
    lib.sparse_decode_attn.restype = ctypes.c_int
    lib.sparse_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.sparse_decode_attn_workspace_size.restype = sz
    lib.sparse_decode_attn_ex.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32, i32,
                                          i32, i32, P, sz, P]
    lib.sparse_decode_attn_ex.restype = ctypes.c_int
    lib.sparse_decode_attn_noalloc.argtypes = [P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32,
                                               i32, i32, i32, P]
    lib.sparse_decode_attn_noalloc.restype = ctypes.c_int
    lib.sparse_decode_attn_paged.argtypes = [P, P, i64, P, P, P, i32, P, i32, i32, i32, i32, P,
                                             ctypes.c_float, P, i32, i32, i32, i32, P]
    lib.sparse_decode_attn_paged.restype = ctypes.c_int
    lib.sparse_decode_attn_fp8.argtypes = [P, P, P, i64, P, P, P, ctypes.c_float, P, i32, i32, i32,
                                           P]
    lib.sparse_decode_attn_fp8.restype = ctypes.c_int
    lib.sparse_decode_attn_fp8_ex.argtypes = [P, P, P, i64, P, P, P, ctypes.c_float, P, i32, i32,
                                              i32, i32, i32, i32, P, sz, P]
    lib.sparse_decode_attn_fp8_ex.restype = ctypes.c_int
    lib.sparse_decode_attn_fp8_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.sparse_decode_attn_fp8_workspace_size.restype = sz
    lib.sparse_decode_attn_fp8_plan_info.argtypes = [i32, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(ctypes.c_int32)]
    lib.sparse_decode_attn_fp8_plan_info.restype = ctypes.c_int
    lib.quantize_kv_fp8.argtypes = [P, P, i32, i32, P, P, i64, P]
    lib.sparse_prefill_attn.argtypes = [P, P, i64, P, i64, P, P, P, ctypes.c_float, P, i32, i32,
                                        i32, i32, P]
    lib.sparse_prefill_attn.restype = ctypes.c_int
    lib.quantize_kv_fp8.restype = ctypes.c_int
    lib.fused_qk_norm_rope_swa_store.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, i32, i32, P,
                                                 i32, P, P, P, i64, i32, i32, i32, P]
    lib.fused_qk_norm_rope_swa_store.restype = ctypes.c_int
    lib.build_decode_indices.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i32, P, P, i64, P]
    lib.build_decode_indices.restype = ctypes.c_int
    lib.spd_validate_indices.argtypes = [P, i64, P, i32, i64, ctypes.POINTER(ctypes.c_int64), P]
    lib.spd_validate_indices.restype = ctypes.c_int
    lib.sparse_decode_attn_plan_info.argtypes = [i32, i32, i32, i32, i32, i32,
                                                 ctypes.POINTER(ctypes.c_int32)]
    lib.sparse_decode_attn_plan_info.restype = ctypes.c_int
    return lib


lib = _load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims" % (name, ndim))


def _raise_on(status: int, call: str):
    if status != SPD_OK:
        raise SpdError(status, call)


def sparse_decode_attn_can_use(H: int, D: int) -> bool:
    return bool(lib.sparse_decode_attn_can_use(int(H), int(D)))


MODE_AUTO, MODE_HEADS, MODE_ROWS, MODE_WIDE, MODE_SPLIT = 0, 1, 2, 3, 4


def sparse_decode_attn_workspace_size(N: int, H: int, D: int, max_len: int = 0,
                                      split_rows: int = 0, mode: int = MODE_AUTO) -> int:
    return int(lib.sparse_decode_attn_workspace_size(int(N), int(H), int(D), int(max_len),
                                                     int(split_rows), int(mode)))


def sparse_decode_attn_plan_info(N: int, H: int, D: int, max_len: int = 0, split_rows: int = 0,
                                 mode: int = MODE_AUTO) -> dict:
    info = (ctypes.c_int32 * 7)()
    st = lib.sparse_decode_attn_plan_info(int(N), int(H), int(D), int(max_len), int(split_rows),
                                          int(mode), info)
    _raise_on(st, "sparse_decode_attn_plan_info")
    return {"mode": {1: "heads", 2: "rows", 4: "split"}[info[0]], "heads_per_group": info[1],
            "head_groups": info[2], "splits": info[3],
            "split_rows": info[4] if info[3] > 1 else None, "wide": bool(info[5]),
            "parities": info[6], "balanced": info[0] == 4 and info[3] > 1 and info[4] == 0}


def sparse_decode_attn(q: torch.Tensor, unified_kv: torch.Tensor, kv_indices: torch.Tensor,
                       kv_indptr: torch.Tensor, attn_sink: torch.Tensor, softmax_scale: float,
                       out: Optional[torch.Tensor] = None, *, max_len: int = 0,
                       split_rows: int = 0, mode: int = MODE_AUTO,
                       workspace: Optional[torch.Tensor] = None,
                       plain: bool = False) -> torch.Tensor:
    """out[N, H, D] (bf16) = sparse decode attention; see include/spd.h.

    plain=True calls the plain form ``sparse_decode_attn`` (automatic
    plan, never split-L, no workspace).  Otherwise ``sparse_decode_attn_ex``
    runs with (max_len, split_rows, mode); ``workspace`` (a device tensor of
    at least ``sparse_decode_attn_workspace_size`` bytes) is allocated here
    when needed and not given -- pass one in when capturing a graph.
    """
    _check(q, "q", torch.bfloat16, 3)
    _check(unified_kv, "unified_kv", torch.bfloat16, 2)
    _check(kv_indices, "kv_indices", torch.int32, 1)
    _check(kv_indptr, "kv_indptr", torch.int32, 1)
    _check(attn_sink, "attn_sink", torch.float32, 1)
    N, H, D = q.shape
    if unified_kv.shape[1] != D or kv_indptr.shape[0] != N + 1 or attn_sink.shape[0] != H:
        raise ValueError("shape mismatch between q, unified_kv, kv_indptr and attn_sink")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (N, H, D):
            raise ValueError("out must be [N, H, D]")
    idx = kv_indices if kv_indices.numel() > 0 else kv_indptr  # any valid pointer; never read
    stream = _stream(q.device)
    if plain:
        st = lib.sparse_decode_attn(_ptr(q), _ptr(unified_kv), unified_kv.shape[0], _ptr(idx),
                                    _ptr(kv_indptr), _ptr(attn_sink), float(softmax_scale),
                                    _ptr(out), N, H, D, stream)
        _raise_on(st, "sparse_decode_attn")
        return out
    need = sparse_decode_attn_workspace_size(N, H, D, max_len, split_rows, mode)
    if need > 0 and workspace is None:
        # zero-filled: a split-mode workspace's arrival counters must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.sparse_decode_attn_ex(_ptr(q), _ptr(unified_kv), unified_kv.shape[0], _ptr(idx),
                                   _ptr(kv_indptr), _ptr(attn_sink), float(softmax_scale),
                                   _ptr(out), N, H, D, int(max_len), int(split_rows), int(mode),
                                   _ptr(workspace), ws_bytes, stream)
    _raise_on(st, "sparse_decode_attn_ex")
    return out


# Workspace the library holds per GPU for sparse_decode_attn_noalloc.
NOALLOC_WORKSPACE_BYTES = 96 << 20


def sparse_decode_attn_noalloc(q: torch.Tensor, unified_kv: torch.Tensor,
                               kv_indices: torch.Tensor, kv_indptr: torch.Tensor,
                               attn_sink: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                               *, max_len: int = 0, split_rows: int = 0,
                               mode: int = MODE_AUTO) -> torch.Tensor:
    """``sparse_decode_attn_noalloc``: sparse_decode_attn_ex with the library's
    per-GPU workspace, so the call allocates nothing (``out`` is required).
    Calls that may overlap on one GPU race on that workspace."""
    _check(q, "q", torch.bfloat16, 3)
    _check(unified_kv, "unified_kv", torch.bfloat16, 2)
    _check(kv_indices, "kv_indices", torch.int32, 1)
    _check(kv_indptr, "kv_indptr", torch.int32, 1)
    _check(attn_sink, "attn_sink", torch.float32, 1)
    _check(out, "out", torch.bfloat16, 3)
    N, H, D = q.shape
    if unified_kv.shape[1] != D or kv_indptr.shape[0] != N + 1 or attn_sink.shape[0] != H:
        raise ValueError("shape mismatch between q, unified_kv, kv_indptr and attn_sink")
    if tuple(out.shape) != (N, H, D):
        raise ValueError("out must be [N, H, D]")
    idx = kv_indices if kv_indices.numel() > 0 else kv_indptr  # any valid pointer; never read
    st = lib.sparse_decode_attn_noalloc(_ptr(q), _ptr(unified_kv), unified_kv.shape[0], _ptr(idx),
                                        _ptr(kv_indptr), _ptr(attn_sink), float(softmax_scale),
                                        _ptr(out), N, H, D, int(max_len), int(split_rows),
                                        int(mode), _stream(q.device))
    _raise_on(st, "sparse_decode_attn_noalloc")
    return out


def build_decode_indices(state_slot: torch.Tensor, swa_len: torch.Tensor,
                         comp_pos: Optional[torch.Tensor], block_table: Optional[torch.Tensor],
                         win: int, k_per_block: int, swa_pages: int,
                         kv_indptr: Optional[torch.Tensor] = None,
                         kv_indices: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Ragged-packed (kv_indptr [N+1], kv_indices [N*(win+topk)] capacity), int32 device tensors.

    Only kv_indices[:kv_indptr[N]] is meaningful; reading kv_indptr[N] on the
    host is the caller's choice (this call never synchronises).
    """
    _check(state_slot, "state_slot", torch.int32, 1)
    _check(swa_len, "swa_len", torch.int32, 1)
    N = state_slot.shape[0]
    topk, max_blocks = 0, 0
    if comp_pos is not None:
        _check(comp_pos, "comp_pos", torch.int32, 2)
        _check(block_table, "block_table", torch.int32, 2)
        topk, max_blocks = comp_pos.shape[1], block_table.shape[1]
        if comp_pos.shape[0] != N or block_table.shape[0] != N:
            raise ValueError("comp_pos and block_table must have N rows")
    cap = N * (int(win) + topk)
    dev = state_slot.device
    if kv_indptr is None:
        kv_indptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    if kv_indices is None:
        kv_indices = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check(kv_indptr, "kv_indptr", torch.int32, 1)
    _check(kv_indices, "kv_indices", torch.int32, 1)
    st = lib.build_decode_indices(_ptr(state_slot), _ptr(swa_len), _ptr(comp_pos), topk,
                                  _ptr(block_table), max_blocks, N, int(win), int(k_per_block),
                                  int(swa_pages), _ptr(kv_indptr), _ptr(kv_indices),
                                  kv_indices.numel(), _stream(dev))
    _raise_on(st, "build_decode_indices")
    return kv_indptr, kv_indices


def sparse_decode_attn_paged(q: torch.Tensor, unified_kv: torch.Tensor, state_slot: torch.Tensor,
                             swa_len: torch.Tensor, comp_pos: Optional[torch.Tensor],
                             block_table: Optional[torch.Tensor], win: int, k_per_block: int,
                             swa_pages: int, attn_sink: torch.Tensor, softmax_scale: float,
                             out: Optional[torch.Tensor] = None, *,
                             mode: int = MODE_AUTO) -> torch.Tensor:
    """out[N, H, D] (bf16): build_decode_indices + sparse_decode_attn in one
    kernel, with each token's rows derived on the device (see include/spd.h).
    Needs win + topk <= 2048; never splits, so it takes no workspace."""
    _check(q, "q", torch.bfloat16, 3)
    _check(unified_kv, "unified_kv", torch.bfloat16, 2)
    _check(state_slot, "state_slot", torch.int32, 1)
    _check(swa_len, "swa_len", torch.int32, 1)
    _check(attn_sink, "attn_sink", torch.float32, 1)
    N, H, D = q.shape
    if unified_kv.shape[1] != D or attn_sink.shape[0] != H or state_slot.shape[0] != N or \
            swa_len.shape[0] != N:
        raise ValueError("shape mismatch between q, unified_kv, state_slot, swa_len and attn_sink")
    topk, max_blocks = 0, 0
    if comp_pos is not None:
        _check(comp_pos, "comp_pos", torch.int32, 2)
        _check(block_table, "block_table", torch.int32, 2)
        topk, max_blocks = comp_pos.shape[1], block_table.shape[1]
        if comp_pos.shape[0] != N or block_table.shape[0] != N:
            raise ValueError("comp_pos and block_table must have N rows")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (N, H, D):
            raise ValueError("out must be [N, H, D]")
    st = lib.sparse_decode_attn_paged(_ptr(q), _ptr(unified_kv), unified_kv.shape[0],
                                      _ptr(state_slot), _ptr(swa_len), _ptr(comp_pos), topk,
                                      _ptr(block_table), max_blocks, int(win), int(k_per_block),
                                      int(swa_pages), _ptr(attn_sink), float(softmax_scale),
                                      _ptr(out), N, H, D, int(mode), _stream(q.device))
    _raise_on(st, "sparse_decode_attn_paged")
    return out


def sparse_prefill_attn(q: torch.Tensor, unified_kv: torch.Tensor, kv_stream: torch.Tensor,
                        win_start: torch.Tensor, win_len: torch.Tensor, attn_sink: torch.Tensor,
                        softmax_scale: float, out: Optional[torch.Tensor] = None, *,
                        tokens_per_group: int = 0) -> torch.Tensor:
    """out[N, H, D] (bf16): token t attends to
    kv_stream[win_start[t] : win_start[t] + win_len[t]]; tokens_per_group
    consecutive tokens share a workgroup (0: automatic; see include/spd.h)."""
    _check(q, "q", torch.bfloat16, 3)
    _check(unified_kv, "unified_kv", torch.bfloat16, 2)
    _check(kv_stream, "kv_stream", torch.int32, 1)
    _check(win_start, "win_start", torch.int32, 1)
    _check(win_len, "win_len", torch.int32, 1)
    _check(attn_sink, "attn_sink", torch.float32, 1)
    N, H, D = q.shape
    if unified_kv.shape[1] != D or win_start.shape[0] != N or win_len.shape[0] != N or \
            attn_sink.shape[0] != H:
        raise ValueError("shape mismatch between q, unified_kv, the windows and attn_sink")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (N, H, D):
            raise ValueError("out must be [N, H, D]")
    st = lib.sparse_prefill_attn(_ptr(q), _ptr(unified_kv), unified_kv.shape[0],
                                 _ptr(kv_stream) if kv_stream.numel() > 0 else None,
                                 kv_stream.numel(), _ptr(win_start), _ptr(win_len),
                                 _ptr(attn_sink), float(softmax_scale), _ptr(out), N, H, D,
                                 int(tokens_per_group), _stream(q.device))
    _raise_on(st, "sparse_prefill_attn")
    return out


def _fp8_codes(t: torch.Tensor, name: str) -> torch.Tensor:
    """An FP8 pool tensor as its uint8 codes (float8_e4m3fn is viewed, not converted)."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _check(t, name, torch.uint8, 2)
    return t


def sparse_decode_attn_fp8_workspace_size(N: int, H: int, D: int, max_len: int = 0,
                                          split_rows: int = 0, mode: int = MODE_AUTO) -> int:
    return int(lib.sparse_decode_attn_fp8_workspace_size(int(N), int(H), int(D), int(max_len),
                                                         int(split_rows), int(mode)))


def sparse_decode_attn_fp8_plan_info(N: int, H: int, D: int, max_len: int = 0,
                                     split_rows: int = 0, mode: int = MODE_AUTO) -> dict:
    info = (ctypes.c_int32 * 7)()
    st = lib.sparse_decode_attn_fp8_plan_info(int(N), int(H), int(D), int(max_len),
                                              int(split_rows), int(mode), info)
    _raise_on(st, "sparse_decode_attn_fp8_plan_info")
    return {"mode": {1: "heads", 2: "rows", 4: "split"}[info[0]], "heads_per_group": info[1],
            "head_groups": info[2], "splits": info[3],
            "split_rows": info[4] if info[3] > 1 else None, "wide_waves": info[5],
            "parities": info[6], "balanced": info[0] == 4 and info[3] > 1 and info[4] == 0}


def sparse_decode_attn_fp8(q: torch.Tensor, kv_fp8: torch.Tensor, kv_scale: torch.Tensor,
                           kv_indices: torch.Tensor, kv_indptr: torch.Tensor,
                           attn_sink: torch.Tensor, softmax_scale: float,
                           out: Optional[torch.Tensor] = None, *, max_len: int = 0,
                           split_rows: int = 0, mode: int = MODE_AUTO,
                           workspace: Optional[torch.Tensor] = None,
                           plain: bool = False) -> torch.Tensor:
    """out[N, H, D] (bf16): sparse decode attention over an FP8 pool whose row r
    is kv_scale[r] * e4m3(kv_fp8[r]) (uint8 codes or a float8_e4m3fn tensor);
    see include/spd.h.  plain=True calls ``sparse_decode_attn_fp8`` (automatic
    plan, no split); otherwise ``sparse_decode_attn_fp8_ex`` runs with
    (max_len, split_rows, mode), and a zero-filled workspace is allocated here
    when its plan needs one and none is given."""
    _check(q, "q", torch.bfloat16, 3)
    codes = _fp8_codes(kv_fp8, "kv_fp8")
    _check(kv_scale, "kv_scale", torch.float32, 1)
    _check(kv_indices, "kv_indices", torch.int32, 1)
    _check(kv_indptr, "kv_indptr", torch.int32, 1)
    _check(attn_sink, "attn_sink", torch.float32, 1)
    N, H, D = q.shape
    if codes.shape[1] != D or kv_scale.shape[0] != codes.shape[0] or \
            kv_indptr.shape[0] != N + 1 or attn_sink.shape[0] != H:
        raise ValueError("shape mismatch between q, kv_fp8, kv_scale, kv_indptr and attn_sink")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, 3)
        if tuple(out.shape) != (N, H, D):
            raise ValueError("out must be [N, H, D]")
    idx = kv_indices if kv_indices.numel() > 0 else kv_indptr  # any valid pointer; never read
    stream = _stream(q.device)
    if plain:
        st = lib.sparse_decode_attn_fp8(_ptr(q), _ptr(codes), _ptr(kv_scale), codes.shape[0],
                                        _ptr(idx), _ptr(kv_indptr), _ptr(attn_sink),
                                        float(softmax_scale), _ptr(out), N, H, D, stream)
        _raise_on(st, "sparse_decode_attn_fp8")
        return out
    need = sparse_decode_attn_fp8_workspace_size(N, H, D, max_len, split_rows, mode)
    if need > 0 and workspace is None:
        # zero-filled: a split-mode workspace's arrival counters must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.sparse_decode_attn_fp8_ex(_ptr(q), _ptr(codes), _ptr(kv_scale), codes.shape[0],
                                       _ptr(idx), _ptr(kv_indptr), _ptr(attn_sink),
                                       float(softmax_scale), _ptr(out), N, H, D, int(max_len),
                                       int(split_rows), int(mode), _ptr(workspace), ws_bytes,
                                       stream)
    _raise_on(st, "sparse_decode_attn_fp8_ex")
    return out


def quantize_kv_fp8(src: torch.Tensor, kv_fp8: torch.Tensor, kv_scale: torch.Tensor,
                    slots: Optional[torch.Tensor] = None) -> None:
    """Store bf16 rows src[n, D] into the FP8 pool (kv_fp8 [num_rows, D] codes,
    kv_scale [num_rows]) at rows slots[n] (0 .. n-1 when None), in place."""
    _check(src, "src", torch.bfloat16, 2)
    codes = _fp8_codes(kv_fp8, "kv_fp8")
    _check(kv_scale, "kv_scale", torch.float32, 1)
    n, D = src.shape
    if codes.shape[1] != D or kv_scale.shape[0] != codes.shape[0]:
        raise ValueError("shape mismatch between src, kv_fp8 and kv_scale")
    if slots is not None:
        _check(slots, "slots", torch.int32, 1)
        if slots.shape[0] != n:
            raise ValueError("slots must have one entry per source row")
    st = lib.quantize_kv_fp8(_ptr(src), _ptr(slots), n, D, _ptr(codes), _ptr(kv_scale),
                             codes.shape[0], _stream(src.device))
    _raise_on(st, "quantize_kv_fp8")


def fused_qk_norm_rope_swa_store(q: torch.Tensor, kv: torch.Tensor, q_weight: torch.Tensor,
                                 kv_weight: torch.Tensor, eps: float, positions: torch.Tensor,
                                 cos_sin: Optional[torch.Tensor], state_slot: torch.Tensor,
                                 win: int, unified_kv: Optional[torch.Tensor] = None,
                                 kv_fp8: Optional[torch.Tensor] = None,
                                 kv_scale: Optional[torch.Tensor] = None,
                                 q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The decode-step producer (see include/spd.h): returns q_out [N, H, D] (bf16,
    normed and rotated; pass q_out=q for in place) and stores each token's normed,
    rotated KV row into its window-ring slot of unified_kv and/or the FP8 pool."""
    _check(q, "q", torch.bfloat16, 3)
    _check(kv, "kv", torch.bfloat16, 2)
    _check(q_weight, "q_weight", torch.float32, 1)
    _check(kv_weight, "kv_weight", torch.float32, 1)
    _check(positions, "positions", torch.int32, 1)
    _check(state_slot, "state_slot", torch.int32, 1)
    N, H, D = q.shape
    max_pos, rope_dim = 0, 0
    if cos_sin is not None:
        _check(cos_sin, "cos_sin", torch.float32, 2)
        max_pos, rope_dim = cos_sin.shape
    if tuple(kv.shape) != (N, D) or q_weight.shape[0] != D or kv_weight.shape[0] != D or \
            positions.shape[0] != N or state_slot.shape[0] != N:
        raise ValueError("shape mismatch between q, kv, the weights, positions and state_slot")
    num_rows = None
    codes = None
    if unified_kv is not None:
        _check(unified_kv, "unified_kv", torch.bfloat16, 2)
        num_rows = unified_kv.shape[0]
    if kv_fp8 is not None:
        codes = _fp8_codes(kv_fp8, "kv_fp8")
        _check(kv_scale, "kv_scale", torch.float32, 1)
        if num_rows is not None and codes.shape[0] != num_rows:
            raise ValueError("the bf16 and FP8 pools must have the same rows")
        num_rows = codes.shape[0]
        if kv_scale.shape[0] != num_rows:
            raise ValueError("kv_scale must have one entry per pool row")
    if num_rows is None:
        raise ValueError("give unified_kv and/or kv_fp8 with kv_scale")
    for pool in (unified_kv, codes):
        if pool is not None and pool.shape[1] != D:
            raise ValueError("pool rows must have D entries")
    if q_out is None:
        q_out = torch.empty_like(q)
    else:
        _check(q_out, "q_out", torch.bfloat16, 3)
        if tuple(q_out.shape) != (N, H, D):
            raise ValueError("q_out must be [N, H, D]")
    st = lib.fused_qk_norm_rope_swa_store(
        _ptr(q), _ptr(q_out), _ptr(kv), _ptr(q_weight), _ptr(kv_weight), float(eps),
        _ptr(positions), _ptr(cos_sin), max_pos, rope_dim, _ptr(state_slot), int(win),
        _ptr(unified_kv), _ptr(codes), _ptr(kv_scale) if codes is not None else None, num_rows,
        N, H, D, _stream(q.device))
    _raise_on(st, "fused_qk_norm_rope_swa_store")
    return q_out


def validate_indices(kv_indices: torch.Tensor, kv_indptr: torch.Tensor, num_rows: int) -> int:
    """-1 when the attention preconditions hold, else the first offending position (syncs)."""
    _check(kv_indices, "kv_indices", torch.int32, 1)
    _check(kv_indptr, "kv_indptr", torch.int32, 1)
    first = ctypes.c_int64(0)
    st = lib.spd_validate_indices(_ptr(kv_indices), kv_indices.numel(), _ptr(kv_indptr),
                                  kv_indptr.shape[0] - 1, int(num_rows), ctypes.byref(first),
                                  _stream(kv_indptr.device))
    _raise_on(st, "spd_validate_indices")
    return int(first.value)

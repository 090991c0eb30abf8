"""fp64 CPU oracle for sparse decode attention and the decode index builder.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never calls it, and it shares no code, header, table or helper with the GPU
library.  The C source (``spd_oracle.c``) states the definition it computes and
the page passage each step follows (sglang PR #28392 summary, "key source
snippet": the ``paged_decode.py`` module docstring).

Arrays are numpy: bf16 data travels as its raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spd_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libspd_oracle.so")
# ASan + UBSan build (clang, the sanitizer runtime the HIP library's host code
# uses too, so both load into one process); SPD_ORACLE_LIB selects it
_SAN_PATH = os.path.join(_BUILD_DIR, "sanitize", "libspd_oracle.so")
_CLANG = "/opt/rocm/llvm/bin/clang"

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile the C oracle with gcc (generic x86-64, OpenMP).  Returns the path.

    sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build with
    clang instead (any finding aborts), for the sanitized CPU test run."""
    if sanitize:
        os.makedirs(os.path.dirname(_SAN_PATH), exist_ok=True)
        tmp = _SAN_PATH + ".tmp%d" % os.getpid()
        cmd = [_CLANG, "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-shared-libsan", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SAN_PATH)
        return _SAN_PATH
    env = os.environ.get("SPD_ORACLE_LIB")
    if env:
        return env
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.spd_oracle_sparse_decode_attn.argtypes = [P, P, i64, P, P, P, ctypes.c_float, i32, i32,
                                                      i32, P, i32, P]
        lib.spd_oracle_sparse_decode_attn.restype = ctypes.c_int
        lib.spd_oracle_build_decode_indices.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i32, P,
                                                        P, i64]
        lib.spd_oracle_build_decode_indices.restype = ctypes.c_int
        lib.spd_oracle_build_decode_indices_clamped.argtypes = \
            lib.spd_oracle_build_decode_indices.argtypes
        lib.spd_oracle_build_decode_indices_clamped.restype = ctypes.c_int
        lib.spd_oracle_sparse_decode_attn_fp8.argtypes = [P, P, P, i64, P, P, P, ctypes.c_float,
                                                          i32, i32, i32, P, i32, P]
        lib.spd_oracle_sparse_decode_attn_fp8.restype = ctypes.c_int
        lib.spd_oracle_quantize_fp8.argtypes = [P, i32, i32, P, P]
        lib.spd_oracle_quantize_fp8.restype = ctypes.c_int
        lib.spd_oracle_qk_norm_rope.argtypes = [P, P, P, P, ctypes.c_float, P, P, i32, i32, P, i32,
                                                i32, i32, i32, P, P, P]
        lib.spd_oracle_qk_norm_rope.restype = ctypes.c_int
        lib.spd_oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.spd_oracle_e4m3_value.restype = ctypes.c_double
        lib.spd_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.spd_oracle_set_threads.restype = None
        lib.spd_oracle_get_threads.argtypes = []
        lib.spd_oracle_get_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().spd_oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().spd_oracle_get_threads())


def sparse_decode_attn(q_bits: np.ndarray, kv_bits: np.ndarray, kv_indices: np.ndarray,
                       kv_indptr: np.ndarray, attn_sink: np.ndarray, softmax_scale: float,
                       tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 attention output ``[n, H, D]`` (n = N, or len(tokens) when given).

    q_bits ``[N, H, D]`` and kv_bits ``[P, D]`` are uint16 bf16 bit patterns,
    kv_indices / kv_indptr ``[N+1]`` int32, attn_sink ``[H]`` float32.
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    attn_sink = np.ascontiguousarray(attn_sink, dtype=np.float32)
    N, H, D = q_bits.shape
    assert kv_bits.ndim == 2 and kv_bits.shape[1] == D
    assert kv_indptr.shape == (N + 1,) and attn_sink.shape == (H,)
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n_out = N if tokens is None else len(tokens)
    out = np.zeros((n_out, H, D), dtype=np.float64)
    if kv_indices.size == 0:
        kv_indices = np.zeros(1, dtype=np.int32)  # never read: every slice is empty
    rc = _load().spd_oracle_sparse_decode_attn(
        _ptr(q_bits), _ptr(kv_bits), kv_bits.shape[0], _ptr(kv_indices), _ptr(kv_indptr),
        _ptr(attn_sink), float(np.float32(softmax_scale)), N, H, D, _ptr(tokens),
        0 if tokens is None else len(tokens), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected its input (code %d)" % rc)
    return out


def e4m3_value(code: int) -> float:
    """The OCP e4m3 value of an 8-bit code (NaN for 0x7f / 0xff)."""
    return float(_load().spd_oracle_e4m3_value(int(code)))


def quantize_fp8(src_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 store of bf16 rows ``[n, D]`` (uint16 bit patterns): returns the e4m3
    codes ``[n, D]`` uint8 and the per-row fp32 scales ``[n]`` (the steps are in
    the C source)."""
    src_bits = np.ascontiguousarray(src_bits, dtype=np.uint16)
    n, D = src_bits.shape
    codes = np.zeros((n, D), dtype=np.uint8)
    scales = np.zeros(n, dtype=np.float32)
    rc = _load().spd_oracle_quantize_fp8(_ptr(src_bits), n, D, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantiser rejected its input (code %d)" % rc)
    return codes, scales


def sparse_decode_attn_fp8(q_bits: np.ndarray, kv_codes: np.ndarray, kv_scale: np.ndarray,
                           kv_indices: np.ndarray, kv_indptr: np.ndarray, attn_sink: np.ndarray,
                           softmax_scale: float, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """sparse_decode_attn over an FP8 pool: row r is kv_scale[r] * e4m3(kv_codes[r])."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_codes = np.ascontiguousarray(kv_codes, dtype=np.uint8)
    kv_scale = np.ascontiguousarray(kv_scale, dtype=np.float32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    attn_sink = np.ascontiguousarray(attn_sink, dtype=np.float32)
    N, H, D = q_bits.shape
    assert kv_codes.ndim == 2 and kv_codes.shape[1] == D and kv_scale.shape == (kv_codes.shape[0],)
    assert kv_indptr.shape == (N + 1,) and attn_sink.shape == (H,)
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n_out = N if tokens is None else len(tokens)
    out = np.zeros((n_out, H, D), dtype=np.float64)
    if kv_indices.size == 0:
        kv_indices = np.zeros(1, dtype=np.int32)
    rc = _load().spd_oracle_sparse_decode_attn_fp8(
        _ptr(q_bits), _ptr(kv_codes), _ptr(kv_scale), kv_codes.shape[0], _ptr(kv_indices),
        _ptr(kv_indptr), _ptr(attn_sink), float(np.float32(softmax_scale)), N, H, D, _ptr(tokens),
        0 if tokens is None else len(tokens), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected its input (code %d)" % rc)
    return out


def qk_norm_rope(q_bits: np.ndarray, kv_bits: np.ndarray, q_weight: np.ndarray,
                 kv_weight: np.ndarray, eps: float, positions: np.ndarray, cos_sin: np.ndarray,
                 state_slot: np.ndarray, win: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The decode-step producer (steps in the C source): q [N, H, D] and kv [N, D] as
    bf16 bits, fp32 weights [D], positions [N], cos_sin [max_pos, rope_dim] fp32.
    Returns (q_out [N, H, D] fp64, kv_out [N, D] fp64, ring slot [N] int64; -1 and
    zero rows for a negative position, or one outside the table when rope_dim > 0)."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    q_weight = np.ascontiguousarray(q_weight, dtype=np.float32)
    kv_weight = np.ascontiguousarray(kv_weight, dtype=np.float32)
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    cos_sin = np.ascontiguousarray(cos_sin, dtype=np.float32)
    state_slot = np.ascontiguousarray(state_slot, dtype=np.int32)
    N, H, D = q_bits.shape
    max_pos, rope_dim = cos_sin.shape
    assert kv_bits.shape == (N, D) and q_weight.shape == (D,) and kv_weight.shape == (D,)
    assert positions.shape == (N,) and state_slot.shape == (N,)
    q_out = np.zeros((N, H, D), dtype=np.float64)
    kv_out = np.zeros((N, D), dtype=np.float64)
    slot = np.zeros(N, dtype=np.int64)
    if cos_sin.size == 0:
        cos_sin = np.zeros(1, dtype=np.float32)
    rc = _load().spd_oracle_qk_norm_rope(_ptr(q_bits), _ptr(kv_bits), _ptr(q_weight),
                                         _ptr(kv_weight), float(eps), _ptr(positions),
                                         _ptr(cos_sin), max_pos, rope_dim, _ptr(state_slot),
                                         int(win), N, H, D, _ptr(q_out), _ptr(kv_out), _ptr(slot))
    if rc != 0:
        raise ValueError("oracle rejected its input (code %d)" % rc)
    return q_out, kv_out, slot


def build_decode_indices(state_slot: np.ndarray, swa_len: np.ndarray,
                         comp_pos: Optional[np.ndarray], block_table: Optional[np.ndarray],
                         win: int, k_per_block: int, swa_pages: int,
                         clamp: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Ragged-packed ``(kv_indptr [N+1], kv_indices [kv_indptr[N]])``, both int32.

    comp_pos ``[N, topk]`` int32 (negative = no entry) or None; block_table
    ``[N, max_blocks]`` int32 (unused when comp_pos is None).  Input outside
    the builder's preconditions raises, unless clamp: then a ring length
    counts as its nearest bound in [0, win] and an entry whose block lies
    past the table counts as no entry (spd_oracle_build_decode_indices_clamped).
    """
    state_slot = np.ascontiguousarray(state_slot, dtype=np.int32)
    swa_len = np.ascontiguousarray(swa_len, dtype=np.int32)
    N = state_slot.shape[0]
    topk, max_blocks = 0, 0
    if comp_pos is not None:
        comp_pos = np.ascontiguousarray(comp_pos, dtype=np.int32)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        topk = comp_pos.shape[1]
        max_blocks = block_table.shape[1]
    capacity = N * (max(int(win), 0) + topk)
    indptr = np.zeros(N + 1, dtype=np.int32)
    indices = np.zeros(max(capacity, 1), dtype=np.int32)
    fn = (_load().spd_oracle_build_decode_indices_clamped if clamp
          else _load().spd_oracle_build_decode_indices)
    rc = fn(_ptr(state_slot), _ptr(swa_len), _ptr(comp_pos), topk, _ptr(block_table), max_blocks, N,
            int(win), int(k_per_block), int(swa_pages), _ptr(indptr), _ptr(indices), capacity)
    if rc != 0:
        raise ValueError("oracle builder rejected its input (code %d)" % rc)
    return indptr, indices[: indptr[-1]].copy()

"""Seeded synthetic inputs for sparse decode attention and the index builder.

Shared by the tests, the benchmark and the smoke check; imported by neither the
GPU library nor the oracle, and holding none of the method's arithmetic (no
slot mapping, no prefix sums of builder output, no attention math).  It only
draws random numbers and lays them out in the shapes the path consumes.

bf16 data is produced as raw ``uint16`` bit patterns: fp32 standard-normal draws
rounded to bf16 with round-to-nearest-even.

Every workload draws from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order: (1) index structure, (2) attn_sink, (3) q, (4) the pool, the pool in
chunks of ``_CHUNK`` values so that multi-GiB pools stream through memory.

Configurations (sizes from the benchmark definitions of this path):

  tiny         N=4, H=8, D=64, P=256; lengths [0, 1, 17, 64]; indices uniform on
               [0, P) with replacement; sink ~ N(0, 1); scale 1/8.
  decode_base  N=64, H=64, D=512, P=65536; window win=128 with state_slot[t]=t
               and a full ring (swa_len=128), so swa_pages = 8192; 512
               compressed slots per token drawn without replacement from
               [swa_pages, P), expressed as builder input with K_PER_BLOCK=1,
               block_table[t][c] = slot_c - swa_pages and comp_pos = 0..511;
               sink ~ N(0, 1); scale 1/sqrt(512).
  ragged       N=256, H=64, D=512, P=1,048,576; tokens 0..191 have length
               uniform on {1..2048}; tokens 192..255 are padding (length 0);
               indices uniform on [0, P) with replacement; sink ~ N(0, 1);
               scale 1/sqrt(512); capacity bound max_len = 2048.
  large        N=1024, H=128, D=512, P=4,194,304; win=128, state_slot[t]=t,
               swa_len=128, swa_pages=131072; K_PER_BLOCK=64 with 63488
               compressed blocks; per token 8 distinct random block ids and
               comp_pos = 0..511; sink ~ N(0, std 2); scale 1/sqrt(512).
  prefill      N=8192, H=64, D=512, P=1,048,576; lengths uniform on {1..640};
               sliding reuse: one stream of uniform indices on [0, P); token t
               takes stream[a_t : a_t + L_t] with a_0 = 0 and
               a_{t+1} = a_t + ceil(L_t / 10); sink ~ N(0, 1); scale 1/sqrt(512).
               meta holds the stream and each token's window (a_t, L_t).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_CHUNK = 1 << 24

SEEDS = {"tiny": 0, "decode_base": 1, "ragged": 2, "large": 3, "prefill": 4, "long_context": 5}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """Standard-normal (times std) fp32 draws, rounded to bf16 bits, generated in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = bf16_bits(x)
    return out.reshape(shape)


@dataclass
class BuilderInputs:
    """Inputs of the decode index builder (window ring slots + compressed slots)."""
    state_slot: np.ndarray      # [N] int32
    swa_len: np.ndarray         # [N] int32, in [0, win]
    comp_pos: Optional[np.ndarray]    # [N, topk] int32, negative = no entry
    block_table: Optional[np.ndarray]  # [N, max_blocks] int32
    win: int
    k_per_block: int
    swa_pages: int

    @property
    def topk(self) -> int:
        return 0 if self.comp_pos is None else int(self.comp_pos.shape[1])

    @property
    def capacity(self) -> int:
        return int(self.state_slot.shape[0]) * (self.win + self.topk)


@dataclass
class Workload:
    name: str
    N: int
    H: int
    D: int
    P: int
    q_bits: object              # [N, H, D] uint16 array (host mode) or bf16 tensor (device mode)
    kv_bits: object             # [P, D] likewise
    attn_sink: np.ndarray       # [H] float32
    softmax_scale: float        # an fp32 value
    max_len: int                # capacity bound on every token's slice length
    kv_indices: Optional[np.ndarray] = None   # ragged CSR given directly
    kv_indptr: Optional[np.ndarray] = None
    builder: Optional[BuilderInputs] = None   # or: built from these inputs
    meta: Dict[str, object] = field(default_factory=dict)


# Where q and the pool are generated: "host" (numpy, uint16 bit arrays) or
# "device" (torch on a GPU: Philox normal draws rounded to bf16 by torch, for
# multi-GiB pools that would take a minute on the host).  Index structure and
# sinks always come from the numpy generator.
_DATA_MODE = {"mode": "host", "device": None}


def set_data_mode(mode: str, device=None) -> None:
    assert mode in ("host", "device")
    _DATA_MODE["mode"] = mode
    _DATA_MODE["device"] = device


def device_normal_bf16(shape, seed: int, device, std: float = 1.0):
    """bf16 torch tensor of N(0, std) draws from a seeded device generator, in chunks."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 26
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        x = torch.randn(e - s, dtype=torch.float32, device=device, generator=gen)
        if std != 1.0:
            x.mul_(std)
        flat[s:e] = x.to(torch.bfloat16)
    return out


def _finish(name, rng, N, H, D, P, sink_std, scale, max_len, **kw) -> Workload:
    sink = (rng.standard_normal(H) * sink_std).astype(np.float32)
    if _DATA_MODE["mode"] == "device":
        base = int(rng.integers(0, 2 ** 62))
        q = device_normal_bf16((N, H, D), base, _DATA_MODE["device"])
        kv = device_normal_bf16((P, D), base + 1, _DATA_MODE["device"])
    else:
        q = normal_bf16(rng, (N, H, D))
        kv = normal_bf16(rng, (P, D))
    return Workload(name=name, N=N, H=H, D=D, P=P, q_bits=q, kv_bits=kv, attn_sink=sink,
                    softmax_scale=float(np.float32(scale)), max_len=max_len, **kw)


def host_bits(x) -> np.ndarray:
    """uint16 bf16 bit patterns on the host, from a numpy array or a bf16 torch tensor."""
    if isinstance(x, np.ndarray):
        return x
    return x.contiguous().view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


def device_bits(x, device):
    """bf16 torch tensor on `device`, from uint16 bit patterns or a bf16 torch tensor."""
    import torch
    if isinstance(x, np.ndarray):
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return x.to(device)


def csr_from_lists(lists) -> tuple:
    """Pack per-token index lists into (kv_indices, kv_indptr) int32 -- input layout only."""
    lens = np.array([len(x) for x in lists], dtype=np.int64)
    indptr = np.zeros(len(lists) + 1, dtype=np.int64)
    np.cumsum(lens, out=indptr[1:])
    idx = np.concatenate([np.asarray(x, dtype=np.int64) for x in lists]) if len(lists) else np.zeros(0)
    return idx.astype(np.int32), indptr.astype(np.int32)


def random_csr(name: str, seed: int, N: int, H: int, D: int, P: int, lengths, *,
               sink_std: float = 1.0, scale: Optional[float] = None, replace: bool = True,
               max_len: Optional[int] = None) -> Workload:
    """Generic ragged workload: token t draws lengths[t] indices uniform on [0, P)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = [int(x) for x in lengths]
    lists = []
    for L in lengths:
        if replace:
            lists.append(rng.integers(0, P, size=L))
        else:
            lists.append(rng.choice(P, size=L, replace=False))
    idx, indptr = csr_from_lists(lists)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ml = max_len if max_len is not None else max([0] + lengths)
    return _finish(name, rng, N, H, D, P, sink_std, scale, ml, kv_indices=idx, kv_indptr=indptr)


def tiny(seed: int = SEEDS["tiny"]) -> Workload:
    return random_csr("tiny", seed, 4, 8, 64, 256, [0, 1, 17, 64], scale=1.0 / 8.0, max_len=64)


def window_plus_compressed(name: str, seed: int, N: int, H: int, D: int, P: int, win: int,
                           topk: int, k_per_block: int, n_blocks_per_token: Optional[int] = None,
                           sink_std: float = 1.0) -> Workload:
    """Builder-shaped workload: a full window ring per token (state_slot[t] = t)
    plus topk compressed positions.  K_PER_BLOCK == 1: topk distinct compressed
    slots per token, without replacement.  K_PER_BLOCK > 1: n_blocks_per_token
    distinct random block ids per token and comp_pos = 0..topk-1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    swa_pages = N * win
    assert swa_pages < P
    comp_rows = P - swa_pages
    state_slot = np.arange(N, dtype=np.int32)
    swa_len = np.full(N, win, dtype=np.int32)
    comp_pos = np.tile(np.arange(topk, dtype=np.int32), (N, 1))
    if k_per_block == 1:
        block_table = np.stack([rng.choice(comp_rows, size=topk, replace=False) for _ in range(N)])
    else:
        n_blocks = comp_rows // k_per_block
        nb = n_blocks_per_token or -(-topk // k_per_block)
        block_table = np.stack([rng.choice(n_blocks, size=nb, replace=False) for _ in range(N)])
    b = BuilderInputs(state_slot=state_slot, swa_len=swa_len, comp_pos=comp_pos,
                      block_table=np.ascontiguousarray(block_table, dtype=np.int32), win=win,
                      k_per_block=k_per_block, swa_pages=swa_pages)
    return _finish(name, rng, N, H, D, P, sink_std, 1.0 / math.sqrt(D), win + topk, builder=b)


def decode_base(seed: int = SEEDS["decode_base"]) -> Workload:
    return window_plus_compressed("decode_base", seed, 64, 64, 512, 65536, 128, 512, 1)


def large(seed: int = SEEDS["large"]) -> Workload:
    return window_plus_compressed("large", seed, 1024, 128, 512, 4194304, 128, 512, 64,
                                  n_blocks_per_token=8, sink_std=2.0)


def ragged_lengths(rng: np.random.Generator, N: int, max_len: int, n_pad: int) -> np.ndarray:
    L = rng.integers(1, max_len + 1, size=N)
    if n_pad:
        L[N - n_pad:] = 0
    return L


def ragged(seed: int = SEEDS["ragged"], N: int = 256, H: int = 64, D: int = 512,
           P: int = 1048576, max_len: int = 2048, pad_frac: float = 0.25) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    n_pad = int(round(N * pad_frac))
    L = ragged_lengths(rng, N, max_len, n_pad)
    lists = [rng.integers(0, P, size=int(x)) for x in L]
    idx, indptr = csr_from_lists(lists)
    w = _finish("ragged", rng, N, H, D, P, 1.0, 1.0 / math.sqrt(D), max_len, kv_indices=idx,
                kv_indptr=indptr)
    w.meta["n_pad"] = n_pad
    return w


def prefill(seed: int = SEEDS["prefill"], N: int = 8192, H: int = 64, D: int = 512,
            P: int = 1048576, max_len: int = 640) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    L = rng.integers(1, max_len + 1, size=N)
    starts = np.zeros(N, dtype=np.int64)
    for t in range(1, N):
        starts[t] = starts[t - 1] + (int(L[t - 1]) + 9) // 10
    stream = rng.integers(0, P, size=int((starts + L).max()))  # every window lies inside it
    lists = [stream[starts[t]: starts[t] + L[t]] for t in range(N)]
    idx, indptr = csr_from_lists(lists)
    w = _finish("prefill", rng, N, H, D, P, 1.0, 1.0 / math.sqrt(D), max_len, kv_indices=idx,
                kv_indptr=indptr)
    # the same lists as windows of the one stream they were cut from
    w.meta.update(stream=stream.astype(np.int32), win_start=starts.astype(np.int32),
                  win_len=L.astype(np.int32))
    return w


def long_context(seed: int = SEEDS["long_context"], N: int = 8, H: int = 64, D: int = 512,
                 P: int = 1048576, length: int = 8192) -> Workload:
    """A small batch of long slices (the case that splits a slice across
    workgroups): N tokens of `length` rows each, rows uniform in [0, P),
    q, kv ~ N(0, 1), sinks ~ N(0, 1).  Not one of the pages' batches: a
    measurement case for the split plan, beside the ragged batch's lengths."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lists = [rng.integers(0, P, size=length) for _ in range(N)]
    idx, indptr = csr_from_lists(lists)
    return _finish("long_context", rng, N, H, D, P, 1.0, 1.0 / math.sqrt(D), length,
                   kv_indices=idx, kv_indptr=indptr)


CONFIGS = {"tiny": tiny, "decode_base": decode_base, "ragged": ragged, "large": large,
           "prefill": prefill, "long_context": long_context}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)

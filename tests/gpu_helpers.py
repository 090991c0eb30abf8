"""Shared helpers of the GPU parity tests: move workloads to the device, run the
HIP path through the binding, evaluate the oracle on all or on sampled tokens,
and compare with the acceptance bound |gpu - ref| <= 1e-2 + 1e-2 |ref|."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W

ATOL = 1e-2
RTOL = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def device_inputs(w: W.Workload):
    d = dev()
    q = W.device_bits(w.q_bits, d)
    kv = W.device_bits(w.kv_bits, d)
    sink = torch.from_numpy(w.attn_sink).to(d)
    return q, kv, sink


def device_csr(indices: np.ndarray, indptr: np.ndarray):
    d = dev()
    idx = torch.from_numpy(np.ascontiguousarray(indices, dtype=np.int32)).to(d)
    ptr = torch.from_numpy(np.ascontiguousarray(indptr, dtype=np.int32)).to(d)
    return idx, ptr


def device_builder_inputs(b: W.BuilderInputs):
    d = dev()
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(d)
    return t(b.state_slot), t(b.swa_len), t(b.comp_pos), t(b.block_table)


def oracle_tokens(w: W.Workload, indices: np.ndarray, indptr: np.ndarray, tokens=None,
                  sink=None) -> np.ndarray:
    """Oracle output for `tokens` (all when None), on a compact copy of just the
    pool rows those tokens read (the oracle's result does not depend on the
    numbering of pool rows)."""
    N = w.N
    if tokens is None:
        tokens = np.arange(N)
    tokens = np.asarray(tokens, dtype=np.int64)
    sl = [indices[indptr[t]:indptr[t + 1]] for t in tokens]
    allidx = np.concatenate(sl) if sl else np.zeros(0, dtype=np.int32)
    uniq, inv = np.unique(allidx, return_inverse=True)
    if isinstance(w.kv_bits, np.ndarray):
        rows = w.kv_bits[uniq] if len(uniq) else np.zeros((1, w.D), dtype=np.uint16)
    else:
        u = torch.from_numpy(uniq.astype(np.int64)).to(w.kv_bits.device)
        rows = W.host_bits(w.kv_bits[u]) if len(uniq) else np.zeros((1, w.D), dtype=np.uint16)
    lens = np.array([len(x) for x in sl], dtype=np.int64)
    sub_ptr = np.zeros(len(tokens) + 1, dtype=np.int32)
    sub_ptr[1:] = np.cumsum(lens)
    qb = W.host_bits(w.q_bits[torch.from_numpy(tokens).to(w.q_bits.device)]) \
        if not isinstance(w.q_bits, np.ndarray) else w.q_bits[tokens]
    s = w.attn_sink if sink is None else sink
    return oracle.sparse_decode_attn(qb, rows, inv.astype(np.int32), sub_ptr, s, w.softmax_scale)


def bf16_to_f64(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d outside |d| <= 1e-2 + 1e-2|ref|; worst at %s: gpu=%r ref=%r"
                             % (what, int(bad.sum()), bad.size, i, gpu[i], ref[i]))
    log("  %s: max|err| %.3g, max err/bound %.3f" % (what, err.max() if err.size else 0.0,
                                                     (err / bound).max() if err.size else 0.0))


def random_builder_inputs(seed, N, win, topk, k, max_blocks, n_blocks) -> W.BuilderInputs:
    """Builder inputs with every kind of token: random window lengths (some 0,
    some full), sentinel entries, all-sentinel rows and padded tokens; valid
    comp_pos entries lie in [0, max_blocks * k), block ids in [0, n_blocks)."""
    rng = np.random.default_rng(seed)
    state_slot = rng.permutation(N + 5)[:N].astype(np.int32)
    swa_len = rng.integers(0, win + 1, size=N).astype(np.int32)
    swa_len[rng.random(N) < 0.15] = 0
    swa_len[rng.random(N) < 0.15] = win
    comp_pos = rng.integers(0, max_blocks * k, size=(N, topk)).astype(np.int32)
    comp_pos[rng.random((N, topk)) < 0.3] = -1
    comp_pos[rng.random(N) < 0.1] = -1                  # all-sentinel rows
    block_table = rng.integers(0, n_blocks, size=(N, max_blocks)).astype(np.int32)
    pad = rng.random(N) < 0.1                          # padded tokens: nothing at all
    swa_len[pad] = 0
    comp_pos[pad] = -1
    return W.BuilderInputs(state_slot, swa_len, comp_pos, block_table, win, k, (N + 5) * win)

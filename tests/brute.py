"""Brute-force restatements used to pin the oracle on tiny inputs.

These are written independently of ``oracle/spd_oracle.c`` and in a different
shape, so that a slip in one is unlikely to be repeated in the other:

* attention: for each (token, head) build the full logit list
  ``[s_1, ..., s_L, sink]``, take an ordinary softmax over it with exactly
  rounded sums (``math.fsum``), and drop the sink's column -- the reading of the
  sink as a virtual key in the softmax denominator (sglang PR #28392 summary,
  "key source snippet": the paged_decode.py module docstring);
* index builder: membership, not construction -- a pool slot p belongs to token
  t's window part iff it lies below swa_pages, p // win == state_slot[t] and
  p % win < swa_len[t]; it belongs to the compressed part once for every
  non-negative comp_pos entry c whose block-table lookup lands on p.
"""
from __future__ import annotations

import math
import struct

import numpy as np


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def attention(q_bits, kv_bits, kv_indices, kv_indptr, attn_sink, softmax_scale):
    N, H, D = q_bits.shape
    sigma = float(np.float32(softmax_scale))
    out = np.zeros((N, H, D), dtype=np.float64)
    for t in range(N):
        sl = [int(x) for x in kv_indices[int(kv_indptr[t]):int(kv_indptr[t + 1])]]
        if not sl:
            continue
        rows = [[bf16_value(kv_bits[r, d]) for d in range(D)] for r in sl]
        for h in range(H):
            qv = [bf16_value(q_bits[t, h, d]) for d in range(D)]
            logits = [sigma * math.fsum(a * b for a, b in zip(qv, row)) for row in rows]
            logits.append(float(attn_sink[h]))
            top = max(logits)
            e = [math.exp(x - top) for x in logits]
            z = math.fsum(e)
            probs = [x / z for x in e[:-1]]  # drop the sink column
            for d in range(D):
                out[t, h, d] = math.fsum(p * row[d] for p, row in zip(probs, rows))
    return out


def builder_membership(state_slot, swa_len, comp_pos, block_table, win, k_per_block, swa_pages,
                       pool_rows):
    """Per token, the sorted multiset of pool slots it must attend to (brute force over the pool)."""
    N = len(state_slot)
    result = []
    for t in range(N):
        slots = []
        for p in range(pool_rows):
            if p < swa_pages and p // win == state_slot[t] and p % win < swa_len[t]:
                slots.append(p)
            if p >= swa_pages and comp_pos is not None:
                for c in comp_pos[t]:
                    c = int(c)
                    if c < 0:
                        continue
                    b = int(block_table[t][c // k_per_block])
                    if (p - swa_pages) // k_per_block == b and (p - swa_pages) % k_per_block == c % k_per_block:
                        slots.append(p)
        result.append(sorted(slots))
    return result

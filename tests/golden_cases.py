"""Load the hand-worked fixtures under tests/golden/ (each file states the
passage it follows and the derivation of every expected value)."""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(v) -> float:
    if isinstance(v, (int, float)):
        return float(v)
    v = v.strip()
    if v == "-inf":
        return -math.inf
    if v.startswith("ln "):
        return math.log(float(v[3:]))
    return float(Fraction(v))


def attention_cases():
    with open(os.path.join(HERE, "attention_worked_examples.json")) as f:
        doc = json.load(f)
    out = []
    for c in doc["cases"]:
        out.append(dict(
            name=c["name"], H=c["H"], D=c["D"],
            q=np.array(c["q"], dtype=np.float32),
            kv=np.array(c["kv"], dtype=np.float32),
            kv_indices=np.array(c["kv_indices"], dtype=np.int32),
            kv_indptr=np.array(c["kv_indptr"], dtype=np.int32),
            attn_sink=np.array([_num(x) for x in c["attn_sink"]], dtype=np.float32),
            softmax_scale=_num(c["softmax_scale"]),
            out=np.vectorize(_num)(np.array(c["out"], dtype=object)).astype(np.float64)))
    return out


def builder_case(name: str = "builder_worked_example.json"):
    with open(os.path.join(HERE, name)) as f:
        c = json.load(f)
    a = lambda k: np.array(c[k], dtype=np.int32)
    return dict(win=c["win"], k_per_block=c["k_per_block"], swa_pages=c["swa_pages"],
                state_slot=a("state_slot"), swa_len=a("swa_len"), comp_pos=a("comp_pos"),
                block_table=a("block_table"), kv_indptr=a("kv_indptr"), kv_indices=a("kv_indices"))

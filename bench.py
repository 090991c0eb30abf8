"""Benchmark: one step = the whole hot path on one batch of synthetic input --
build_decode_indices (window ring + compressed slots -> ragged CSR) followed by
sparse_decode_attn -- on the decode_base configuration (N=64 tokens, H=64,
D=512, 640 pool rows per token, 64 MiB pool), through the C ABI.

Inputs are resident in HBM before timing starts.  R rotating input sets
(separate pool, queries, builder inputs, outputs) keep the touched footprint
above twice the 256 MB Infinity Cache, so steps are fed from HBM.  Each step
is a HIP graph (captured once per set) replayed from the host.

Prints one JSON line: tokens/s (whole job), gathered KV GB/s, the roofline
record of the attention call, and the oracle timed on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse decode attn tokens/s + gathered KV GB/s (% of MI355X HBM roofline)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--sets", type=int, default=16)
    p.add_argument("--eager", action="store_true", help="launch kernels directly instead of graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def algorithmic_bytes(indptr: np.ndarray, N: int, H: int, D: int) -> dict:
    L = np.diff(indptr.astype(np.int64))
    sum_l = int(L.sum())
    nonempty = int((L > 0).sum())
    kv = sum_l * D * 2
    total = kv + nonempty * H * D * 2 + N * H * D * 2 + 4 * sum_l + 4 * (N + 1) + 4 * H
    return {"sum_L": sum_l, "kv_bytes": kv, "B_alg": total}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; --gpus %d is not supported (the path would "
              "shard by tokens with no exchange step)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_paged_decode_ragged_amd as spd
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.decode_base()
    b = w.builder
    N, H, D = w.N, w.H, w.D
    max_len = w.max_len
    cap = b.capacity
    ws_bytes = spd.sparse_decode_attn_workspace_size(N, H, D, max_len, 0)

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    q0 = W.device_bits(w.q_bits, dev)
    kv0 = W.device_bits(w.kv_bits, dev)
    sets = []
    for r in range(args.sets):
        s = dict(q=q0.clone(), kv=kv0.clone(), sink=torch.from_numpy(w.attn_sink).to(dev),
                 ss=t(b.state_slot), sl=t(b.swa_len), cp=t(b.comp_pos), bt=t(b.block_table),
                 ptr=torch.zeros(N + 1, dtype=torch.int32, device=dev),
                 idx=torch.zeros(cap, dtype=torch.int32, device=dev),
                 out=torch.empty((N, H, D), dtype=torch.bfloat16, device=dev),
                 ws=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev))
        sets.append(s)
    del q0, kv0

    def build(s):
        spd.build_decode_indices(s["ss"], s["sl"], s["cp"], s["bt"], b.win, b.k_per_block,
                                 b.swa_pages, kv_indptr=s["ptr"], kv_indices=s["idx"])

    def attn(s):
        spd.sparse_decode_attn(s["q"], s["kv"], s["idx"], s["ptr"], s["sink"], w.softmax_scale,
                               out=s["out"], max_len=max_len, workspace=s["ws"])

    def step(s):
        build(s)
        attn(s)

    # eager warm-up, then one graph per set (full step) and one per set (attention only)
    for s in sets:
        step(s)
    torch.cuda.synchronize()
    step_graphs, attn_graphs = [], []
    if not args.eager:
        cs = torch.cuda.Stream()
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                step(s)
            step_graphs.append(g)
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2, stream=cs):
                attn(s)
            attn_graphs.append(g2)
        torch.cuda.synchronize()

    def run_steps(k, graphs, fn):
        for i in range(k):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                fn(sets[i % len(sets)])

    run_steps(args.warmup, step_graphs, step)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(args.steps, step_graphs, step)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps

    # attention call alone (the dominant kernel), same rotation, for the roofline
    run_steps(min(args.warmup, 64), attn_graphs, attn)
    torch.cuda.synchronize()
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    n_attn = max(args.steps, 100)
    a0.record()
    run_steps(n_attn, attn_graphs, attn)
    a1.record()
    torch.cuda.synchronize()
    us_attn = a0.elapsed_time(a1) * 1e3 / n_attn

    indptr = sets[0]["ptr"].cpu().numpy()
    ab = algorithmic_bytes(indptr, N, H, D)
    tokens_per_s = N / (ms_per_step * 1e-3)
    gathered_gbps = ab["kv_bytes"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["B_alg"] / (us_attn * 1e-6) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_base", "N": N, "H": H, "D": D, "pool_rows": w.P,
                   "indices_per_token": max_len, "window": b.win, "compressed_per_token": b.topk,
                   "split_plan": "auto(max_len=%d)" % max_len, "rotating_sets": args.sets,
                   "launch": "eager" if args.eager else "hip_graph_per_step",
                   "step": "build_decode_indices + sparse_decode_attn"},
        "gathered_kv_GBps": round(gathered_gbps, 1),
        "gathered_kv_frac_of_hbm_peak": round(gathered_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "sparse_decode_attn call (attn_main + attn_combine)",
                     "us_per_call": round(us_attn, 3), "bytes_per_call": ab["B_alg"]},
    }

    if not args.no_cpu_baseline:
        import oracle
        oracle.set_threads(os.cpu_count() or 1)
        optr, oidx = oracle.build_decode_indices(b.state_slot, b.swa_len, b.comp_pos,
                                                 b.block_table, b.win, b.k_per_block, b.swa_pages)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.sparse_decode_attn(w.q_bits, w.kv_bits, oidx, optr, w.attn_sink, w.softmax_scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        rec["cpu_baseline"] = {"value": round(N * reps / el, 2), "unit": "tokens/s",
                               "cores": oracle.get_threads(), "kind": "oracle",
                               "sample": "full decode_base batch (64 tokens, attention only, fp64 "
                                         "two-pass) repeated %d times, %.1f s" % (reps, el)}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

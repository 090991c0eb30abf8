"""Benchmark of the hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
build_decode_indices (window ring + compressed slots -> ragged CSR) followed by
sparse_decode_attn, through the C ABI.  The default workload is decode_base
(N=64 tokens, H=64, D=512, 640 pool rows per token: 128 window + 512
compressed, 64 MiB pool), the configuration the metric is quoted on.  Other
workloads (--workload) are for exploration; those given as ready CSR indices
(ragged, prefill) have no builder step.

Inputs are resident in HBM before timing starts.  R rotating input sets
(separate pool, queries, builder inputs, outputs) keep the touched footprint
above twice the 256 MB Infinity Cache, so steps are fed from HBM.  The timed
loops replay one HIP graph that holds one step per set back to back (single-step
graphs cover a remainder), timed with HIP events on the replay stream.

Prints one JSON line: tokens/s for the whole job, gathered KV GB/s, the
roofline record of the attention kernel, and the oracle timed on this host's
cores on a bounded sample.  Two variants of the attention call are timed the
same way and reported beside it: the page transform fused into the kernel
(sparse_decode_attn_paged) and the call over an FP8 pool filled from the same
bf16 rows by the quantising store (sparse_decode_attn_fp8).  For builder-shaped
workloads the decode-step producer that writes the window rows
(fused_qk_norm_rope_swa_store) is timed too.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA peak of the MI355X
METRIC = "sparse decode attn tokens/s + gathered KV GB/s (% of MI355X HBM roofline)"
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="decode_base",
                   choices=["decode_base", "tiny", "ragged", "large", "prefill", "long_context"])
    p.add_argument("--long-tokens", type=int, default=8, help="long_context: tokens")
    p.add_argument("--long-rows", type=int, default=8192, help="long_context: rows per token")
    p.add_argument("--mode", default="auto", choices=["auto", "heads", "rows", "wide", "split"])
    p.add_argument("--split-rows", type=int, default=0)
    p.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = automatic)")
    p.add_argument("--eager", action="store_true", help="launch kernels directly, no graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8-pool measurement")
    p.add_argument("--no-producer", action="store_true", help="skip the producer measurement")
    p.add_argument("--no-prefill", action="store_true", help="skip the shared-window measurement")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-floor", action="store_true",
                   help="skip the floor legs (gather without arithmetic, empty launch, output "
                        "store, device copy)")
    p.add_argument("--calibration-copy-mib", type=int, default=0,
                   help="also run a kernel of known traffic three times (bitwise_not over this "
                        "many MiB of int32: reads and writes exactly that much), which scales "
                        "the HBM byte counters")
    p.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                   help="summarise rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE "
                        "runs of this script) instead of benchmarking")
    p.add_argument("--pmc-copy-mib", type=int, default=0,
                   help="size of the calibration copy in the runs given to --pmc-summary")
    return p.parse_args()


def kernel_sources(kernel: str) -> tuple:
    """The source files an attention kernel is built from."""
    if "split" in kernel:
        return ("attn_split.hip", "fp8_device.h", "attn_device.h", "spd_internal.h")
    if "fp8" in kernel:
        return ("attn_fp8.hip", "fp8_device.h", "attn_device.h", "spd_internal.h")
    return ("attn.hip", "attn_device.h", "spd_internal.h")


def kernel_sources_digest(kernel: str) -> str:
    """sha256 over the kernel's sources: a traffic figure taken from counters is
    only reported while these are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_paged_decode_ragged_amd", "csrc")
    for name in kernel_sources(kernel):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]




def fp8_kernel(plan: dict, D: int) -> str:
    """The kernel sparse_decode_attn_fp8_ex launches for a plan of
    sparse_decode_attn_fp8_plan_info: the split kernel over codes, workgroups
    of 32 W heads on 32-head waves (W = 3: 64 heads on four waves, two
    parities), or the 16-head rows kernel."""
    if plan["mode"] == "split":
        return "attn_split_kernel<%d,%d,%d,true>" % (D, plan["heads_per_group"] // 32,
                                                      plan["parities"])
    w = plan["wide_waves"]
    if w == 3:
        return "attn_wide_fp8_kernel<%d,4,2>" % D
    if w:
        return "attn_wide_fp8_kernel<%d,%d>" % (D, w)
    return "attn_rows_fp8_kernel<%d>" % D


def recorded_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes of `kernel` from the committed counter summary
    profiles/hbm_traffic_<workload>.md, or None when there is none or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if (fields.get("kernel") != kernel or fields.get("workload") != workload
            or fields.get("source_digest") != kernel_sources_digest(kernel)):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pmc_summary(dirs, copy_mib):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from rocprofv3
    counter CSVs, and the factors that scale each counter to bytes: what it reads
    for the calibration kernel of the same run (copy_mib MiB read and written)."""
    import csv
    import glob
    import statistics
    per = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = (r["Kernel_Name"], r["Counter_Name"])
                    per.setdefault(key, []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    out = {}
    for (name, counter), vals in per.items():
        if "bitwise_not" in name:  # the calibration kernel (see --calibration-copy-mib)
            name = "__copy_calibration__"
        out.setdefault(name, {})[counter] = (statistics.mean(v[1] for v in vals), len(vals))
    cal = out.get("__copy_calibration__", {})
    factors = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        if copy_mib and counter in cal:
            factors[counter] = copy_mib * 1024.0 / cal[counter][0]
    return out, factors


def algorithmic_bytes(indptr: np.ndarray, N: int, H: int, D: int) -> dict:
    """Bytes the method must move per call: gathered KV rows, q of non-empty
    tokens, the output, the index list, indptr and the sinks."""
    L = np.diff(indptr.astype(np.int64))
    sum_l = int(L.sum())
    nonempty = int((L > 0).sum())
    kv = sum_l * D * 2
    qo = nonempty * H * D * 2 + N * H * D * 2
    total = kv + qo + 4 * sum_l + 4 * (N + 1) + 4 * H
    return {"sum_L": sum_l, "kv_bytes": kv, "qo_bytes": qo, "B_alg": total, "nonempty": nonempty}


def mfma_flops(sum_l: int, H: int, D: int) -> int:
    """MFMA work the method must do per call: S = q K^T and O = P V, each
    2 H D flop per gathered row (multiply and add)."""
    return 4 * H * D * sum_l


def covered_positions(stream_len: int, start: np.ndarray, length: np.ndarray) -> int:
    """Stream positions that at least one window [start, start + length) covers,
    counting only the windows the shared-window call reads (length > 0, inside
    the stream; any other window is empty): that call reads each of them once."""
    start = np.asarray(start, dtype=np.int64)
    end = start + np.asarray(length, dtype=np.int64)
    ok = (start >= 0) & (end > start) & (end <= stream_len)
    cover = np.zeros(stream_len + 1, dtype=np.int64)
    np.add.at(cover, start[ok], 1)
    np.add.at(cover, end[ok], -1)
    return int((np.cumsum(cover)[:-1] > 0).sum())


def cpu_baseline(w, indptr, indices, seconds):
    """The oracle as it stands, on this host's cores, on a bounded token sample."""
    import oracle
    import workloads as W
    import torch
    oracle.set_threads(os.cpu_count() or 1)
    N = w.N
    L = np.diff(indptr.astype(np.int64))
    order = np.random.default_rng(0).permutation(N)

    def run(tokens):
        tokens = np.sort(tokens)
        sl = [indices[indptr[t]:indptr[t + 1]] for t in tokens]
        allidx = np.concatenate(sl) if sl else np.zeros(0, dtype=np.int32)
        uniq, inv = np.unique(allidx, return_inverse=True)
        if isinstance(w.kv_bits, np.ndarray):
            rows = w.kv_bits[uniq]
            qb = w.q_bits[tokens]
        else:
            rows = W.host_bits(w.kv_bits[torch.from_numpy(uniq.astype(np.int64)).to(w.kv_bits.device)])
            qb = W.host_bits(w.q_bits[torch.from_numpy(tokens).to(w.q_bits.device)])
        sub = np.zeros(len(tokens) + 1, dtype=np.int32)
        sub[1:] = np.cumsum([len(x) for x in sl])
        t0 = time.perf_counter()
        oracle.sparse_decode_attn(qb, rows, inv.astype(np.int32), sub, w.attn_sink, w.softmax_scale)
        return time.perf_counter() - t0

    def median_rate(threads, budget):
        """Median tokens/s of three timed passes on `threads` threads, each
        pass about budget / 3 seconds: a sample of tokens (the whole batch
        when it is quick), repeated k times, after one untimed pass."""
        oracle.set_threads(threads)
        probe = order[: min(N, 8)]
        run(probe)  # warm-up
        dt = max(run(probe), 1e-4)
        per = (budget / 3) / dt * len(probe)  # tokens one pass can take
        n = int(min(N, max(len(probe), per)))
        sample = order[:n]
        k = max(1, int(round(per / n)))
        rates, el = [], 0.0
        for _ in range(3):
            d = sum(run(sample) for _ in range(k))
            el += d
            rates.append(k * n / d)
        return float(np.median(rates)), rates, n, k, int(L[sample].sum()), el

    def describe(n, k, rows, el, threads):
        return ("3 passes, each %d x %d of %d tokens (%d pool rows gathered), %.1f s on %d "
                "thread%s" % (k, n, N, rows, el, threads, "" if threads == 1 else "s"))

    all_cores = os.cpu_count() or 1
    v, rates, n, k, rows, el = median_rate(all_cores, seconds)
    used = oracle.get_threads()
    v1, rates1, n1, k1, rows1, el1 = median_rate(1, seconds)
    oracle.set_threads(all_cores)
    # gathered KV GB/s at the median rate: the sample's rows per token
    row_bytes = 2 * w.D * rows / max(n, 1)
    return {"value": round(v, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(), "gathered_kv_GBps": round(v * row_bytes / 1e9, 3),
            "passes_tokens_per_s": [round(r, 2) for r in rates],
            "value_1core": round(v1, 2), "passes_1core_tokens_per_s": [round(r, 2) for r in rates1],
            "sample": "fp64 two-pass attention only, median of " + describe(n, k, rows, el, used) +
                      "; one core: " + describe(n1, k1, rows1, el1, 1)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_probe():
    """libspd_probe.so (include/spd_probe.h): the measurement kernels."""
    import ctypes
    path = os.path.join(ROOT, "sparse_paged_decode_ragged_amd", "_lib", "libspd_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("libspd_probe.so not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.spd_probe_gather.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
    L.spd_probe_null.argtypes = [i32, P]
    L.spd_probe_store.argtypes = [P, i64, i32, P]
    return L


def probe_call(st: int, what: str) -> None:
    if st != 0:
        raise RuntimeError("%s failed with status %d" % (what, st))


def one_cu_parts(N: int) -> int:
    """Partitions per token that give each CU (256 of them) one share of a
    token's rows: every gathered row then enters exactly one CU."""
    return max(1, min(32, round(256 / max(N, 1))))


def touched_bytes(indices: np.ndarray, N: int, H: int, D: int) -> dict:
    """Bytes one set's attention call touches: its distinct pool rows, q, out,
    the indices and kv_indptr (the footprint that must exceed the Infinity
    Cache across the rotating sets)."""
    uniq = int(len(np.unique(indices))) if len(indices) else 0
    tb = uniq * 2 * D + 2 * N * H * D * 2 + 4 * len(indices) + 4 * (N + 1)
    return {"unique_rows": uniq, "gathered_rows": int(len(indices)),
            "unique_row_fraction": round(uniq / max(len(indices), 1), 4), "bytes": int(tb)}


def main():
    args = parse()
    if args.pmc_summary:
        out, factors = pmc_summary(args.pmc_summary, args.pmc_copy_mib)
        print(json.dumps({"per_kernel_KiB_per_dispatch": out, "scale": factors}, indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU; --gpus %d is not supported (the path would "
              "shard by tokens with no exchange step)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_paged_decode_ragged_amd as spd
    import workloads as W

    dev = torch.device("cuda:0")
    if args.workload in ("ragged", "large", "prefill", "long_context"):
        W.set_data_mode("device", dev)
    w = (W.make(args.workload, N=args.long_tokens, length=args.long_rows)
         if args.workload == "long_context" else W.make(args.workload))
    N, H, D = w.N, w.H, w.D
    max_len = w.max_len
    mode = {"auto": spd.MODE_AUTO, "heads": spd.MODE_HEADS, "rows": spd.MODE_ROWS,
            "wide": spd.MODE_WIDE, "split": spd.MODE_SPLIT}[args.mode]
    plan = spd.sparse_decode_attn_plan_info(N, H, D, max_len, args.split_rows, mode)
    ws_bytes = spd.sparse_decode_attn_workspace_size(N, H, D, max_len, args.split_rows, mode)
    b = w.builder
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q0 = W.device_bits(w.q_bits, dev)
    kv0 = W.device_bits(w.kv_bits, dev)
    sets = []

    def new_set(r):
        s = dict(q=q0 if r == 0 else q0.clone(), kv=kv0 if r == 0 else kv0.clone(),
                 sink=torch.from_numpy(w.attn_sink).to(dev),
                 out=torch.empty((N, H, D), dtype=torch.bfloat16, device=dev),
                 ws=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev))
        if b is not None:
            s.update(ss=t(b.state_slot), sl=t(b.swa_len), cp=t(b.comp_pos), bt=t(b.block_table),
                     ptr=torch.zeros(N + 1, dtype=torch.int32, device=dev),
                     idx=torch.zeros(b.capacity, dtype=torch.int32, device=dev))
        else:
            s.update(ptr=t(w.kv_indptr), idx=t(w.kv_indices))
        s["gw"] = torch.zeros(N * max(plan["head_groups"] * plan["splits"], one_cu_parts(N)) + 1,
                              dtype=torch.int32, device=dev)  # the gather probe's words
        sets.append(s)

    # The rotating sets: enough that the bytes the attention calls touch
    # (distinct rows, q, out, indices) exceed three times the 256 MB Infinity
    # Cache, so each call finds its rows in HBM.  Set 0's lists (built on the
    # GPU for builder-shaped workloads) size the rotation.
    new_set(0)
    if b is not None:
        spd.build_decode_indices(sets[0]["ss"], sets[0]["sl"], sets[0]["cp"], sets[0]["bt"], b.win,
                                 b.k_per_block, b.swa_pages, kv_indptr=sets[0]["ptr"],
                                 kv_indices=sets[0]["idx"])
        torch.cuda.synchronize()
        ptr0 = sets[0]["ptr"].cpu().numpy()
        idx0 = sets[0]["idx"].cpu().numpy()[: ptr0[-1]]
    else:
        idx0 = w.kv_indices
    touched = touched_bytes(idx0, N, H, D)
    n_sets = args.sets or max(2, min(32, math.ceil(3 * MALL_BYTES / touched["bytes"])))
    for r in range(1, n_sets):
        new_set(r)

    def build(s):
        spd.build_decode_indices(s["ss"], s["sl"], s["cp"], s["bt"], b.win, b.k_per_block,
                                 b.swa_pages, kv_indptr=s["ptr"], kv_indices=s["idx"])

    def attn(s):
        spd.sparse_decode_attn(s["q"], s["kv"], s["idx"], s["ptr"], s["sink"], w.softmax_scale,
                               out=s["out"], max_len=max_len, split_rows=args.split_rows,
                               mode=mode, workspace=s["ws"])

    def step(s):
        if b is not None:
            build(s)
        attn(s)

    # The same step with the page transform fused into the attention kernel
    # (builder-shaped workloads whose lists fit the paged call).
    has_paged = b is not None and b.win + b.topk <= 2048
    # the paged call never splits a slice: it takes the mode asked for unless
    # that is the split mode
    paged_mode = mode if mode in (spd.MODE_AUTO, spd.MODE_HEADS, spd.MODE_ROWS,
                                  spd.MODE_WIDE) else spd.MODE_AUTO

    def paged(s):
        spd.sparse_decode_attn_paged(s["q"], s["kv"], s["ss"], s["sl"], s["cp"], s["bt"], b.win,
                                     b.k_per_block, b.swa_pages, s["sink"], w.softmax_scale,
                                     out=s["out"], mode=paged_mode)

    # The attention call over an FP8 pool (e4m3 codes + one fp32 scale per row)
    # in its automatic plan for the same capacity bound, each set's pool filled
    # from its bf16 pool by the quantising store before timing; an FP8 pool is
    # half the bytes, so twice the sets keep the touched footprint out of the
    # Infinity Cache.
    has_fp8 = not args.no_fp8 and args.split_rows == 0
    fp8_sets = []
    if has_fp8:
        plan8 = spd.sparse_decode_attn_fp8_plan_info(N, H, D, max_len)
        ws8_bytes = spd.sparse_decode_attn_fp8_workspace_size(N, H, D, max_len)
        n8 = max(2, min(32, math.ceil(2 * MALL_BYTES / (w.P * D))))
        for r in range(n8):
            base = sets[r % n_sets]
            kv8 = torch.empty((w.P, D), dtype=torch.uint8, device=dev)
            ksc = torch.empty(w.P, dtype=torch.float32, device=dev)
            spd.quantize_kv_fp8(base["kv"], kv8, ksc)
            fp8_sets.append(dict(base, q=base["q"].clone(), kv8=kv8, ksc=ksc,
                                 out=torch.empty((N, H, D), dtype=torch.bfloat16, device=dev),
                                 ws8=torch.zeros(max(ws8_bytes, 16), dtype=torch.uint8,
                                                 device=dev)))

    # The decode-step producer (builder-shaped workloads): RMSNorm + RoPE of q
    # and of each token's new KV row, the KV row stored into its window-ring
    # slot of the set's bf16 pool; q_out is a buffer of its own, so the
    # attention legs keep their inputs.  Rotary width 64, positions < 4096.
    has_producer = not args.no_producer and b is not None
    rope_dim, max_pos = 64, 4096
    if has_producer:
        prng = np.random.default_rng(12345)
        ang = np.arange(max_pos)[:, None] * 10000.0 ** (-2.0 * np.arange(rope_dim // 2) / rope_dim)
        cos_sin = torch.from_numpy(
            np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).to(dev)
        qw = torch.from_numpy((1 + 0.1 * prng.standard_normal(D)).astype(np.float32)).to(dev)
        kw = torch.from_numpy((1 + 0.1 * prng.standard_normal(D)).astype(np.float32)).to(dev)
        for s in sets:
            s.update(q_prod=torch.empty_like(s["q"]), kv_new=W.device_bits(W.normal_bf16(prng, (N, D)), dev),
                     pos=torch.from_numpy(prng.integers(0, max_pos, size=N).astype(np.int32)).to(dev))

    # Prefill-shaped workloads whose lists are windows of one index stream: the
    # same batch through sparse_prefill_attn (tokens that share rows share a
    # workgroup).
    has_prefill = not args.no_prefill and "stream" in w.meta
    if has_prefill:
        m = w.meta
        pf_stream, pf_start, pf_len = t(m["stream"]), t(m["win_start"]), t(m["win_len"])
        for s in sets:
            s.update(out_pf=torch.empty((N, H, D), dtype=torch.bfloat16, device=dev))

    def prefill(s, group=0):
        spd.sparse_prefill_attn(s["q"], s["kv"], pf_stream, pf_start, pf_len, s["sink"],
                                w.softmax_scale, out=s["out_pf"], tokens_per_group=group)

    shared_group = 128 // H  # the grouping that fills four waves with shared tokens

    def prefill_shared(s):
        prefill(s, shared_group)

    def producer(s):
        spd.fused_qk_norm_rope_swa_store(s["q"], s["kv_new"], qw, kw, 1e-6, s["pos"], cos_sin,
                                         s["ss"], b.win, unified_kv=s["kv"], q_out=s["q_prod"])

    def attn_fp8(s):
        spd.sparse_decode_attn_fp8(s["q"], s["kv8"], s["ksc"], s["idx"], s["ptr"], s["sink"],
                                   w.softmax_scale, out=s["out"], max_len=max_len,
                                   workspace=s["ws8"])

    # Floor legs (libspd_probe.so): the same rows gathered by the same LDS-DMA
    # pattern with no arithmetic, in the plan's decomposition (head groups x
    # partitions: each group re-reads a token's rows) and in one where every
    # row enters one CU; an empty 256-workgroup launch; the output written by
    # 256 workgroups.  Each runs on the same rotating sets as the calls.
    has_floor = not args.no_floor
    if has_floor:
        probe = load_probe()
    g_plan, p_plan, p_one = plan["head_groups"], plan["splits"], one_cu_parts(N)
    out_bytes = N * H * D * 2

    def cur_stream():
        import ctypes
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def gather_plan(s):
        probe_call(probe.spd_probe_gather(s["kv"].data_ptr(), s["idx"].data_ptr(), s["ptr"].data_ptr(),
                                          N, D, g_plan, p_plan, s["gw"].data_ptr(), cur_stream()),
                   "spd_probe_gather")

    def gather_one(s):
        probe_call(probe.spd_probe_gather(s["kv"].data_ptr(), s["idx"].data_ptr(), s["ptr"].data_ptr(),
                                          N, D, 1, p_one, s["gw"].data_ptr(), cur_stream()),
                   "spd_probe_gather")

    def null_leg(s):
        probe_call(probe.spd_probe_null(256, cur_stream()), "spd_probe_null")

    def store_leg(s):
        probe_call(probe.spd_probe_store(s["out"].data_ptr(), out_bytes, 256, cur_stream()),
                   "spd_probe_store")

    floor_kinds = ((("gather_plan", gather_plan), ("gather_one", gather_one), ("null", null_leg),
                    ("store", store_leg)) if has_floor else ())

    for s in sets:  # eager warm-up (and the indices the graphs will rebuild)
        step(s)
    for s in fp8_sets:
        attn_fp8(s)
    torch.cuda.synchronize()
    # One graph per set for each of (step, attention call), plus one graph that
    # holds every set's call back to back: the timed loops replay the latter,
    # so consecutive calls are not separated by per-graph launch gaps.
    single = {"step": [], "attn": [], "paged": [], "producer": [], "prefill": [],
              "prefill_shared": [], "gather_plan": [], "gather_one": [], "null": [], "store": []}
    chain = {}
    cs = torch.cuda.Stream()
    if not args.eager:
        kinds = ((("step", step), ("attn", attn)) + ((("paged", paged),) if has_paged else ()) +
                 ((("producer", producer),) if has_producer else ()) +
                 ((("prefill", prefill), ("prefill_shared", prefill_shared)) if has_prefill else ()) +
                 floor_kinds)
        for name, fn in kinds:
            for s in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    fn(s)
                single[name].append(g)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                for s in sets:
                    fn(s)
            chain[name] = g
        if has_fp8:
            single["fp8"] = []
            for s in fp8_sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    attn_fp8(s)
                single["fp8"].append(g)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                for s in fp8_sets:
                    attn_fp8(s)
            chain["fp8"] = g
        torch.cuda.synchronize()

    def run_calls(k, name, fn):
        """Exactly k calls, rotating over the sets."""
        group = fp8_sets if name == "fp8" else sets
        if args.eager:
            for i in range(k):
                fn(group[i % len(group)])
            return
        for _ in range(k // len(group)):
            chain[name].replay()
        for i in range(k % len(group)):
            single[name][i].replay()

    def timed(k, name, fn):
        # events on the stream the calls run on (graphs replay on the current stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run_calls(k, name, fn)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if args.calibration_copy_mib:
        # a kernel of known traffic and a name of its own: bitwise_not over
        # calibration_copy_mib MiB of int32 reads and writes exactly that much
        n = (args.calibration_copy_mib << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    run_calls(args.warmup, "step", step)
    ms_per_step = timed(args.steps, "step", step) / args.steps
    # the attention call alone, same rotation: the roofline record's kernel
    run_calls(min(args.warmup, 64), "attn", attn)
    n_attn = max(args.steps, 100)
    us_attn = timed(n_attn, "attn", attn) * 1e3 / n_attn

    us_paged = None
    if has_paged:
        run_calls(min(args.warmup, 64), "paged", paged)
        us_paged = timed(n_attn, "paged", paged) * 1e3 / n_attn

    us_pf = None
    if has_prefill:
        run_calls(min(args.warmup, 64), "prefill", prefill)
        us_pf = timed(n_attn, "prefill", prefill) * 1e3 / n_attn
        run_calls(min(args.warmup, 64), "prefill_shared", prefill_shared)
        us_pf_shared = timed(n_attn, "prefill_shared", prefill_shared) * 1e3 / n_attn

    us_prod = None
    if has_producer:
        run_calls(min(args.warmup, 64), "producer", producer)
        us_prod = timed(n_attn, "producer", producer) * 1e3 / n_attn

    us_fp8 = None
    if has_fp8:
        run_calls(min(args.warmup, 64), "fp8", attn_fp8)
        us_fp8 = timed(n_attn, "fp8", attn_fp8) * 1e3 / n_attn

    floor = {}
    if has_floor:
        for name, fn in floor_kinds:
            run_calls(min(args.warmup, 64), name, fn)
            floor[name] = timed(n_attn, name, fn) * 1e3 / n_attn
        # a plain device copy of 512 MiB (reads and writes that much)
        n_copy = 512 << 20
        src = torch.ones(n_copy // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        floor["copy"] = e0.elapsed_time(e1) * 1e3 / 20
        del src, dst

    indptr = sets[0]["ptr"].cpu().numpy()
    indices = sets[0]["idx"].cpu().numpy()[: indptr[-1]]
    ab = algorithmic_bytes(indptr, N, H, D)
    tokens_per_s = N / (ms_per_step * 1e-3)
    gathered_gbps = ab["kv_bytes"] / (ms_per_step * 1e-3) / 1e9
    achieved = ab["B_alg"] / (us_attn * 1e-6) / 1e9
    if plan["mode"] == "rows":
        kernel = "attn_rows_kernel<%d>" % D
    elif plan["mode"] == "split":
        kernel = "attn_split_kernel<%d,%d,%d,false>" % (D, plan["heads_per_group"] // 32,
                                                        plan["parities"])
    elif plan.get("wide"):
        kernel = "attn_wide_kernel<%d,%d>" % (D, plan["heads_per_group"] // 32)
    else:
        kernel = "attn_heads_kernel<%d,%d>" % (D, plan["heads_per_group"] // 16)
        if plan["splits"] > 1:
            kernel += " + attn_combine_kernel"

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
        "config": {"workload": args.workload, "N": N, "H": H, "D": D, "pool_rows": w.P,
                   "max_len": max_len, "sum_L": ab["sum_L"], "nonempty_tokens": ab["nonempty"],
                   "plan": plan, "rotating_sets": n_sets,
                   "touched_bytes_per_set": touched["bytes"],
                   "touched_bytes_all_sets": touched["bytes"] * n_sets,
                   "unique_rows": touched["unique_rows"],
                   "unique_row_fraction": touched["unique_row_fraction"],
                   "seed": W.SEEDS.get(args.workload), "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None),
                   # sum of set 0's q and pool bit patterns (as int16): identifies the inputs
                   "input_checksum": int(q0.view(torch.int16).sum(dtype=torch.int64).item() +
                                         kv0.view(torch.int16).sum(dtype=torch.int64).item()),
                   "launch": "eager" if args.eager else "hip_graph_of_%d_steps" % n_sets,
                   "step": ("build_decode_indices + " if b is not None else "") + "sparse_decode_attn"},
        "gathered_kv_GBps": round(gathered_gbps, 1),
        "nonempty_tokens_per_s": round(ab["nonempty"] / (ms_per_step * 1e-3), 1),
        "gathered_kv_frac_of_hbm_peak": round(gathered_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": recorded_traffic(kernel, args.workload),
                     "kernel": kernel, "us_per_call": round(us_attn, 3),
                     "bytes_per_call": ab["B_alg"],
                     # the secondary bound: the same call's MFMA work against the bf16 peak
                     "mfma": {"flop_per_call": mfma_flops(ab["sum_L"], H, D),
                              "achieved_TFLOPs": round(mfma_flops(ab["sum_L"], H, D) / us_attn / 1e6, 1),
                              "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(mfma_flops(ab["sum_L"], H, D) / us_attn / 1e6 /
                                            MFMA_BF16_PEAK_TFLOPS, 4)}},
    }
    # the rows the call touches once each (prefill's windows overlap: its
    # gathered-byte rate can exceed HBM through cache reuse, this one cannot)
    ub = touched["unique_rows"] * 2 * D
    rec["unique_kv"] = {"bytes": ub, "GBps": round(ub / (us_attn * 1e-6) / 1e9, 1),
                        "frac": round(ub / (us_attn * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    if floor:
        kvb = ab["kv_bytes"]

        def gleg(us, groups, parts):
            return {"groups": groups, "parts": parts, "us_per_call": round(us, 3),
                    "kv_bytes": kvb, "bytes_into_cus": groups * kvb,
                    "GBps": round(kvb / (us * 1e-6) / 1e9, 1),
                    "frac": round(kvb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        cgb = 2 * (512 << 20) / (floor["copy"] * 1e-6) / 1e9
        rec["floor"] = {
            "kernels": "libspd_probe.so (include/spd_probe.h), same rotating sets and graphs",
            "launch_us": round(floor["null"], 3),
            "output_store_us": round(floor["store"], 3), "output_bytes": out_bytes,
            "gather_plan": gleg(floor["gather_plan"], g_plan, p_plan),
            "gather_one_cu": gleg(floor["gather_one"], 1, p_one),
            "copy": {"bytes_read_plus_written": 2 * (512 << 20), "us": round(floor["copy"], 2),
                     "GBps": round(cgb, 1), "frac": round(cgb / HBM_PEAK_GBPS, 4)}}
    if us_paged is not None:
        pp = spd.sparse_decode_attn_plan_info(N, H, D, 0, 0, paged_mode)  # the paged call never splits
        kernel_paged = ("attn_rows_kernel<%d, paged>" % D if pp["mode"] == "rows" else
                        "attn_wide_kernel<%d,%d, paged>" % (D, pp["heads_per_group"] // 32)
                        if pp.get("wide") else
                        "attn_heads_kernel<%d,%d, paged>" % (D, pp["heads_per_group"] // 16))
        # what the fused kernel must move: the rows, q, out, the sinks and the
        # builder inputs it reads (state_slot, swa_len, comp_pos, one block-table
        # entry per valid compressed entry) instead of kv_indptr / kv_indices
        n_win = int(np.clip(b.swa_len, 0, b.win).sum())
        b_paged = (ab["kv_bytes"] + ab["qo_bytes"] + 4 * H + 8 * N + 4 * N * b.topk +
                   4 * (ab["sum_L"] - n_win))
        ach_p = b_paged / (us_paged * 1e-6) / 1e9
        rec["fused_page_transform"] = {
            "step": "sparse_decode_attn_paged", "ms_per_step": round(us_paged * 1e-3, 6),
            "tokens_per_s": round(N / (us_paged * 1e-6), 1),
            "kernel": kernel_paged,
            "us_per_call": round(us_paged, 3), "bytes_per_call": int(b_paged),
            "achieved_GBps": round(ach_p, 1), "frac": round(ach_p / HBM_PEAK_GBPS, 4)}
    if us_fp8 is not None:
        # what the FP8 call must move: D code bytes and a 4-byte scale per
        # gathered row, q, out, the indices, kv_indptr and the sinks
        b_fp8 = ab["sum_L"] * (D + 4) + ab["qo_bytes"] + 4 * ab["sum_L"] + 4 * (N + 1) + 4 * H
        ach8 = b_fp8 / (us_fp8 * 1e-6) / 1e9
        k8 = fp8_kernel(plan8, D)
        rec["fp8_pool"] = {
            "call": "sparse_decode_attn_fp8_ex", "kernel": k8, "max_len": max_len,
            "splits": plan8["splits"], "rotating_sets": len(fp8_sets),
            "us_per_call": round(us_fp8, 3),
            "traffic": recorded_traffic(k8, args.workload + "_fp8"),
            "tokens_per_s": round(N / (us_fp8 * 1e-6), 1), "bytes_per_call": int(b_fp8),
            "achieved_GBps": round(ach8, 1), "frac": round(ach8 / HBM_PEAK_GBPS, 4)}
    if us_pf is not None:
        # what the shared-window call must move: q of non-empty tokens and out,
        # each stream position some window covers once (its row and its index),
        # the windows and the sinks
        m = w.meta
        U = covered_positions(len(m["stream"]), m["win_start"], m["win_len"])
        b_pf = ab["qo_bytes"] + U * (2 * D + 4) + 8 * N + 4 * H
        achf = b_pf / (us_pf * 1e-6) / 1e9
        rec["prefill"] = {
            "call": "sparse_prefill_attn", "kernel": "attn_wide_kernel<%d,%d, windows>" % (
                D, 4 if H == 128 else 2),
            "tokens_per_workgroup": 1 if H >= 64 else 2, "us_per_call": round(us_pf, 3),
            "tokens_per_s": round(N / (us_pf * 1e-6), 1), "covered_stream_positions": U,
            "bytes_per_call": int(b_pf), "achieved_GBps": round(achf, 1),
            "frac": round(achf / HBM_PEAK_GBPS, 4),
            "speedup_vs_decode_call": round(us_attn / us_pf, 3),
            "traffic": recorded_traffic("attn_wide_kernel<%d,%d, windows>" % (D, 4 if H == 128 else 2),
                                        args.workload + "_windows"),
            "tokens_per_workgroup_%d_us" % shared_group: round(us_pf_shared, 3)}
    if us_prod is not None:
        # q read and written, each token's KV row read and stored, the two
        # weights, the table rows used, positions and state slots
        b_prod = 4 * N * H * D + 4 * N * D + 8 * D + 4 * N * rope_dim + 8 * N
        achp = b_prod / (us_prod * 1e-6) / 1e9
        rec["producer"] = {
            "call": "fused_qk_norm_rope_swa_store",
            # the library takes two rows a wave from N*H + N >= 32768 rows, else one
            "kernel": "qk_norm_rope_store_kernel<%d,%d>" % (D, 2 if N * H + N >= 32768 else 1),
            "rope_dim": rope_dim, "us_per_call": round(us_prod, 3), "bytes_per_call": int(b_prod),
            "achieved_GBps": round(achp, 1), "frac": round(achp / HBM_PEAK_GBPS, 4)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, indptr, indices, args.cpu_seconds)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

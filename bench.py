#!/usr/bin/env python3
"""Benchmark of the paged-KV-cache hot path on one MI355X.

Default workload: Llama-2-7B-shaped decode -- 64 sequences, 32 query heads =
32 KV heads of dim 128, fp16 KV, block_size 16, context lengths uniform on
[1, 2048], tables from a random permutation of a pool of 64 * 128 blocks --
with the cache of all 32 layers resident in HBM (one 2 GiB K+V pool per
layer, 64 GiB in total), so that no decode finds its K/V in a cache level.

One step = one decode iteration over the whole path:
  host   the C++ block manager appends one token to every sequence (a new
         block when the last one is full) and packs tables / lengths / slots;
  H2D    the packed arrays go to the device (pinned, asynchronous);
  order  pa_decode_order sorts the sequences longest first (one small
         kernel, shared by every layer of the step);
  per layer (x32)
         pa_decode_append writes the new token's K/V into the cache and
         runs attention for all 64 sequences in one launch (--fused 0:
         pa_reshape_and_cache, then pa_decode).

Printed: one JSON line.  `value` is KV GB/s over the whole step (bytes of
cached K/V that decode must read, summed over layers, divided by wall time per
step; no events inside the steps -- on this stack each recorded event costs
several microseconds between kernels); `roofline` is the decode call alone:
after the timed steps, --steps sweeps of the step's decode call over the
layers of the last step's batch run back to back, bracketed by HIP events on the launch stream,
and the average call duration divides the call's algorithmic KV bytes;
`cpu_baseline` times the fp64 oracle on one layer of the same workload on the
host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama7b", choices=["llama7b", "gqa", "long", "copy", "scatter", "swap", "prefix", "prefill",
                            "prefill-long", "chunked", "sweep", "sampling", "read", "tiny"],
                   help="llama7b: the Llama-2-7B decode batch (default); gqa: 64 query heads over 8 KV "
                        "heads (matrix-core kernel); long: 16 x 4096 tokens; copy: block-copy calibration; scatter: the slot-mapped K/V write; "
                        "swap: block swaps between HBM and pinned host memory; prefix: 100 requests "
                        "sharing a 1000-token system prompt; prefill: causal attention of 32 prompts "
                        "(mean 500 tokens) over the paged cache; prefill-long: full causal prompts of 1k-8k "
                        "tokens; sweep: decode of 256 sequences at "
                        "block_size 8/16/32/64; sampling: 32 samples of one prompt with copy-on-write; "
                        "read: read-only streaming ceilings (contiguous, and the decode's block pattern); "
                        "tiny: latency of the 4-sequence tiny case")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--batch", type=int, default=0, help="sequences (0: 64 for llama7b, 256 for gqa)")
    p.add_argument("--block-size", type=int, default=16)
    p.add_argument("--head-dim", type=int, default=128,
                   help="gqa, prefill, prefill-long: head_dim of the batch (64/128/256)")
    p.add_argument("--partition", type=int, default=0, help="decode partition size (0 = library default)")
    p.add_argument("--fused", type=int, default=1,
                   help="decode workloads: 1 writes the new K/V inside the decode call (pa_decode_append), "
                        "0 runs pa_reshape_and_cache then pa_decode")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--compare-default", type=int, default=1,
                   help="long: also time the library's default partition (0 skips it, e.g. for counter passes)")
    p.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="oracle CPU time: whole-layer decodes are repeated until this much has been spent")
    return p.parse_args()


KERNEL_SOURCES = {"llama7b": ("decode.hip",), "gqa": ("decode.hip", "decode_gqa.hip"),
                  "gqa_d64": ("decode.hip", "decode_gqa.hip"), "gqa_d256": ("decode.hip", "decode_gqa.hip"),
                  "prefill": ("prefill.hip",)}


def code_tokens(text: str) -> str:
    """The source with comments removed and whitespace runs folded to one
    space: what the compiler sees, so that an edit of a comment keeps counter
    summaries taken on the same code valid.  String and character literals
    are kept whole (a '//' inside one is not a comment)."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(workload, ("decode.hip",)):
        with open(os.path.join(ROOT, "paged_kv_cache_390_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def pmc_summary(workload: str):
    """The committed PMC summary of the workload's timed kernel (the decode
    call, or pa_prefill), if it was taken on the current kernel sources;
    else None."""
    name = "prefill_pmc.json" if workload == "prefill" else f"decode_{workload}_pmc.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash(workload):
        return None
    return d


def traffic_from_profiles(workload: str):
    """HBM bytes per call from the committed PMC summary (see pmc_summary)."""
    d = pmc_summary(workload)
    return None if d is None else d.get("hbm_bytes_per_call", d.get("hbm_bytes_per_decode_call"))


def traffic_fields(workload: str) -> dict:
    """roofline fields from the PMC summary: the measured HBM bytes per call
    (`traffic`), the same run's algorithmic bytes per call and their ratio,
    and the cached tokens of the profiled calls -- the counter run is a short
    one whose batch has grown fewer steps than the timed one, so its bytes
    are compared with its own algorithmic bytes, never with this line's."""
    d = pmc_summary(workload)
    if d is None:
        return {"traffic": None}
    out = {"traffic": d.get("hbm_bytes_per_call", d.get("hbm_bytes_per_decode_call"))}
    alg = d.get("algorithmic_total_bytes_per_call")
    if alg:
        out["traffic_algorithmic_bytes"] = alg
        out["traffic_ratio"] = round(out["traffic"] / alg, 4)
    if d.get("cached_tokens_per_call"):
        out["traffic_ctx_tokens"] = d["cached_tokens_per_call"]
    return out


def host_cpu() -> dict:
    """The host the oracle runs on: logical CPUs, those this process may use,
    the job's CPU share (OMP_NUM_THREADS) and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": model}


def stats_of(xs, scale: float = 1e3, nd: int = 3) -> dict:
    """median / mean / min / max of a list of seconds, times `scale` (ms by
    default), and the sample count."""
    import statistics
    return {"median": round(statistics.median(xs) * scale, nd), "mean": round(sum(xs) / len(xs) * scale, nd),
            "min": round(min(xs) * scale, nd), "max": round(max(xs) * scale, nd), "n": len(xs)}


def tiny_latency(dev, reps: int = 100, oracle_reps: int = 200, with_oracle: bool = True) -> dict:
    """The tiny case (4 sequences of 1/5/12/50 tokens, B = 4, 2 heads x 16,
    sequence 2 on the page's table [7, 3, 1]): pa_decode latency, each call
    bracketed by its own HIP events (launch included), and the oracle's
    latency on the same inputs."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    w = workloads.tiny(seed=0)
    S, B = len(w.lens), w.block_size
    bm = pa.BlockManager(w.num_blocks, B)
    for s, (n, t) in enumerate(zip(w.lens, w.tables)):
        bm.set_table(s, t, n)
    width = max(len(t) for t in w.tables)
    slots = np.concatenate([bm.get_slots(s, 0, n) for s, n in enumerate(w.lens)])
    tables, lens = bm.get_tables(range(S), width)
    kc = torch.zeros((w.num_blocks, w.num_kv_heads, B, w.head_dim), dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    pa.pa_reshape_and_cache(torch.from_numpy(w.k_tokens).to(dev), torch.from_numpy(w.v_tokens).to(dev),
                            torch.from_numpy(slots).to(dev), kc, vc)
    q = torch.from_numpy(w.q).to(dev)
    d_t, d_l = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    out = torch.empty_like(q)
    for _ in range(10):
        pa.pa_decode(out, q, kc, vc, d_t, d_l, w.scale, B)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        pa.pa_decode(out, q, kc, vc, d_t, d_l, w.scale, B)
        b.record()
    torch.cuda.synchronize()
    res = {"workload": "tiny", "gpu_us": stats_of([a.elapsed_time(b) / 1e3 for a, b in ev], 1e6, 2)}
    if with_oracle:
        import oracle
        kc_h, vc_h = kc.cpu().numpy(), vc.cpu().numpy()
        ts = []
        for _ in range(oracle_reps):
            t0 = time.perf_counter()
            oracle.decode(w.q, kc_h, vc_h, tables, lens, w.scale, nthreads=1)
            ts.append(time.perf_counter() - t0)
        res["oracle_us_1_thread"] = stats_of(ts, 1e6, 2)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the decode path would shard "
              "by sequence or by KV head with no exchange between GPUs", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("bench.py: --steps >= 1 and --warmup >= 0 required")

    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    if not torch.cuda.is_available():
        sys.exit("bench.py: no GPU visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()                                     # fail loudly if the HIP library is missing

    if args.workload == "copy":
        return copy_bench(args, dev)
    if args.workload == "scatter":
        return scatter_bench(args, dev)
    if args.workload == "swap":
        return swap_bench(args, dev)
    if args.workload == "prefix":
        return prefix_bench(args, dev)
    if args.workload == "prefill":
        return prefill_bench(args, dev)
    if args.workload == "chunked":
        return chunked_bench(args, dev)
    if args.workload == "prefill-long":
        return prefill_long_bench(args, dev)
    if args.workload == "sweep":
        return sweep_bench(args, dev)
    if args.workload == "sampling":
        return sampling_bench(args, dev)
    if args.workload == "read":
        return read_bench(args, dev)
    if args.workload == "tiny":
        return tiny_bench(args, dev)

    L = args.layers
    B = args.block_size
    K, W = args.steps, args.warmup
    if args.workload == "llama7b":
        w = workloads.llama7b_decode(seed=args.seed, num_seqs=args.batch or 64, block_size=B)
        wl_name = "llama2-7b-decode"
        ctx_desc = "U[1,2048]"
    elif args.workload == "gqa":
        w = workloads.gqa_decode(seed=args.seed, num_seqs=args.batch or 256, block_size=B, head_dim=args.head_dim)
        wl_name = "gqa-64q-8kv-decode" if args.head_dim == 128 else f"gqa-64q-8kv-d{args.head_dim}-decode"
        ctx_desc = "U[1,2048]"
    else:
        w = workloads.long_context(seed=args.seed, num_seqs=16, block_size=B,
                                   spare_blocks=16 * workloads.ceil_div(W + K + 1, B))
        wl_name = "long-context-decode"
        ctx_desc = "4096"
    S, H, Hkv, D, NB = len(w.lens), w.num_heads, w.num_kv_heads, w.head_dim, w.num_blocks
    grow = W + K + 1
    width = workloads.ceil_div(int(w.lens.max()) + grow, B)

    # ---- pools for every layer (inputs resident in HBM before timing)
    log(f"[bench] {wl_name}: S={S} H={H} Hkv={Hkv} D={D} B={B} NB={NB}/layer layers={L} "
        f"pool {2 * NB * Hkv * B * D * 2 / 2**30:.1f} GiB/layer")
    t = time.perf_counter()
    kcs, vcs = [], []
    for l in range(L):
        k, v = w.pool(l, dev)
        kcs.append(k)
        vcs.append(v)
    torch.cuda.synchronize()
    log(f"[bench] pools generated in {time.perf_counter() - t:.1f}s")
    oracle_pool = (kcs[0].cpu().numpy(), vcs[0].cpu().numpy()) if args.cpu_baseline else None

    q, key, val = w.new_tokens(0, dev)

    # ---- block manager: the pages' tables (a permutation of the pool), n - 1 tokens cached
    bm = pa.BlockManager(NB, B)
    for s, n in enumerate(w.lens.tolist()):
        bm.set_table(s, w.perm_tables[s, :workloads.ceil_div(n - 1, B)], n - 1)
    seqs = np.arange(S, dtype=np.int64)
    part = args.partition
    if args.workload == "long" and part == 0:
        part = 512                      # the long-context workload fixes 512-token partitions + the merge kernel
    ws_bytes = max(pa.pa_decode_workspace_size(S, H, Hkv, D, B, width * B, part),
                   pa.pa_decode_workspace_size(S, H, Hkv, D, B, width * B, 0))
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    nbuf = 2
    h_tables = [torch.empty((S, width), dtype=torch.int32).pin_memory() for _ in range(nbuf)]
    h_lens = [torch.empty(S, dtype=torch.int32).pin_memory() for _ in range(nbuf)]
    h_slots = [torch.empty(S, dtype=torch.int64).pin_memory() for _ in range(nbuf)]
    d_tables = torch.empty((S, width), dtype=torch.int32, device=dev)
    d_lens = torch.empty(S, dtype=torch.int32, device=dev)
    d_slots = torch.empty(S, dtype=torch.int64, device=dev)
    copied = [None] * nbuf
    out = torch.empty((S, H, D), dtype=torch.float16, device=dev)
    d_order = torch.empty(S, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    kv_per_token = 2 * Hkv * D * 2           # K and V, fp16, one layer

    def decode_call(l, p=None):
        p = part if p is None else p
        if args.fused:
            pa.pa_decode_append(out, q, key, val, kcs[l], vcs[l], d_tables, d_lens, w.scale, B,
                                max_context_len=width * B, partition_size=p, workspace=workspace,
                                seq_order=d_order)
        else:
            pa.pa_decode(out, q, kcs[l], vcs[l], d_tables, d_lens, w.scale, B, max_context_len=width * B,
                         partition_size=p, workspace=workspace, seq_order=d_order)

    def step(i):
        b = i % nbuf
        if copied[b] is not None:
            copied[b].synchronize()          # the pinned buffer's previous upload has been consumed
        slots, pairs = bm.append_tokens(seqs)
        assert len(pairs) == 0
        bm.get_tables(seqs, width, out=h_tables[b].numpy(), lens_out=h_lens[b].numpy())
        h_slots[b].numpy()[:] = slots
        ctx = int(h_lens[b].numpy().astype(np.int64).sum())
        d_tables.copy_(h_tables[b], non_blocking=True)
        d_lens.copy_(h_lens[b], non_blocking=True)
        if not args.fused:                   # the fused call takes each slot from the table
            d_slots.copy_(h_slots[b], non_blocking=True)
        e = torch.cuda.Event()
        e.record(stream)
        copied[b] = e
        pa.pa_decode_order(d_lens, width * B, out=d_order)     # one dispatch order for every layer
        for l in range(L):
            if args.fused:
                decode_call(l)
            else:
                pa.pa_reshape_and_cache(key, val, d_slots, kcs[l], vcs[l])
                decode_call(l)
        return ctx

    all_ctx = 0                              # cached tokens over every decode call of the run
    for i in range(W):
        all_ctx += step(i) * L
    torch.cuda.synchronize()

    ctx_sum = 0
    ctx_last = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ctx_last = step(W + i)
        ctx_sum += ctx_last
        all_ctx += ctx_last * L
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    wall = t1 - t0
    ms_per_step = wall / K * 1e3
    kv_bytes_total = ctx_sum * kv_per_token * L          # over the K timed steps
    value = kv_bytes_total / wall / 1e9
    tokens_per_s_layer = S * L / (wall / K)

    # ---- the decode call alone: K sweeps over the layers of the last step's
    # batch, back to back, events only between sweeps (in fused mode each
    # call writes the same new K/V into the same slots again)
    sweep_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    sweep_ev[0].record(stream)
    for i in range(K):
        for l in range(L):
            decode_call(l)
        sweep_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [sweep_ev[i].elapsed_time(sweep_ev[i + 1]) / L for i in range(K)]
    all_ctx += ctx_last * L * K
    # the long-context line also times the library's default partition on
    # the same batch (interleaved with the fixed one, sweeps over the layers)
    alt = None
    default_p = pa.pa_decode_default_partition(S, H, Hkv, D, B, width * B)
    if args.workload == "long" and default_p != part and args.compare_default:
        t_fixed, t_default = [], []
        for i in range(max(K // 2, 2)):
            for p_, acc in ((part, t_fixed), (0, t_default)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for l in range(L):
                    decode_call(l, p_)
                e1.record(stream)
                torch.cuda.synchronize()
                acc.append(e0.elapsed_time(e1) / L / 1e3)
        alt = {"partition_size": default_p, "us_per_call_median": round(statistics.median(t_default) * 1e6, 2),
               "GB_s": round(ctx_last * kv_per_token / statistics.median(t_default) / 1e9, 2),
               "fixed_partition_us_per_call_median": round(statistics.median(t_fixed) * 1e6, 2)}
        log(f"[bench] library default partition {default_p}: {alt['us_per_call_median']} us per call = "
            f"{alt['GB_s']} GB/s (partition {part} interleaved: {alt['fixed_partition_us_per_call_median']} us)")
    dec_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    kv_per_launch = ctx_last * kv_per_token
    achieved = kv_per_launch / dec_avg_s / 1e9
    log(f"[bench] step {ms_per_step:.3f} ms ({L} layers) = {value:.0f} GB/s ({100 * value / HBM_PEAK_GBS:.1f}% of "
        f"peak); decode call avg {dec_avg_s * 1e6:.1f} us = {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of peak); per-sweep call avg min {min(dec_ms) * 1e3:.1f} us "
        f"max {max(dec_ms) * 1e3:.1f} us")

    # ---- oracle on the host cores, same workload (layer 0, one decode)
    cpu = None
    tiny = None
    if args.cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        tables, lens = bm.get_tables(seqs, width)
        q_h = q.cpu().numpy()
        kc_h, vc_h = oracle_pool
        layer_kv = int(lens.astype(np.int64).sum()) * kv_per_token
        per_call, spent = [], 0.0
        while len(per_call) < 3 or spent < args.cpu_seconds:
            c0 = time.perf_counter()
            oracle.decode(q_h, kc_h, vc_h, tables, lens, w.scale, nthreads=threads)
            per_call.append(time.perf_counter() - c0)
            spent += per_call[-1]
        c0 = time.perf_counter()
        oracle.decode(q_h, kc_h, vc_h, tables, lens, w.scale, nthreads=1)
        one = time.perf_counter() - c0
        med = statistics.median(per_call)
        cpu = {"value": round(layer_kv / med / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(per_call)} x one layer's decode of the same batch ({S} seqs x {H} heads, "
                         f"{int(lens.sum())} cached tokens, {layer_kv / 1e9:.3f} GB of K/V), fp64 C oracle on "
                         f"{threads} threads, {spent:.1f} s; value from the median call",
               "per_call_ms": stats_of(per_call),
               "value_from_mean": round(layer_kv * len(per_call) / spent / 1e9, 4),
               "single_thread": {"value": round(layer_kv / one / 1e9, 4), "unit": "GB/s",
                                 "ms_per_call": round(one * 1e3, 1),
                                 "sample": "one call of the same layer's decode on 1 thread"},
               **host_cpu()}
        log(f"[bench] cpu oracle: {cpu['value']} GB/s on {threads} threads (median of {len(per_call)} calls, "
            f"{spent:.1f}s); 1 thread {cpu['single_thread']['value']} GB/s")
        tiny = tiny_latency(dev)
        log(f"[bench] tiny case: pa_decode {tiny['gpu_us']['median']} us (median, launch included), oracle "
            f"{tiny['oracle_us_1_thread']['median']} us on 1 thread")

    traffic = traffic_fields(args.workload if args.workload != "gqa" or args.head_dim == 128
                             else f"gqa_d{args.head_dim}")
    line = {
        "metric": "paged-decode achieved KV GB/s (% of HBM peak) + tokens/s per layer, bs=16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer": round(tokens_per_s_layer, 1),
        "decode_only": {"GB_s": round(achieved, 2), "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
                        "tokens_per_s_per_layer": round(S / dec_avg_s, 1), "us_per_call": round(dec_avg_s * 1e6, 2),
                        "us_per_call_by_sweep": stats_of([x / 1e3 for x in dec_ms], 1e6, 2),
                        "GB_s_from_median_sweep": round(kv_per_launch / (statistics.median(dec_ms) / 1e3) / 1e9, 2)},
        "config": {"workload": wl_name, "batch": S, "block_size": B, "num_heads": H, "num_kv_heads": Hkv,
                   "head_dim": D, "context": ctx_desc, "layers_resident": L, "pool_blocks_per_layer": NB,
                   "partition_size": part or default_p,
                   "step": ("host append+tables, H2D, decode order, per layer pa_decode_append (new K/V "
                            "written inside the decode call)" if args.fused else
                            "host append+tables, H2D, decode order, per layer reshape_and_cache + decode")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), **traffic,
                     "kernel": "decode call (partition kernel + merge kernel when a context is split)",
                     "algorithmic_bytes_per_call": kv_per_launch, "cached_tokens_per_call": ctx_last},
        "decode_calls": {"count": (W + 2 * K) * L, "cached_tokens_total": all_ctx},
        "decode_only_library_default_partition": alt,
        "cpu_baseline": cpu,
        "tiny_latency": tiny,
    }
    print(json.dumps(line), flush=True)


def copy_bench(args, dev):
    """Block copies of known size through pa_copy_blocks: a plain streaming
    copy (every byte read once and written once) used as the same-box
    bandwidth reference and as the calibration kernel for the HBM byte
    counters."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa

    NB, Hkv, B, D = 8192, 32, 16, 128
    npairs = 4096
    k = torch.zeros((NB, Hkv, B, D), dtype=torch.float16, device=dev)
    v = torch.zeros_like(k)
    perm = np.random.default_rng(args.seed).permutation(NB)
    pairs = torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).astype(np.int64)).to(dev)
    block_bytes = Hkv * B * D * 2
    moved = 2 * npairs * block_bytes            # K and V blocks, each read once and written once
    for _ in range(args.warmup):
        pa.pa_copy_blocks([k], [v], pairs)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        pa.pa_copy_blocks([k], [v], pairs)
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / len(ms) / 1e3
    gbs = 2 * moved / avg / 1e9               # read + write
    log(f"[bench] copy: {npairs} pairs x 2 x {block_bytes // 1024} KiB, {moved / 2**30:.2f} GiB read + "
        f"written per call, avg {avg * 1e6:.1f} us = {gbs:.0f} GB/s (read+write)")
    print(json.dumps({"metric": "block-copy GB/s (read+write)", "value": round(gbs, 2), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                      "bytes_read_per_call": moved, "bytes_written_per_call": moved,
                      "us_per_call": round(avg * 1e6, 2),
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
                      "config": {"workload": "copy-blocks", "pairs": npairs, "block_bytes": block_bytes}}),
          flush=True)


def scatter_bench(args, dev):
    """pa_reshape_and_cache on its own: the prompts of the prefill workload
    (32 prompts, 15,360 tokens, lengths clip(N(500, 150), 16, 2048)) written
    into their slots at the Llama-2-7B head shape (32 x 128, fp16, B = 16),
    slots from the product block manager; then one decode step's write (64
    tokens, the Llama decode batch's size), which is bound by launch latency.
    Every byte of K and V is read once and written once."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    Hkv, D, B = 32, 128, args.block_size
    sw = workloads.block_size_sweep(seed=args.seed, num_seqs=32, gen_max=1)
    lens_l = [int(n) - 1 for n in sw.lens]
    T = int(sum(lens_l))
    NB = sum(-(-n // B) for n in lens_l) + 8
    bm = pa.BlockManager(NB, B)
    slots = np.concatenate([bm.add_sequence(s, n) for s, n in enumerate(lens_l)])
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    kc = torch.zeros((NB, Hkv, B, D), dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    key = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
    val = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
    d_slots = torch.from_numpy(slots).to(dev)
    results = []
    for name, t in (("prompts", T), ("decode-step", 64)):
        k_t, v_t, s_t = key[:t], val[:t], d_slots[:t]
        for _ in range(max(args.warmup, 3)):
            pa.pa_reshape_and_cache(k_t, v_t, s_t, kc, vc)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            pa.pa_reshape_and_cache(k_t, v_t, s_t, kc, vc)
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        moved = 2 * t * Hkv * D * 2                   # K and V bytes, each read once and written once
        gbs = 2 * moved / us / 1e3
        log(f"[bench] scatter {name}: {t} tokens x {Hkv} x {D}, {us:.1f} us per call = {gbs:.0f} GB/s (read+write)")
        results.append({"write": name, "tokens": t, "us": round(us, 2), "GB_s": round(gbs, 2)})
    best = results[0]
    print(json.dumps({"metric": "slot-mapped KV write GB/s (read+write)", "value": best["GB_s"], "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                      "dtype": "f16", "writes": results,
                      "roofline": {"bound": "hbm", "achieved": best["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(best["GB_s"] / HBM_PEAK_GBS, 4), "traffic": None},
                      "config": {"workload": "reshape-and-cache", "tokens": T, "num_kv_heads": Hkv, "head_dim": D,
                                 "block_size": B}}), flush=True)


def swap_bench(args, dev):
    """Swap a batch of 16 sequences x 2048 tokens (Llama-2-7B heads, B=16)
    out to pinned host memory and back, over --layers layers (default here
    4: 2 GiB each way).  Timed with HIP events around each pa_swap_blocks
    call; the host block manager's bookkeeping and the pairs' upload sit
    outside the events.  GB/s per direction against PCIe 5.0 x16 (64 GB/s
    per direction)."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa

    L = args.layers if args.layers != 32 else 4
    S, n, Hkv, B, D = 16, 2048, 32, 16, 128
    need = S * n // B
    NB, NH = need + 64, need + 64
    log(f"[bench] swap: {S} x {n} tokens, {L} layers, {2 * L} caches of {NB} blocks x {Hkv * B * D * 2 // 1024} KiB")
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    caches = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(2 * L)]
    hosts = [torch.empty((NH, Hkv, B, D), dtype=torch.float16).pin_memory() for _ in range(2 * L)]
    bm = pa.BlockManager(NB, B, NH)
    for s in range(S):
        bm.add_sequence(s, n)
    seqs = list(range(S))
    moved = need * len(caches) * Hkv * B * D * 2        # bytes per direction: every block of every cache
    t_out, t_in = [], []
    for it in range(args.warmup + args.steps):
        pout = torch.from_numpy(bm.swap_out(seqs)).to(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pa.pa_swap_blocks(caches, hosts, pout, pa.PA_SWAP_OUT)
        b.record()
        pin = torch.from_numpy(bm.swap_in(seqs)).to(dev)
        c, d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c.record()
        pa.pa_swap_blocks(caches, hosts, pin, pa.PA_SWAP_IN)
        d.record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            t_out.append(a.elapsed_time(b) / 1e3)
            t_in.append(c.elapsed_time(d) / 1e3)
    out_gbs = moved / (sum(t_out) / len(t_out)) / 1e9
    in_gbs = moved / (sum(t_in) / len(t_in)) / 1e9
    log(f"[bench] swap out {moved / 2**30:.2f} GiB in {1e3 * sum(t_out) / len(t_out):.2f} ms = {out_gbs:.1f} GB/s; "
        f"in {1e3 * sum(t_in) / len(t_in):.2f} ms = {in_gbs:.1f} GB/s")
    print(json.dumps({"metric": "KV block swap GB/s per direction (HBM <-> pinned host)", "value": round(
        min(out_gbs, in_gbs), 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "swap_out_GB_s": round(out_gbs, 2), "swap_in_GB_s": round(in_gbs, 2),
        "bytes_per_direction": moved, "pcie_peak_GB_s": 64.0,
        "config": {"workload": "swap", "sequences": S, "tokens": n, "layers": L, "num_kv_heads": Hkv,
                   "block_size": B, "head_dim": D}}), flush=True)


def prefix_bench(args, dev):
    """100 requests whose prompts start with one 1000-token system prompt
    (the n1n.ai page's example), each followed by its own 1..200 tokens,
    Llama-2-7B heads, B = 16, --layers layers resident.  The product block
    manager shares the prompt's 62 full blocks (one copy, count 100); one
    decode step per layer is timed with HIP events.  Reported: logical KV
    GB/s (what the kernel attends over, the shared blocks counted once per
    request) next to the unique bytes in HBM per step, and the host time of
    the cached prompt admissions."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa

    L = args.layers
    R, P, Hkv, H, B, D = 100, 1000, 32, 32, 16, 128
    rng = np.random.default_rng(args.seed)
    system = rng.integers(0, 32000, size=P).tolist()
    suffix = rng.integers(1, 201, size=R).tolist()
    toks = [system + rng.integers(0, 32000, size=s).tolist() for s in suffix]
    NB = P // B + sum(-(-(P + s) // B) - P // B for s in suffix) + 64
    bm = pa.BlockManager(NB, B)
    t0 = time.perf_counter()
    cached = [bm.add_sequence_cached(r, toks[r])[1] for r in range(R)]
    admit_us = (time.perf_counter() - t0) / R * 1e6
    used = NB - bm.num_free()
    width = -(-max(len(t) for t in toks) // B)
    tables, lens = bm.get_tables(range(R), width)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    kcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
    vcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
    q = torch.randn((R, H, D), generator=g, device=dev, dtype=torch.float16)
    d_tables, d_lens = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    out = torch.empty_like(q)
    ws = torch.zeros(max(1, pa.pa_decode_workspace_size(R, H, Hkv, D, B, width * B, args.partition)),
                     dtype=torch.uint8, device=dev)

    def call(l):
        pa.pa_decode(out, q, kcs[l], vcs[l], d_tables, d_lens, 1 / np.sqrt(D), B, max_context_len=width * B,
                     partition_size=args.partition, workspace=ws)

    for _ in range(args.warmup):
        for l in range(L):
            call(l)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps * L)]
    for i in range(args.steps):
        for l in range(L):
            a, b = ev[i * L + l]
            a.record()
            call(l)
            b.record()
    torch.cuda.synchronize()
    us = np.mean([a.elapsed_time(b) for a, b in ev]) * 1e3
    kv_tok = 2 * Hkv * D * 2
    logical = int(lens.astype(np.int64).sum()) * kv_tok
    unique = used * B * kv_tok
    log(f"[bench] prefix: {R} requests, {used} blocks in use ({sum(-(-len(t) // B) for t in toks)} unshared), "
        f"admission {admit_us:.1f} us/request on the host; decode {us:.1f} us/layer = {logical / us / 1e3:.0f} GB/s "
        f"logical, {unique / us / 1e3:.0f} GB/s of unique blocks")
    print(json.dumps({"metric": "prefix-shared decode: logical KV GB/s", "value": round(logical / us / 1e3, 2),
                      "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": True, "us_per_layer": round(us, 2),
                      "unique_GB_s": round(unique / us / 1e3, 2), "blocks_in_use": used,
                      "blocks_unshared": sum(-(-len(t) // B) for t in toks),
                      "cached_tokens": int(sum(cached)), "admission_us_per_request": round(admit_us, 2),
                      "config": {"workload": "prefix", "requests": R, "system_prompt": P,
                                 "own_tokens": "U[1,200]", "num_heads": H, "num_kv_heads": Hkv,
                                 "head_dim": D, "block_size": B, "layers_resident": L}}), flush=True)


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix cores, published


def prefill_bench(args, dev):
    """Prompt prefill over the paged cache: 32 prompts with lengths
    clip(N(500, 150), 16, 2048) (the prompt mix of the block-size
    experiment on the 5688vip.com page), Llama-2-7B heads (32 x 128), B = 16,
    --layers layers resident (default here 4).  Each timed call is one
    layer's pa_prefill over every prompt (the K/V already scattered); then
    the whole prompt path per layer -- K/V write and attention -- as
    pa_reshape_and_cache + pa_prefill and as one pa_prefill_append.  The
    sequences are dispatched longest first: pa_decode_order once per step,
    timed with the first layer's call.  Algorithmic flops = sum over heads
    and new tokens of 4 * D * (causal positions seen); against the dense
    fp16 matrix-core peak."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    L = args.layers if args.layers != 32 else 4
    S, H, Hkv, D, B = 32, 32, 32, args.head_dim, args.block_size
    sw = workloads.block_size_sweep(seed=args.seed, num_seqs=S, gen_max=1)
    lens_l = [int(n) - 1 for n in sw.lens]                 # the prompt part only
    T = int(sum(lens_l))
    NB = sum(-(-n // B) for n in lens_l) + 8
    bm = pa.BlockManager(NB, B)
    slots = np.concatenate([bm.add_sequence(s, n) for s, n in enumerate(lens_l)])
    width = -(-max(lens_l) // B)
    tables, lens = bm.get_tables(range(S), width)
    qs = np.concatenate([[0], np.cumsum(lens_l)]).astype(np.int32)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    kcs, vcs, keys, vals = [], [], [], []
    d_slots = torch.from_numpy(slots).to(dev)
    for _ in range(L):
        kc = torch.empty((NB, Hkv, B, D), dtype=torch.float16, device=dev)
        vc = torch.empty_like(kc)
        key = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
        val = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float16)
        pa.pa_reshape_and_cache(key, val, d_slots, kc, vc)
        kcs.append(kc)
        vcs.append(vc)
        keys.append(key)
        vals.append(val)
    q = torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float16)
    out = torch.empty_like(q)
    d_t, d_l, d_q = (torch.from_numpy(x).to(dev) for x in (tables, lens, qs))
    mq = max(lens_l)
    flops = sum(4.0 * D * H * n * (n + 1) / 2 for n in lens_l)
    # the sequences longest first, computed once per step (inside the first
    # layer's timed call) and shared by every layer
    order = torch.empty(S, dtype=torch.int32, device=dev)

    def step_order():
        pa.pa_decode_order(d_l, mq, out=order)

    def call(l):
        pa.pa_prefill(out, q, kcs[l], vcs[l], d_t, d_l, d_q, 1 / np.sqrt(D), max_query_len=mq, seq_order=order)

    for _ in range(max(args.warmup, 3)):
        step_order()
        for l in range(L):
            call(l)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps * L)]
    for i in range(args.steps):
        for l in range(L):
            a, b = ev[i * L + l]
            a.record()
            if l == 0:
                step_order()
            call(l)
            b.record()
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    tflops = flops / us / 1e6
    log(f"[bench] prefill: {S} prompts, {T} tokens (max {mq}), {L} layers; {us:.1f} us per layer = "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / MFMA_F16_PEAK_TFLOPS:.1f}% of dense fp16 MFMA peak), "
        f"{T / us * 1e6:.0f} prompt tokens/s per layer")

    # ---- the whole prompt path per layer: writing the prompts' K/V and the
    # attention, as two calls (pa_reshape_and_cache, pa_prefill) or one
    # (pa_prefill_append), in interleaved rounds of passes over the layers
    def two_calls(l):
        if l == 0:
            step_order()
        pa.pa_reshape_and_cache(keys[l], vals[l], d_slots, kcs[l], vcs[l])
        call(l)

    def fused(l):
        if l == 0:
            step_order()
        pa.pa_prefill_append(out, q, keys[l], vals[l], kcs[l], vcs[l], d_t, d_l, d_q, 1 / np.sqrt(D),
                             max_query_len=mq, seq_order=order)

    path_us = {"two_calls": [], "fused": []}
    for _ in range(max(args.steps // 2, 2)):
        for name, fn in (("two_calls", two_calls), ("fused", fused)):
            for l in range(L):
                fn(l)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for l in range(L):
                fn(l)
            b.record()
            torch.cuda.synchronize()
            path_us[name].append(a.elapsed_time(b) * 1e3 / L)
    two_us = float(np.median(path_us["two_calls"]))
    fused_us = float(np.median(path_us["fused"]))
    log(f"[bench] prompt path per layer (K/V write + attention): pa_reshape_and_cache + pa_prefill {two_us:.1f} us, "
        f"pa_prefill_append {fused_us:.1f} us ({T / fused_us * 1e6:.0f} prompt tokens/s per layer)")
    print(json.dumps({"metric": "paged prefill TFLOP/s", "value": round(tflops, 2), "unit": "TFLOP/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                      "us_per_layer": round(us, 2), "tokens_per_s_per_layer": round(T / us * 1e6, 1),
                      "prompt_path_us_per_layer": {"reshape_and_cache+prefill": round(two_us, 2),
                                                   "prefill_append": round(fused_us, 2)},
                      "dtype": "f16",
                      "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                                   "traffic": traffic_from_profiles("prefill") if D == 128 else None},
                      "config": {"workload": "prefill", "prompts": S, "tokens": T, "max_prompt": mq,
                                 "num_heads": H, "num_kv_heads": Hkv, "head_dim": D, "block_size": B,
                                 "layers_resident": L}}), flush=True)


def chunked_bench(args, dev):
    """Chunked prefill: a short chunk of new tokens per sequence over a long
    cached context, few sequences -- the shape that gives pa_prefill too few
    workgroups unless the context is split.  Two batches: 4 sequences x 8192
    cached tokens with 32 new each at Llama-2-7B heads (32 x 128), and 16 x
    4096 with 16 new each at 32 query / 8 KV heads; B = 16, --layers layers
    resident (default here 4).  K/V bytes = every cached token's K and V of
    every KV head, read once; the kernel is HBM-bound at these shapes (16-32
    new tokens per KV head: 4 x g x 128 x rows flops per 512 bytes)."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa

    L = args.layers if args.layers != 32 else 4
    B, D = args.block_size, 128
    results = []
    for S, n, m, H, Hkv in ((4, 8192, 32, 32, 32), (16, 4096, 16, 32, 8)):
        nbps = -(-n // B)
        NB = S * nbps + 8
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed)
        kcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
        vcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
        perm = np.random.default_rng(args.seed).permutation(NB)[:S * nbps].reshape(S, nbps).astype(np.int32)
        T = S * m
        q = torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float16)
        out = torch.empty_like(q)
        d_t = torch.from_numpy(perm).to(dev)
        d_l = torch.full((S,), n, dtype=torch.int32, device=dev)
        d_q = torch.arange(0, T + 1, m, dtype=torch.int32, device=dev)
        ws_n = pa.pa_prefill_workspace_size(T, S, H, Hkv, D, B, nbps, m)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def call(l, split=True):
            pa.pa_prefill(out, q, kcs[l], vcs[l], d_t, d_l, d_q, 1 / np.sqrt(D), max_query_len=m,
                          workspace=ws, split=split)

        timed = {}
        for split in (False, True):
            for _ in range(max(args.warmup, 3)):
                for l in range(L):
                    call(l, split)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps * L)]
            for i in range(args.steps):
                for l in range(L):
                    a, b = ev[i * L + l]
                    a.record()
                    call(l, split)
                    b.record()
            torch.cuda.synchronize()
            timed[split] = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        kv = S * n * Hkv * D * 2 * 2
        gbs = kv / timed[True] / 1e3
        log(f"[bench] chunked: {S} x {n} cached, {m} new, {H}/{Hkv} heads: {timed[True]:.1f} us split "
            f"({ws_n >> 20} MiB workspace) = {gbs:.0f} GB/s of K/V ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); "
            f"unsplit {timed[False]:.1f} us")
        results.append({"batch": f"{S}x{n}+{m}, {H}/{Hkv} heads", "us_split": round(timed[True], 2),
                        "us_unsplit": round(timed[False], 2), "kv_GB_s": round(gbs, 1)})
    best = results[0]
    print(json.dumps({"metric": "chunked prefill K/V GB/s (split context)", "value": best["kv_GB_s"],
                      "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": True, "dtype": "f16", "batches": results,
                      "roofline": {"bound": "hbm", "achieved": best["kv_GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(best["kv_GB_s"] / HBM_PEAK_GBS, 4), "traffic": None},
                      "config": {"workload": "chunked", "block_size": B, "head_dim": D, "layers_resident": L}}),
          flush=True)


def prefill_long_bench(args, dev):
    """Prefill of long full prompts: every token new, causal, at Llama-2-7B
    heads (32 x --head-dim, 128 by default; one batch at 32 query / 8 KV
    heads), B = 16, --layers
    layers resident (default here 4): 32 x 1024, 16 x 2048, 8 x 4096, 4 x
    8192 tokens -- the steady state of the prefill loop, next to the
    short-prompt mix of --workload prefill.  Flops as for that workload:
    4 x 128 x heads x (positions each token attends to)."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa

    L = args.layers if args.layers != 32 else 4
    B, D = args.block_size, args.head_dim
    results = []
    for S, n, H, Hkv in ((32, 1024, 32, 32), (16, 2048, 32, 32), (8, 4096, 32, 32), (4, 8192, 32, 32),
                         (8, 4096, 32, 8)):
        nbps = -(-n // B)
        NB = S * nbps + 8
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed)
        kcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
        vcs = [torch.randn((NB, Hkv, B, D), generator=g, device=dev, dtype=torch.float16) for _ in range(L)]
        perm = np.random.default_rng(args.seed).permutation(NB)[:S * nbps].reshape(S, nbps).astype(np.int32)
        T = S * n
        q = torch.randn((T, H, D), generator=g, device=dev, dtype=torch.float16)
        out = torch.empty_like(q)
        d_t = torch.from_numpy(perm).to(dev)
        d_l = torch.full((S,), n, dtype=torch.int32, device=dev)
        d_q = torch.arange(0, T + 1, n, dtype=torch.int32, device=dev)
        ws_n = pa.pa_prefill_workspace_size(T, S, H, Hkv, D, B, nbps, n)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def call(l):
            pa.pa_prefill(out, q, kcs[l], vcs[l], d_t, d_l, d_q, 1 / np.sqrt(D), max_query_len=n, workspace=ws)

        for _ in range(max(args.warmup, 3)):
            for l in range(L):
                call(l)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps * L)]
        for i in range(args.steps):
            for l in range(L):
                a, b = ev[i * L + l]
                a.record()
                call(l)
                b.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        flops = 4.0 * D * H * S * n * (n + 1) / 2
        tf = flops / us / 1e6
        log(f"[bench] prefill-long: {S} x {n} tokens, {H}/{Hkv} heads: {us:.1f} us = {tf:.1f} TFLOP/s "
            f"({100 * tf / MFMA_F16_PEAK_TFLOPS:.1f}% of dense fp16 MFMA peak)")
        results.append({"batch": f"{S}x{n}, {H}/{Hkv} heads", "us": round(us, 2), "TFLOP_s": round(tf, 1)})
    best = results[3]
    print(json.dumps({"metric": "paged prefill TFLOP/s, long full prompts", "value": best["TFLOP_s"],
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": True, "dtype": "f16", "batches": results,
                      "roofline": {"bound": "mfma", "achieved": best["TFLOP_s"], "peak": MFMA_F16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(best["TFLOP_s"] / MFMA_F16_PEAK_TFLOPS, 4),
                                   "traffic": None},
                      "config": {"workload": "prefill-long", "block_size": B, "head_dim": D, "layers_resident": L}}),
          flush=True)


def sweep_bench(args, dev):
    """Block-size sweep: 256 sequences with context = prompt (N(500, 150),
    clipped to [16, 2048]) + generated (U[1, 1024]) -- the length mix of the
    5688vip.com page's block-size experiment -- at the Llama-2-7B head shape,
    one set of token values laid out at B = 8, 16, 32, 64 (pool = the blocks
    the sequences need, tables a random permutation).  For each B: pa_decode
    timed with HIP events (K/V ~4.2 GB, far beyond the 256 MB MALL), KV GB/s,
    and the bytes the partly filled last blocks leave unused."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    w = workloads.block_size_sweep(seed=args.seed)
    S = len(w.lens)
    k, v = w.tokens(dev)
    q = w.query(dev)
    kv_tok = 2 * w.num_kv_heads * w.head_dim * 2
    logical = int(w.lens.astype(np.int64).sum()) * kv_tok
    res = {}
    for B in (8, 16, 32, 64):
        tables = w.perm_tables(B)
        NB = sum(len(t) for t in tables)
        bm = pa.BlockManager(NB, B)
        for s in range(S):
            bm.set_table(s, tables[s], int(w.lens[s]))
        slots = np.concatenate([bm.get_slots(s, 0, int(w.lens[s])) for s in range(S)])
        width = max(len(t) for t in tables)
        tab, lens = bm.get_tables(range(S), width)
        kc = torch.empty((NB, w.num_kv_heads, B, w.head_dim), dtype=torch.float16, device=dev)
        vc = torch.empty_like(kc)
        pa.pa_reshape_and_cache(k, v, torch.from_numpy(slots).to(dev), kc, vc)
        d_t, d_l = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
        ws = torch.zeros(max(1, pa.pa_decode_workspace_size(S, w.num_heads, w.num_kv_heads, w.head_dim, B,
                                                            width * B, 0)), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)

        def call():
            pa.pa_decode(out, q, kc, vc, d_t, d_l, w.scale, B, max_context_len=width * B, workspace=ws)

        for _ in range(max(args.warmup, 5)):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        waste = sum(len(t) * B - int(n) for t, n in zip(tables, w.lens)) * kv_tok
        res[B] = {"us": round(us, 2), "GB_s": round(logical / us / 1e3, 1),
                  "pct_hbm_peak": round(100 * logical / us / 1e3 / HBM_PEAK_GBS, 2),
                  "tail_waste_MB": round(waste / 1e6, 1), "table_entries": int(NB),
                  "partition": pa.pa_decode_default_partition(S, w.num_heads, w.num_kv_heads, w.head_dim, B,
                                                              width * B)}
        log(f"[bench] sweep B={B}: {us:.1f} us = {logical / us / 1e3:.0f} GB/s, tail waste {waste / 1e6:.1f} MB, "
            f"{NB} blocks")
        del kc, vc
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "paged-decode KV GB/s by block size", "value": res[16]["GB_s"], "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "higher_is_better": True, "by_block_size": res,
                      "kv_bytes_per_call": logical,
                      "config": {"workload": "block-size-sweep", "batch": S, "context": "N(500,150)+U[1,1024]",
                                 "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                                 "head_dim": w.head_dim}}), flush=True)


def sampling_bench(args, dev):
    """Parallel sampling with copy-on-write: one 1000-token prompt (63
    blocks, the last holding 8 tokens) forked into 32 samples; every step
    appends one token per sample through the block manager (step 0: 31
    copy-on-write pairs -> pa_copy_blocks), writes the 32 new K/V rows and
    decodes all 32 samples (one pa_decode_append; --fused 0: scatter, then
    decode) -- the lpnh.cn/news/2758356 section 4 scenario,
    Llama-2-7B heads, B = 16, one layer.  Reported: time per step, and the
    logical KV bytes the decodes attend over per second (shared prompt
    blocks counted once per sample; they are re-read from the caches)."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    w = workloads.parallel_sampling(seed=args.seed)
    NB, B, N = w.num_blocks, w.block_size, w.num_samples
    bm = pa.BlockManager(NB, B)
    kp, vp = w.prompt_tokens(dev)
    kc = torch.empty((NB, w.num_kv_heads, B, w.head_dim), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    pa.pa_reshape_and_cache(kp, vp, torch.from_numpy(bm.add_sequence(0, w.prompt_len)).to(dev), kc, vc)
    for c in range(1, N):
        bm.fork(0, c)
    seqs = list(range(N))
    width = workloads.ceil_div(w.prompt_len + w.steps, B)
    toks = [w.step_tokens(i, dev) for i in range(w.steps)]
    out = torch.empty_like(toks[0][0])
    ws = torch.zeros(max(1, pa.pa_decode_workspace_size(N, w.num_heads, w.num_kv_heads, w.head_dim, B, width * B,
                                                        0)), dtype=torch.uint8, device=dev)
    kv_tok = 2 * w.num_kv_heads * w.head_dim * 2
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    logical = 0
    ncow = 0
    for i in range(w.steps):
        q, key, val = toks[i]
        slots, pairs = bm.append_tokens(seqs)
        ncow += len(pairs)
        if len(pairs):
            pa.pa_copy_blocks([kc], [vc], torch.from_numpy(pairs).to(dev))
        tables, lens = bm.get_tables(seqs, width)
        if args.fused:                       # the new K/V written inside the decode call
            pa.pa_decode_append(out, q, key, val, kc, vc, torch.from_numpy(tables).to(dev),
                                torch.from_numpy(lens).to(dev), w.scale, B, max_context_len=width * B, workspace=ws)
        else:
            pa.pa_reshape_and_cache(key, val, torch.from_numpy(slots).to(dev), kc, vc)
            pa.pa_decode(out, q, kc, vc, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), w.scale,
                         B, max_context_len=width * B, workspace=ws)
        logical += int(lens.astype(np.int64).sum()) * kv_tok
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    used = NB - bm.num_free()
    log(f"[bench] sampling: {w.steps} steps of {N} samples in {wall * 1e3:.1f} ms ({wall / w.steps * 1e6:.1f} us "
        f"per step incl. host work), {ncow} copy-on-write pairs, {used} blocks at the end "
        f"({N * workloads.ceil_div(w.prompt_len + w.steps, B)} unshared); {logical / wall / 1e9:.0f} GB/s logical KV")
    print(json.dumps({"metric": "parallel-sampling decode step (COW), logical KV GB/s",
                      "value": round(logical / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": w.steps,
                      "higher_is_better": True, "us_per_step": round(wall / w.steps * 1e6, 2),
                      "cow_pairs": ncow, "blocks_at_end": used,
                      "blocks_unshared": N * workloads.ceil_div(w.prompt_len + w.steps, B),
                      "config": {"workload": "parallel-sampling", "samples": N, "prompt": w.prompt_len,
                                 "block_size": B, "num_heads": w.num_heads, "head_dim": w.head_dim,
                                 "fused": bool(args.fused)}}), flush=True)


def read_bench(args, dev):
    """Read-only streaming ceilings on this chip (include/pa_bench.h), timed
    like the decode call: a plain contiguous read of a 4 GiB buffer, one MiB
    per workgroup; and the Llama-2-7B decode batch's access pattern -- the K
    and V slabs of every block of every (sequence, KV head), scattered by the
    tables -- over --layers resident layers, with no arithmetic, on two
    batches: every context at 2048 tokens (the pattern's own ceiling: equal
    workgroups, all resident at once) and contexts U[1, 2048] (the headline
    batch, in index order).  Beside each, pa_decode on the same batch and
    layers (default partition, longest-first order computed once).  Each is
    timed with HIP events around --steps sweeps; GB/s from the median
    sweep."""
    import numpy as np
    import torch

    import paged_kv_cache_390_amd as pa
    import workloads

    B, L = args.block_size, args.layers
    S0 = args.batch or 64
    mixed = workloads.llama7b_decode(seed=args.seed, num_seqs=S0, block_size=B)
    uniform = workloads.llama7b_decode(seed=args.seed, num_seqs=S0, block_size=B, min_len=2048)
    H, Hkv, D, NB = mixed.num_heads, mixed.num_kv_heads, mixed.head_dim, mixed.num_blocks
    pools = [mixed.pool(l, dev) for l in range(L)]
    kv_tok = 2 * Hkv * D * 2

    def sweeps(call, per_sweep):
        for _ in range(max(args.warmup, 3)):
            for l in range(per_sweep):
                call(l)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            for l in range(per_sweep):
                call(l)
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) / 1e3 / per_sweep for i in range(args.steps)]

    def entry(nbytes, t):
        return {"bytes_per_call": nbytes, "us_per_call": stats_of(t, 1e6, 2),
                "GB_s": round(nbytes / statistics.median(t) / 1e9, 2)}

    res = {}
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    bsink = torch.empty(max(1, buf.numel() >> 20), dtype=torch.int32, device=dev)
    res["contiguous_read"] = entry(buf.numel(), sweeps(lambda l: pa.pa_bench_stream_read(buf, bsink), 1))
    del buf
    for name, w in (("uniform_2048", uniform), ("mixed_U1_2048", mixed)):
        S = len(w.lens)
        tables = torch.from_numpy(np.ascontiguousarray(w.perm_tables)).to(dev)
        lens = torch.from_numpy(w.lens).to(dev)
        width = tables.shape[1]
        q, _, _ = w.new_tokens(0, dev)
        out = torch.empty_like(q)
        ws = torch.empty(max(1, pa.pa_decode_workspace_size(S, H, Hkv, D, B, width * B, 0)), dtype=torch.uint8,
                         device=dev)
        order = pa.pa_decode_order(lens, width * B)
        sink = torch.empty(S * Hkv, dtype=torch.int32, device=dev)
        n = w.lens.astype(np.int64)
        res[f"block_pattern_read_{name}"] = entry(
            int((-(-n // B) * B).sum()) * kv_tok,
            sweeps(lambda l: pa.pa_bench_block_read(pools[l][0], pools[l][1], tables, lens, sink), L))
        res[f"decode_{name}"] = entry(
            int(n.sum()) * kv_tok,
            sweeps(lambda l: pa.pa_decode(out, q, pools[l][0], pools[l][1], tables, lens, w.scale, B,
                                          max_context_len=width * B, workspace=ws, seq_order=order), L))
    for k, r in res.items():
        log(f"[bench] {k}: {r['us_per_call']['median']} us per call (median) = {r['GB_s']} GB/s "
            f"({100 * r['GB_s'] / HBM_PEAK_GBS:.1f}% of peak)")
    ceiling = res["block_pattern_read_uniform_2048"]["GB_s"]
    print(json.dumps({"metric": "read-only streaming GB/s (same-chip ceiling for paged decode)",
                      "value": ceiling, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "higher_is_better": True, "dtype": "f16", "data": "synthetic",
                      "reads": res,
                      "decode_over_block_read": {
                          k: round(res[f"decode_{k}"]["GB_s"] / res[f"block_pattern_read_{k}"]["GB_s"], 4)
                          for k in ("uniform_2048", "mixed_U1_2048")},
                      "config": {"workload": "read-ceiling", "batch": S0, "block_size": B, "num_kv_heads": Hkv,
                                 "head_dim": D, "layers_resident": L}}), flush=True)


def tiny_bench(args, dev):
    """Latency of the tiny case (4 sequences of 1/5/12/50 tokens, block_size
    4, 2 heads x 16; sequence 2 on the 5688vip.com page's table [7, 3, 1]):
    pa_decode with each call between its own HIP events (launch included),
    and the fp64 oracle on one thread on the same inputs."""
    r = tiny_latency(dev, reps=max(args.steps, 20))
    log(f"[bench] tiny: pa_decode {r['gpu_us']['median']} us median ({r['gpu_us']['min']}..{r['gpu_us']['max']}), "
        f"oracle {r['oracle_us_1_thread']['median']} us")
    print(json.dumps({"metric": "paged-decode latency, tiny case", "value": r["gpu_us"]["median"], "unit": "us",
                      "n_gpus": 1, "steps": r["gpu_us"]["n"], "higher_is_better": False, "dtype": "f16",
                      "data": "synthetic", **r,
                      "config": {"workload": "tiny", "lens": [1, 5, 12, 50], "block_size": 4, "num_heads": 2,
                                 "head_dim": 16}}), flush=True)


if __name__ == "__main__":
    main()

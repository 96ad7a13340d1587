#!/usr/bin/env python3
"""Benchmark: one PagedAttention decode step on one MI355X.

A step is the whole hot path over one synthetic batch: the host allocator
appends one token per sequence (slot mapping), rebuilds the block tables,
context lengths and the longest-first launch order into a pinned staging
buffer that a GPU kernel uploads, the cache write stores the new tokens' K/V,
and paged decode attention (with its partition merge) runs over every
sequence's full context.  Inputs are resident in HBM before timing.

Default workload: the LLaMA-13B-shaped decode layer (128 sequences, 40 heads
of 128, bf16 KV, block 16, log-normal context lengths with median 600 clipped
to [16, 4096], 128 new tokens per step).

Prints one JSON line (metric, value = effective KV GB/s of the step, roofline
of the decode kernels, CPU-oracle baseline on a bounded sample).
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published


def _args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--shape", type=int, default=2,
                    help="decode shape index 0..4 (default 2), or 5 for the chunked-prefill step")
    ap.add_argument("--partition", type=int, default=-1, help="-1 auto, 0 single pass, else tokens")
    ap.add_argument("--path", choices=["auto", "valu", "mfma"], default="auto",
                    help="decode kernel: automatic choice, vector ALUs or matrix cores")
    ap.add_argument("--order", choices=["longest", "index"], default="longest",
                    help="launch order of the sequences handed to the decode kernel")
    ap.add_argument("--separate-write", action="store_true",
                    help="write the step's new tokens with its own cache-write launch instead "
                         "of the decode call that writes them (paged_attention_decode_write)")
    ap.add_argument("--serial-upload", action="store_true",
                    help="upload each step's tables on the compute stream instead of a side "
                         "stream overlapped with the previous step's attention")
    ap.add_argument("--upload-kernel", action="store_true",
                    help="decode steps: upload each step's tables with their own upload launch "
                         "(side stream, or --serial-upload) instead of within the previous step's "
                         "decode launch (paged_attention_decode_step / "
                         "paged_attention_decode_shared_prefix_step)")
    ap.add_argument("--staging-depth", type=int, default=8,
                    help="pinned staging buffers in flight (steps the host may run ahead)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-oracle sample budget")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode a batch with a shared prefix through "
                         "paged_attention_decode_shared_prefix_step (the prefix partition "
                         "computed once per tile of sharing sequences; "
                         "paged_attention_decode_shared_prefix with --upload-kernel)")
    ap.add_argument("--prefix-tokens", type=int, default=None,
                    help="length of the shared prefix of a batch with sharing (the GQA batch: "
                         "1024 as specified); sharers are drawn among longer sequences")
    ap.add_argument("--prefix-cache", action="store_true",
                    help="measure admitting requests that share a cached 2,000-token system "
                         "prompt, against the same requests computed in full")
    ap.add_argument("--swap", action="store_true",
                    help="measure preemption swapping instead: a quarter of the sequences "
                         "swapped out to pinned host memory and back, per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy a known number of cache blocks with the "
                         "library's block-copy kernel (a reference for HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_PREFIX", "WRITE_PREFIX", "OUT_JSON"),
                    default=None, help="HBM traffic per decode launch from two rocprofv3 --pmc runs "
                    "(FETCH_SIZE, WRITE_SIZE) of `bench.py --calibrate-copy`; PREFIX.log holds "
                    "each run's output")
    ap.add_argument("--summarize-profile", metavar="PREFIX", default=None,
                    help="print a summary of rocprofv3 csv output PREFIX_kernel_{stats,trace}.csv "
                         "(mean over the last --steps dispatches) and exit")
    return ap.parse_args()


def cpu_baseline(wl, tables, ctx, budget_s: float) -> dict:
    """Time the fp64 oracle on whole sequences of the same batch until the
    budget is spent; report its KV GB/s."""
    import oracle.attention as OA
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    s = wl.shape
    order = np.random.default_rng(0).permutation(s.num_seqs)
    done_bytes = done_tok = 0
    nseq = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:  # whole passes over the batch order
        for b in order:
            c = int(ctx[b])
            OA.paged_decode(wl.q[b:b + 1], wl.k_cache, wl.v_cache, tables[b:b + 1],
                            ctx[b:b + 1], s.scale, s.dtype)
            done_bytes += c * 2 * s.num_kv_heads * s.head_dim * s.elem_bytes
            done_tok += c
            nseq += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{nseq} sequence decodes drawn from the {s.num_seqs}-sequence batch "
                      f"(all {s.num_q_heads} heads each), {done_tok} context tokens, "
                      f"{dt:.1f} s, numpy fp64",
            "seq_tokens_per_s": round(done_tok / dt, 1)}


def summarize_profile(prefix: str, last: int) -> int:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run (csv output):
    the stats table, and per kernel the mean over its last ``last`` dispatches
    (the timed steps) from the trace."""
    import csv
    stats = list(csv.DictReader(open(prefix + "_kernel_stats.csv")))
    trace = list(csv.DictReader(open(prefix + "_kernel_trace.csv")))
    print("| kernel | calls | avg us | min us | max us | % time |")
    print("|---|---|---|---|---|---|")
    for r in stats:
        print(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.2f} |")
    print()
    print(f"Mean over the last {last} dispatches of each kernel (the timed steps):")
    print()
    by = {}
    for r in trace:
        by.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    for name, v in by.items():
        v.sort()
        d = np.array([x[1] for x in v[-last:]]) / 1e3
        print(f"- `{name[:110]}`: {d.mean():.2f} us (n={len(d)}, min {d.min():.2f}, max {d.max():.2f})")
    return 0


KERNEL_SOURCES = {
    "decode": ("decode.hip", "attn_common.h", "pkv_device.h"),
    "prefill": ("prefill.hip", "attn_common.h", "pkv_device.h"),
}


def kernel_source_hash(kind: str) -> str:
    """sha256 of the sources of the decode or the prefill kernels (a traffic
    record is valid only for the kernels it was measured on)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_292_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _bench_line(log_path: str) -> dict:
    for line in open(log_path, errors="replace"):
        if line.startswith('{"metric"'):
            return json.loads(line)
    raise RuntimeError(f"no bench JSON line in {log_path}")


def summarize_counters(fetch_prefix: str, write_prefix: str, last: int, out_json: str) -> int:
    """HBM bytes per decode launch from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for the block-copy kernel moving a known number of bytes."""
    import csv

    def per_kernel(prefix, counter):
        rows = [r for r in csv.DictReader(open(prefix + "_counter_collection.csv"))
                if r["Counter_Name"] == counter]
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(
                (int(r["Dispatch_Id"]), float(r["Counter_Value"]) * 1024.0))
        for v in by.values():
            v.sort()
        return by

    fetch = per_kernel(fetch_prefix, "FETCH_SIZE")
    write = per_kernel(write_prefix, "WRITE_SIZE")
    cal = _bench_line(fetch_prefix + ".log")["calibration_copy"]
    bench = _bench_line(fetch_prefix + ".log")

    def one(by, name_part):
        keys = [k for k in by if name_part in k]
        assert len(keys) == 1, (name_part, keys)
        return by[keys[0]]

    # the first block-copy dispatch is the calibration one (the later ones time it)
    f_factor = cal["bytes_read"] / one(fetch, "copy_blocks_kernel")[0][1]
    w_factor = cal["bytes_written"] / one(write, "copy_blocks_kernel")[0][1]
    kind = "prefill" if bench["config"].get("chunk_tokens") else "decode"
    parts = (["prefill_lds_kernel", "merge_prefill_kernel"] if kind == "prefill"
             else ["decode_", "reduce_partitions_kernel"])
    fetch_b = sum(np.mean([x[1] for x in v[-last:]]) for k, v in fetch.items()
                  if any(p in k for p in parts))
    write_b = sum(np.mean([x[1] for x in v[-last:]]) for k, v in write.items()
                  if any(p in k for p in parts))
    traffic = fetch_b * f_factor + write_b * w_factor
    rf = bench["roofline"]
    alg = rf.get("algorithmic_bytes_all_timed_launches", rf.get("algorithmic_bytes_per_launch"))
    rec = {"workload": bench["config"]["workload"], "decode_path": bench["config"].get("decode_path"),
           "kernel_source_sha256": kernel_source_hash(kind), "kernels": parts,
           "traffic_bytes_per_launch": int(traffic),
           "fetch_bytes_raw": int(fetch_b), "write_bytes_raw": int(write_b),
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round(traffic / alg, 4),
           "steps": bench["steps"], "warmup": bench["warmup"],
           # the launch configuration the counters were taken on
           "partition_size": bench["config"]["partition_size"],
           "upload": bench["config"].get("upload")}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return 0


def load_traffic(workload: str, path_name: str, kind: str):
    """Stored HBM traffic per launch for this workload, if it was measured on
    the current sources of its kernels; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_{path_name}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    return rec


def traffic_for(rec, partition_size: int, upload: str, prefill: bool, steps: int, warmup: int,
                alg_bytes: int):
    """HBM traffic per launch for this run from a stored counter record
    (``load_traffic``): None unless the record was taken with this run's
    partition size and (decode) upload placement; the record's own figure
    for the same step counts, else its traffic per algorithmic byte times
    this run's algorithmic bytes (other step counts read other contexts).
    Returns (traffic or None, note or None)."""
    if rec is None or rec.get("partition_size") != partition_size:
        return None, None
    if not prefill and rec.get("upload") != upload:
        return None, None
    if rec["steps"] == steps and rec["warmup"] == warmup:
        return rec["traffic_bytes_per_launch"], None
    return (int(round(rec["traffic_over_algorithmic"] * alg_bytes)),
            f"{rec['steps']}-step counter run, traffic/algorithmic {rec['traffic_over_algorithmic']}")


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, per direction, published


def read_ceiling(P, torch, buf, stream, achieved_gbs: float) -> dict:
    """What HBM delivers to a plain read stream on this GPU: the library's
    streaming-read kernel (the decode kernels' 16-byte non-temporal loads
    and nothing else) over ``buf`` (the K cache, far larger than the
    caches), best of a few grid sizes, 5 timed reads each after one warm-up;
    and the decode kernel's rate as a fraction of it."""
    cus = torch.cuda.get_device_properties(buf.device).multi_processor_count
    nbytes = buf.numel() * buf.element_size()
    best, best_wg = 0.0, 0
    for mult in (1, 2, 4, 8, 16):
        wg = cus * mult
        out = torch.empty(wg, dtype=torch.int32, device=buf.device)
        P.stream_read(buf, out, wg, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            P.stream_read(buf, out, wg, stream)
        e1.record(stream)
        e1.synchronize()
        gbs = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if gbs > best:
            best, best_wg = gbs, wg
    return {"GBps": round(best, 1), "frac": round(achieved_gbs / best, 4), "bytes": int(nbytes),
            "workgroups": best_wg, "kernel": "stream_read (16-byte non-temporal loads only)"}


def run_swap(args) -> int:
    """Swap round trips of the shape's batch: every step, the host allocator
    swaps a quarter of the sequences out (every 4th, shared blocks once),
    the swap kernel copies their blocks to the pinned host pool, then they
    are swapped back in to fresh device blocks.  Kernel times by HIP events
    on the launch stream; a contiguous runtime copy (DMA engine) of the same
    bytes in each direction is timed beside it for reference."""
    import torch
    import paged_kv_cache_292_amd as P
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.shape(args.shape)
    # headroom: blocks a swapped sequence shares with a resident one stay on
    # the device, and swap-in gives the swapped sequence fresh copies
    wl = W.make_workload(s, with_payload=False, extra_tokens=1024)
    B, Hkv, D, bs = s.num_seqs, s.num_kv_heads, s.head_dim, s.block_size
    tdt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    N = wl.num_blocks
    k_cache = torch.randn((N, bs, Hkv, D), device=dev).to(tdt)
    v_cache = torch.randn((N, bs, Hkv, D), device=dev).to(tdt)
    alloc = P.Allocator(N, bs, wl.free_order)
    alloc.replay(wl.ops)
    group = list(range(0, B, 4))
    nh = sum(alloc.num_blocks_of(g) for g in group)
    alloc.set_host_pool(nh)
    k_host = torch.empty((nh, bs, Hkv, D), dtype=tdt).pin_memory()
    v_host = torch.empty((nh, bs, Hkv, D), dtype=tdt).pin_memory()
    stream = torch.cuda.current_stream()
    block_bytes = bs * Hkv * D * s.elem_bytes
    t_out, t_in, h_out, h_in, moved = [], [], [], [], []
    for i in range(args.warmup + args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        t0 = time.perf_counter()
        po = alloc.swap_out(group)
        t1 = time.perf_counter()
        d_po = torch.from_numpy(po).to(dev)
        e[0].record(stream)
        P.swap_blocks(k_cache, v_cache, k_host, v_host, d_po, P.SWAP_OUT)
        e[1].record(stream)
        t2 = time.perf_counter()
        pi = alloc.swap_in(group)
        t3 = time.perf_counter()
        d_pi = torch.from_numpy(pi).to(dev)
        e[2].record(stream)
        P.swap_blocks(k_cache, v_cache, k_host, v_host, d_pi, P.SWAP_IN)
        e[3].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            t_out.append(e[0].elapsed_time(e[1]) * 1e-3)
            t_in.append(e[2].elapsed_time(e[3]) * 1e-3)
            h_out.append(t1 - t0)
            h_in.append(t3 - t2)
            moved.append(len(po))
    nbytes = 2 * int(np.mean(moved)) * block_bytes  # K and V, one direction
    # DMA reference: one contiguous runtime copy of the same bytes each way
    flat_h = k_host.view(-1).view(torch.uint8)[: nbytes // 2]
    flat_h2 = v_host.view(-1).view(torch.uint8)[: nbytes // 2]
    flat_d = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    flat_d2 = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    dma = {"h2d": [], "d2h": []}
    for i in range(args.warmup + args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        flat_d.copy_(flat_h, non_blocking=True)
        flat_d2.copy_(flat_h2, non_blocking=True)
        e[1].record(stream)
        e[2].record(stream)
        flat_h.copy_(flat_d, non_blocking=True)
        flat_h2.copy_(flat_d2, non_blocking=True)
        e[3].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            dma["h2d"].append(e[0].elapsed_time(e[1]) * 1e-3)
            dma["d2h"].append(e[2].elapsed_time(e[3]) * 1e-3)
    out_gbs = nbytes / float(np.mean(t_out)) / 1e9
    in_gbs = nbytes / float(np.mean(t_in)) / 1e9
    res = {
        "metric": "KV swap bandwidth: device <-> pinned host blocks, swap kernel",
        "value": round(2 * nbytes / (float(np.mean(t_out)) + float(np.mean(t_in))) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((float(np.mean(t_out)) + float(np.mean(t_in))) * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic (random cache contents; the shape's length mix and placement)",
        "config": {"workload": s.name, "num_seqs": B, "swapped_seqs": len(group),
                   "blocks_per_direction": int(np.mean(moved)), "block_bytes": block_bytes,
                   "bytes_per_direction": nbytes},
        "swap_out_GBps": round(out_gbs, 2), "swap_in_GBps": round(in_gbs, 2),
        "swap_out_us": round(float(np.mean(t_out)) * 1e6, 1),
        "swap_in_us": round(float(np.mean(t_in)) * 1e6, 1),
        "host_allocator_us": {"swap_out": round(float(np.mean(h_out)) * 1e6, 1),
                              "swap_in": round(float(np.mean(h_in)) * 1e6, 1)},
        "dma_reference_GBps": {"h2d": round(nbytes / float(np.mean(dma["h2d"])) / 1e9, 2),
                               "d2h": round(nbytes / float(np.mean(dma["d2h"])) / 1e9, 2)},
        "roofline": {"bound": "host link", "achieved": round(min(out_gbs, in_gbs), 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(min(out_gbs, in_gbs) / HOST_LINK_PEAK_GBS, 4), "traffic": None},
    }
    alloc.close()
    print(json.dumps(res), flush=True)
    return 0


def run_prefix_cache(args) -> int:
    """Admission of a batch of new requests that share a 2,000-token system
    prompt (16 requests of 2,000 + 512 tokens; LLaMA-13B attention shape: 40
    heads of 128, bf16, blocks of 16).  A step: the host allocator admits the
    batch (add_prompt), the tables and slots are uploaded, the cache write
    stores the computed tokens' K/V and chunked prefill runs their queries
    over the whole prompt; the batch is then freed (untimed).  With the prefix
    cache the system prompt's blocks stay cached between steps and only each
    request's own 512 tokens are computed; without it every token is."""
    import torch
    import paged_kv_cache_292_amd as P

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, bs, sys_len, own = 16, 40, 40, 128, 16, 2000, 512
    rng = np.random.default_rng(20)
    system = rng.integers(0, 32000, size=sys_len).astype(np.int32)
    L = sys_len + own
    # fresh own tokens for every request of every step (only the system
    # prompt repeats); the same prompts for both runs
    total = args.warmup + args.steps
    own_tokens = rng.integers(0, 32000, size=(total, B, own)).astype(np.int32)
    N = B * (-(-L // bs)) + 64
    k_cache = torch.randn((N, bs, Hkv, D), device=dev).to(torch.bfloat16)
    v_cache = torch.randn((N, bs, Hkv, D), device=dev).to(torch.bfloat16)
    new_k = torch.randn((B * L, Hkv, D), device=dev).to(torch.bfloat16)
    new_v = torch.randn((B * L, Hkv, D), device=dev).to(torch.bfloat16)
    q = torch.randn((B * L, Hq, D), device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    res = {}
    for share in (True, False):
        alloc = P.Allocator(N, bs)
        if share:
            alloc.enable_prefix_cache()
            alloc.add_prompt(10_000, system)  # the system prompt computed once, earlier
            alloc.free(10_000)                # its blocks stay cached in the free list
        mb = -(-L // bs) + 1
        slots = np.empty(B * L, dtype=np.int64)
        times, dev_times, computed = [], [], []
        for it in range(args.warmup + args.steps):
            prompts = [np.concatenate([system, own_tokens[it, i]]) for i in range(B)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            n_slots, counts = 0, []
            for i, pr in enumerate(prompts):
                sl, c = alloc.add_prompt(i, pr, slots_out=slots[n_slots:])
                counts.append(L - c)
                n_slots += len(sl)
            tables, ctx = alloc.build_block_tables(list(range(B)), mb)
            starts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
            d_slots = torch.from_numpy(slots[:n_slots]).to(dev, non_blocking=False)
            d_tab = torch.from_numpy(tables).to(dev)
            d_ctx = torch.from_numpy(ctx).to(dev)
            d_st = torch.from_numpy(starts).to(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            P.kv_reshape_and_cache(new_k[:n_slots], new_v[:n_slots], k_cache, v_cache, d_slots)
            T = int(starts[-1])
            P.paged_attention_prefill(out[:T], q[:T], d_st, max(counts), k_cache, v_cache, d_tab,
                                      d_ctx, L, 1.0 / np.sqrt(D), 0, None)
            e1.record(stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(B):
                alloc.free(i)
            if it >= args.warmup:
                times.append(t1 - t0)
                dev_times.append(e0.elapsed_time(e1) * 1e-3)
                computed.append(T)
        key = "with_prefix_cache" if share else "without_prefix_cache"
        step = float(np.mean(times))
        res[key] = {"step_ms": round(step * 1e3, 3),
                    "device_ms": round(float(np.mean(dev_times)) * 1e3, 3),
                    "computed_tokens_per_step": int(np.mean(computed)),
                    "prompt_tokens_per_s": round(B * L / step, 1),
                    "requests_per_s": round(B / step, 1)}
        if share:
            lk, ht, nc = alloc.prefix_cache_stats()
            res[key]["block_hit_rate"] = round(ht / max(lk, 1), 4)
        alloc.close()
    w, wo = res["with_prefix_cache"], res["without_prefix_cache"]
    line = {
        "metric": "prompt admission with a shared 2,000-token system prompt: prompt tokens/s",
        "value": w["prompt_tokens_per_s"], "unit": "prompt tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": w["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random tokens, K/V and queries)",
        "config": {"workload": "shared_system_prompt_bf16", "num_requests": B,
                   "system_prompt_tokens": sys_len, "own_tokens": own, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs},
        "with_prefix_cache": w, "without_prefix_cache": wo,
        "speedup": round(wo["step_ms"] / w["step_ms"], 2),
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    args = _args()
    if args.summarize_profile:
        return summarize_profile(args.summarize_profile, args.steps)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1],
                                  args.steps, args.summarize_counters[2])
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        return 2
    if args.swap:
        return run_swap(args)
    if args.prefix_cache:
        return run_prefix_cache(args)
    import torch
    import paged_kv_cache_292_amd as P
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P.set_decode_path({"auto": P.PATH_AUTO, "valu": P.PATH_VALU, "mfma": P.PATH_MFMA}[args.path])
    s = W.shape(args.shape)
    if args.prefix_tokens is not None:
        if not s.num_sharers:
            raise SystemExit("--prefix-tokens needs a batch with a shared prefix (--shape 3)")
        s = W.shape(args.shape, shared_prefix_tokens=args.prefix_tokens)
    total_steps = args.warmup + args.steps
    step_new = 1 if s.new_tokens else 0
    chunk = s.chunk  # > 0: a chunked-prefill step of this many tokens per sequence
    step_tok = chunk if chunk else step_new  # tokens each sequence gains per step
    # decode steps with new tokens write them inside the decode launch, and
    # (unless --upload-kernel) every decode launch also uploads the next
    # step's tables, which the host prepares one step ahead
    fused_write = bool(step_new) and not s.chunk and not args.separate_write
    in_step = ((fused_write or not (step_new or s.chunk))
               and not args.upload_kernel and not args.serial_upload)
    # growth room: in_step prepares one step more than it decodes
    wl = W.make_workload(s, extra_tokens=(total_steps + int(in_step)) * step_tok)
    B, Hq, Hkv, D, bs = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size
    dt_code = P.F32 if s.dtype == "f32" else P.BF16
    tdt = torch.float32 if s.dtype == "f32" else torch.bfloat16

    def up(a):
        if s.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    alloc = P.Allocator(wl.num_blocks, bs, wl.free_order)
    alloc.replay(wl.ops)
    seqs = np.arange(B, dtype=np.int64)
    final_ctx = wl.ctx + (total_steps - 1 + int(in_step)) * step_tok
    max_blocks = int(((final_ctx + bs - 1) // bs).max())
    max_ctx_final = int(final_ctx.max())

    q = up(wl.q)
    k_cache = up(wl.k_cache)
    v_cache = up(wl.v_cache)
    rows = B * chunk if chunk else B  # query rows per step
    out = torch.empty((rows, Hq, D), dtype=tdt, device=dev)
    new_k = new_v = None
    if step_tok:
        nks, nvs = [wl.new_k], [wl.new_v]
        for i in range(1, total_steps):
            k_, v_ = W.step_tokens(s, i)
            nks.append(k_)
            nvs.append(v_)
        new_k = up(np.stack(nks))
        new_v = up(np.stack(nvs))
    if chunk:
        ws_bytes = P.prefill_workspace_bytes(rows, Hq, D, max_ctx_final, args.partition)
        d_qstart = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * chunk).to(dev)
        chunk_counts = np.full(B, chunk, dtype=np.int32)
    else:
        if args.shared_prefix:
            if not s.num_sharers or step_new:
                raise SystemExit("--shared-prefix needs a batch with sharing and no new tokens")
            args.partition = s.shared_prefix_tokens  # partition 0 is the shared prefix
        ws_bytes = P.decode_workspace_bytes(B, Hq, Hkv, D, bs, max_ctx_final, args.partition,
                                            dt_code)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    shared = bool(args.shared_prefix) and not chunk
    if shared:  # the members, from the allocator's tables
        members, flag = alloc.shared_prefix_members(seqs, s.shared_prefix_tokens)
        d_members = torch.from_numpy(members).to(dev)
        d_member_flag = torch.from_numpy(flag).to(dev)
    part_used = (P.prefill_partition_size(B, chunk, Hq, Hkv, max_ctx_final, args.partition)
                 if chunk else
                 P.decode_partition_size(B, Hq, Hkv, D, bs, max_ctx_final, args.partition, dt_code))

    # One pinned staging buffer per in-flight step, laid out as the device
    # buffer it is copied to: slots int64 [B] | tables int32 [B, max_blocks] |
    # context lengths int32 [B].  One H2D copy per step.
    nbuf = args.staging_depth  # the host waits only for copies this many steps back
    n_slot_b, n_tab_b, n_ctx_b, n_ord_b = 8 * B * max(step_tok, 1), 4 * B * max_blocks, 4 * B, 4 * B
    stage_bytes = n_slot_b + n_tab_b + n_ctx_b + n_ord_b
    stage_bytes = (stage_bytes + 15) // 16 * 16
    h_stage = [torch.empty(stage_bytes, dtype=torch.uint8).pin_memory() for _ in range(nbuf)]
    h_flat = [hs.numpy() for hs in h_stage]
    host_flat = np.zeros(stage_bytes, dtype=np.uint8)  # ordinary memory, same layout
    host_sl = host_flat[:n_slot_b].view(np.int64)
    host_tb = host_flat[n_slot_b:n_slot_b + n_tab_b].view(np.int32).reshape(B, max_blocks)
    o_cx = n_slot_b + n_tab_b
    host_cx = host_flat[o_cx:o_cx + n_ctx_b].view(np.int32)
    host_ord = host_flat[o_cx + n_ctx_b:o_cx + n_ctx_b + n_ord_b].view(np.int32)
    # Two device staging buffers: step i's tables are uploaded on a side
    # stream while step i-1's attention still reads the other buffer (the
    # upload depends only on the host allocator, not on the previous step).
    d_stages = [torch.empty(stage_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]

    def stage_views(d):
        return (d[:n_slot_b].view(torch.int64),
                d[n_slot_b:n_slot_b + n_tab_b].view(torch.int32).view(B, max_blocks),
                d[o_cx:o_cx + n_ctx_b].view(torch.int32),
                d[o_cx + n_ctx_b:o_cx + n_ctx_b + n_ord_b].view(torch.int32))

    d_views = [stage_views(d) for d in d_stages]
    use_order = args.order == "longest"
    copied = [torch.cuda.Event() for _ in range(nbuf)]
    stream = torch.cuda.current_stream()
    up_stream = stream if args.serial_upload else torch.cuda.Stream()  # default priority
    up_done = [torch.cuda.Event() for _ in range(2)]
    att_done = [torch.cuda.Event() for _ in range(2)]
    new_k_steps = [new_k[i] for i in range(total_steps)] if step_tok else None
    new_v_steps = [new_v[i] for i in range(total_steps)] if step_tok else None

    # per-step algorithmic bytes of the decode call
    E = s.elem_bytes

    qrows = chunk if chunk else 1  # query rows per sequence

    def decode_bytes(ctx):
        """Unique K/V bytes of the step's sequences, and those plus q, out,
        tables, lengths and (partitioned) the partials written and read back."""
        kv = int(ctx.sum()) * 2 * Hkv * D * E
        nb = int(((ctx + bs - 1) // bs).sum())
        other = 2 * B * qrows * Hq * D * E + 4 * nb + 4 * B
        if fused_write:  # the new rows read from the input and written into the cache
            other += 2 * 2 * B * Hkv * D * E
        if in_step:  # the next step's arrays written into device memory
            other += stage_bytes
        if part_used > 0:
            if shared:  # members: the prefix, then partitions of max(2048, prefix)
                F = s.shared_prefix_tokens  # tokens; the others: max(2048, prefix)
                Pp = max(2048, F)
                np_ = np.where(flag != 0, np.where(ctx > F, 1 + (ctx - F + Pp - 1) // Pp, 1),
                               (ctx + Pp - 1) // Pp)
            else:
                np_ = (ctx + part_used - 1) // part_used
            multi = np_[np_ > 1].sum()
            other += int(multi) * qrows * Hq * (D + 2) * 4 * 2
        return kv, kv + other

    # HIP events bracket the attention call on every EVENT_EVERY-th step of
    # the timed region (each timing event adds a few microseconds of command
    # processing to the step it is recorded in)
    EVENT_EVERY = 4
    timed_ev = [i for i in range(args.warmup, total_steps) if (i - args.warmup) % EVENT_EVERY == 0]
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for i in timed_ev}
    ctx_hist = []
    host_s = []
    wait_s = []

    def step(i):
        t_w = time.perf_counter()
        j = i % nbuf
        if i >= nbuf:
            copied[j].synchronize()  # staging buffer j is free again
        t_h = time.perf_counter()
        wait_s.append(t_h - t_w)
        # The allocator writes into ordinary (cached) host memory; one bulk
        # copy then moves the step's slots, tables and lengths into the pinned
        # staging buffer, which is uncached and never read back by the host.
        cx = np.empty(B, np.int32)
        if chunk:
            alloc.append_tokens(seqs, chunk_counts, out=host_sl)
            alloc.build_block_tables(seqs, max_blocks, pad=-1, tables_out=host_tb, ctx_out=cx)
            maxc = int(cx.max())
            if use_order:
                host_ord[:] = P.longest_first_order(cx)
        elif step_new:
            maxc = alloc.decode_step_prepare(seqs, max_blocks, host_sl, host_tb, cx,
                                             order_out=host_ord if use_order else None)
        else:
            alloc.build_block_tables(seqs, max_blocks, pad=-1, tables_out=host_tb, ctx_out=cx)
            maxc = int(cx.max())
            if use_order:
                host_ord[:] = P.longest_first_order(cx)
        host_cx[:] = cx
        np.copyto(h_flat[j], host_flat)
        ds = i % 2
        d_slots, d_tables, d_ctx, d_order = d_views[ds]
        # one stream orders everything by itself; with a side stream, the
        # upload waits for the attention that last read its buffer and the
        # attention for the upload
        serial = up_stream is stream
        if i >= 2 and not serial:
            up_stream.wait_event(att_done[ds])  # step i-2's attention read this buffer
        P.upload_pinned(d_stages[ds], h_stage[j], stream=up_stream)
        copied[j].record(up_stream)
        if not serial:
            up_done[ds].record(up_stream)
            stream.wait_event(up_done[ds])
        if step_tok and not fused_write:
            P.kv_reshape_and_cache(new_k_steps[i], new_v_steps[i], k_cache, v_cache, d_slots)
        if i in ev:
            ev[i][0].record(stream)
        if chunk:
            P.paged_attention_prefill(out, q, d_qstart, chunk, k_cache, v_cache, d_tables, d_ctx,
                                      maxc, s.scale, args.partition, workspace,
                                      seq_order=d_order if use_order else None)
        elif fused_write:
            P.paged_attention_decode_write(out, q, new_k_steps[i], new_v_steps[i], k_cache,
                                           v_cache, d_tables, d_ctx, maxc, s.scale,
                                           args.partition, workspace,
                                           seq_order=d_order if use_order else None)
        elif shared:
            P.paged_attention_decode_shared_prefix(out, q, k_cache, v_cache, d_tables, d_ctx, maxc,
                                                   s.scale, d_members, d_member_flag,
                                                   s.shared_prefix_tokens, workspace,
                                                   seq_order=d_order if use_order else None)
        else:
            P.paged_attention_decode(out, q, k_cache, v_cache, d_tables, d_ctx, maxc, s.scale,
                                     args.partition, workspace,
                                     seq_order=d_order if use_order else None)
        if i in ev:
            ev[i][1].record(stream)
        if not serial:
            att_done[ds].record(stream)
        ctx_hist.append(cx)
        host_s.append(time.perf_counter() - t_h)

    # In-step upload: the host prepares step k's tables into pinned buffer
    # k % nbuf before step k - 1 is launched; step k - 1's decode launch copies
    # them into the device staging buffer that step k reads (the other one of
    # two), and the event after it frees the pinned buffer.  Per step: one
    # launch and one event, no second stream.
    prepared = {}

    def host_prepare(k):
        j = k % nbuf
        t_w = time.perf_counter()
        if k >= nbuf:
            copied[j].synchronize()  # the launch that copied this buffer's last contents
        t_h = time.perf_counter()
        cx = np.empty(B, np.int32)
        if step_new:
            maxc = alloc.decode_step_prepare(seqs, max_blocks, host_sl, host_tb, cx,
                                             order_out=host_ord if use_order else None)
        else:
            alloc.build_block_tables(seqs, max_blocks, pad=-1, tables_out=host_tb, ctx_out=cx)
            maxc = int(cx.max())
            if use_order:
                host_ord[:] = P.longest_first_order(cx)
        host_cx[:] = cx
        np.copyto(h_flat[j], host_flat)
        prepared[k] = (maxc, cx, time.perf_counter() - t_h, t_h - t_w)

    def step_in_step(i):
        host_prepare(i + 1)
        maxc, cx = prepared.pop(i)[:2]
        host_s.append(prepared[i + 1][2])  # this iteration's host work: the next step's
        wait_s.append(prepared[i + 1][3])
        ds = i % 2
        _, d_tables, d_ctx, d_order = d_views[ds]
        if i in ev:
            ev[i][0].record(stream)
        if shared:
            P.paged_attention_decode_shared_prefix_step(
                out, q, k_cache, v_cache, d_tables, d_ctx, maxc, s.scale, d_members,
                d_member_flag, s.shared_prefix_tokens, d_stages[1 - ds], h_stage[(i + 1) % nbuf],
                workspace, seq_order=d_order if use_order else None)
        else:
            nk, nv = (new_k_steps[i], new_v_steps[i]) if step_new else (None, None)
            P.paged_attention_decode_step(out, q, nk, nv, k_cache, v_cache,
                                          d_tables, d_ctx, maxc, s.scale, d_stages[1 - ds],
                                          h_stage[(i + 1) % nbuf], args.partition, workspace,
                                          seq_order=d_order if use_order else None)
        if i in ev:
            ev[i][1].record(stream)
        copied[(i + 1) % nbuf].record(stream)
        ctx_hist.append(cx)

    if in_step:  # step 0's tables: one upload before the first launch
        host_prepare(0)
        P.upload_pinned(d_stages[0], h_stage[0], stream=stream)
        copied[0].record(stream)
        step = step_in_step

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    K = args.steps
    timed = slice(args.warmup, total_steps)
    per_step = [decode_bytes(c.astype(np.int64)) for c in ctx_hist]
    kv_bytes = [x[0] for x in per_step]
    alg_bytes = [x[1] for x in per_step]
    ctx_tokens = [int(c.sum()) for c in ctx_hist]
    kv_t = sum(kv_bytes[timed])
    tok_t = sum(ctx_tokens[timed])
    dec_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in timed_ev])
    dec_avg_s = float(dec_ms.mean()) / 1e3
    alg_per_launch = float(np.mean([alg_bytes[i] for i in timed_ev]))  # the same launches
    achieved = alg_per_launch / dec_avg_s / 1e9
    value = kv_t / elapsed / 1e9

    # Unique K/V bytes of the last step (shared prefix blocks once): per
    # distinct physical block, the most rows any sequence reads from it.
    rows_of = {}
    last_ctx = ctx_hist[-1].astype(np.int64)
    for b in range(B):
        nb = int((last_ctx[b] + bs - 1) // bs)
        for k in range(nb):
            blk = int(host_tb[b, k])
            rows_of[blk] = max(rows_of.get(blk, 0), int(min(bs, last_ctx[b] - k * bs)))
    unique_ratio = sum(rows_of.values()) / max(1, int(last_ctx.sum()))
    res = {
        "metric": "paged decode attention: effective KV HBM GB/s (% of peak), seq-tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, seeded length mix and placement)",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(tok_t / elapsed, 1),
        "decode_tokens_per_s": round(B * K / elapsed, 1),
        "kv_unique_over_logical": round(unique_ratio, 4),
        "value_unique_GBps": round(value * unique_ratio, 2),
        "host_us_per_step": round(float(np.mean(host_s[timed])) * 1e6, 1),
        "host_wait_us_per_step": round(float(np.mean(wait_s[timed])) * 1e6, 1),
        "config": {
            "workload": s.name, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": bs, "mean_context": round(tok_t / K / B, 1),
            "max_context": int(wl.ctx.max()) + (total_steps - 1) * step_tok,
            "new_tokens_per_step": B * step_tok,
            "partition_size": part_used, "kv_bytes_per_step": int(kv_t // K),
            "decode_path": args.path, "launch_order": args.order, "chunk_tokens": chunk,
            "shared_prefix_decode": shared,
            "upload": ("within the previous step's decode launch" if in_step else
                       "own launch on the compute stream" if args.serial_upload else
                       "own launch on a side stream"),
            "shared_prefix_tokens": s.shared_prefix_tokens, "num_sharers": s.num_sharers,
        },
        "roofline": {
            "kernel": ("paged_attention_decode"
                       + ("_step (cache write and next upload fused)" if in_step and fused_write
                          else "_shared_prefix_step (next upload fused)" if in_step and shared
                          else "_step (next upload fused)" if in_step
                          else "_write (cache write fused)" if fused_write else "")
                       + (" (single pass)" if part_used == 0 else
                          " (shared prefix once per tile of members, partition kernel + "
                          "log-sum-exp merge)" if shared else
                          " (partition kernel + log-sum-exp merge)")),
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "avg_launch_us": round(dec_avg_s * 1e6, 2),
            "median_launch_us": round(float(np.median(dec_ms)) * 1e3, 2),
            "algorithmic_bytes_per_launch": int(alg_per_launch),
            "event_timed_launches": len(timed_ev),
            # over every timed launch (the counters average all of them)
            "algorithmic_bytes_all_timed_launches": int(np.mean(alg_bytes[timed])),
        },
    }
    if chunk:
        # prefill: attention flops (q.K and P.V, 2 flops per multiply-add) over
        # each query's visible tokens; a dense bf16 contraction on the matrix cores
        def flops(ctx):
            pos_sum = sum(int(c) * chunk - chunk * (chunk - 1) // 2 for c in ctx)
            return 4 * D * Hq * pos_sum
        fl = float(np.mean([flops(ctx_hist[i]) for i in timed_ev]))  # the timed launches
        tflops = fl / dec_avg_s / 1e12
        res["roofline"] = {
            "kernel": ("paged_attention_prefill (matrix-core kernel, single pass)" if part_used == 0
                       else "paged_attention_prefill (matrix-core partition kernel + merge)"),
            "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "avg_launch_us": round(dec_avg_s * 1e6, 2),
            "median_launch_us": round(float(np.median(dec_ms)) * 1e3, 2),
            "flops_per_launch": int(fl),
            "event_timed_launches": len(timed_ev),
            "kv_GBps_unique": round(achieved, 1),
            "algorithmic_bytes_per_launch": int(alg_per_launch),
            "algorithmic_bytes_all_timed_launches": int(np.mean(alg_bytes[timed])),
        }
        res["prefill_tokens_per_s"] = round(rows * K / elapsed, 1)
    # (counters are recorded for the ordinary decode path only, and apply
    # only to the partitioning and upload placement they were taken with)
    tr = None if shared else load_traffic(s.name, args.path, "prefill" if chunk else "decode")
    traffic, scaled_from = traffic_for(tr, part_used, res["config"]["upload"], bool(chunk),
                                       args.steps, args.warmup,
                                       res["roofline"]["algorithmic_bytes_per_launch"])
    res["roofline"]["traffic"] = traffic
    if scaled_from:
        res["roofline"]["traffic_scaled_from"] = scaled_from
    # a pool at least 1.5 times the 256 MB last-level cache: a repeated pass
    # over it evicts every line before its reuse, so the reads stream from HBM
    if not chunk and k_cache.numel() * k_cache.element_size() >= (384 << 20):
        res["roofline"]["read_ceiling"] = read_ceiling(P, torch, k_cache, stream,
                                                       res["roofline"]["achieved"])
    if args.calibrate_copy:
        # block i -> block N/2 + i for M blocks, K and V: M * block bytes read and
        # written per cache.  Done after timing; the cache contents are not used again.
        M = min(4096, wl.num_blocks // 2)
        pairs = torch.stack([torch.arange(M), torch.arange(M) + wl.num_blocks // 2], 1).to(dev)
        pairs = pairs.to(torch.int64)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        P.copy_blocks(k_cache, v_cache, pairs)  # the dispatch the counters calibrate on
        c0.record(stream)
        for _ in range(5):
            P.copy_blocks(k_cache, v_cache, pairs)
        c1.record(stream)
        torch.cuda.synchronize()
        nbytes = 2 * M * bs * Hkv * D * E
        res["calibration_copy"] = {"blocks": M, "bytes_read": nbytes, "bytes_written": nbytes,
                                   "copy_blocks_GBps": round(2 * nbytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        tb, cx = alloc.build_block_tables(seqs, max_blocks, pad=-1)
        # the oracle runs on the host copy of the pool as drawn (values differ from
        # the device only in the slots the timed steps overwrote; timing only)
        res["cpu_baseline"] = cpu_baseline(wl, tb, cx.astype(np.int64), args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    alloc.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

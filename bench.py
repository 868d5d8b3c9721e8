"""Benchmark of one paged-decode step on one MI355X.

A step is the whole hot path for one batch, over every layer: copy-on-write
block copies (when the allocator asked for any), the store of the step's new
K/V rows, and paged decode attention (balanced split kernel + merge).  The
block tables, slot mapping and context lengths come from the library's C++
allocator; its per-step host cost is timed separately (``host_step_us``) since
it runs on the CPU ahead of the GPU work.

Inputs are synthetic and resident in HBM before timing starts; every layer has
its own K/V cache so that the 256 MB last-level cache cannot serve re-reads.

Prints one JSON line.  ``value`` is the step's algorithmic HBM traffic divided
by its time (GB/s); ``roofline`` reports the decode call alone, timed with
HIP events around each call inside the timed region; ``cpu_baseline`` is the
fp64 CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload mha|mix|prefix|long_bs16|...]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "pa_decode achieved HBM GB/s (% of MI355X peak) + decode tokens/s, bs32 ctx2048"
PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E, AMD specification
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_382_amd", "csrc", "decode.hip")


# --------------------------------------------------------------------------
# algorithmic bytes (what the method must move, not what an implementation
# happens to move)
# --------------------------------------------------------------------------

def decode_bytes(lens, num_q_heads, num_kv_heads, head_dim, block_size):
    """K/V rows attended + q in + out + used table entries + context lengths."""
    lens = [int(x) for x in lens]
    kv = sum(lens) * num_kv_heads * head_dim * 2 * 2
    q_out = 2 * len(lens) * num_q_heads * head_dim * 2
    tables = sum(-(-L // block_size) for L in lens) * 4 + 4 * len(lens)
    return kv + q_out + tables


def store_bytes(num_tokens, num_kv_heads, head_dim):
    """Read the new K and V rows, write them to the cache, read the slots."""
    return 4 * num_tokens * num_kv_heads * head_dim * 2 + 4 * num_tokens


def copy_bytes(num_pairs, block_size, num_kv_heads, head_dim):
    """Read and write one whole block of K and of V per pair."""
    return num_pairs * 2 * 2 * block_size * num_kv_heads * head_dim * 2


def decode_flops(lens, num_q_heads, head_dim):
    return 4 * sum(int(x) for x in lens) * num_q_heads * head_dim


def kv_bytes_per_request(layers, hidden, tokens, bytes_per_element=2):
    """K and V of every layer for one request."""
    return 2 * layers * hidden * tokens * bytes_per_element


# --------------------------------------------------------------------------

def workload_by_name(name):
    if name in W.ALL:
        return W.ALL[name]
    if name.startswith("long_bs"):
        return W.long_workload(int(name[len("long_bs"):]))
    raise SystemExit(f"unknown workload {name}")


def describe(wl, plan):
    lens = list(plan.context_lens)
    return (f"{wl.name}: fp16, {wl.num_q_heads} query / {wl.num_kv_heads} KV heads, "
            f"head_dim {wl.head_dim}, batch {len(lens)}, context {min(lens)}..{max(lens)} "
            f"(sum {sum(lens)}), block {wl.block_size}, pool {wl.num_blocks} blocks, "
            f"{wl.layers} layers with distinct caches")


def source_digest():
    with open(DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(wl_name):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, or
    None when the decode kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"decode_{wl_name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("decode_source_sha256_16") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_step_cost(wl, reps=20):
    """Median / p99 microseconds of the allocator's per-step host work
    (append one slot per sequence + export tables and lengths)."""
    import paged_kv_cache_382_amd as pa
    # Same plan, with room for `reps` more tokens per sequence.
    extra = -(-reps // wl.block_size) + 1
    roomy = W.shrink(wl, num_blocks=wl.num_blocks + extra * wl.num_seqs,
                     max_blocks_per_seq=wl.max_blocks_per_seq + extra)
    alloc = pa.Allocator(roomy.num_blocks, roomy.block_size, roomy.max_blocks_per_seq,
                         W.free_order(roomy.num_blocks, wl.seed))
    plan = W.plan_for(roomy, alloc)
    ids = list(plan.seq_ids)
    lat = []
    for _ in range(reps):
        t0 = time.perf_counter()
        try:
            alloc.append_batch(ids)
        except pa.PaError:
            break
        alloc.export(ids, roomy.max_blocks_per_seq)
        lat.append((time.perf_counter() - t0) * 1e6)
    if not lat:
        return None
    return {"median": float(np.median(lat)), "p99": float(np.percentile(lat, 99)),
            "reps": len(lat)}


def cpu_baseline(wl, plan, kc0, vc0, q0, budget_s):
    """The fp64 oracle on the host cores: one layer, sequences taken in batch
    order until about ``budget_s`` seconds of work."""
    from threadpoolctl import threadpool_limits

    from oracle import decode_ref
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, 16)
    kh = kc0.cpu().numpy()
    vh = vc0.cpu().numpy()
    qh = q0.cpu().numpy()
    tables = np.asarray(plan.block_tables, dtype=np.int32)
    lens = np.asarray(plan.context_lens, dtype=np.int32)
    done, tokens, nbytes, elapsed = 0, 0, 0, 0.0
    with threadpool_limits(limits=threads):
        while elapsed < budget_s and done < 64 * len(lens):
            s = done % len(lens)
            t0 = time.perf_counter()
            decode_ref(qh[s:s + 1], kh, vh, tables[s:s + 1], lens[s:s + 1], wl.scale)
            elapsed += time.perf_counter() - t0
            done += 1
            tokens += int(lens[s])
            nbytes += decode_bytes(lens[s:s + 1], wl.num_q_heads, wl.num_kv_heads,
                                   wl.head_dim, wl.block_size)
    return {
        "value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, one layer of the same workload: {done} sequence "
                   f"decodes ({tokens} context tokens, batch order, repeating) in "
                   f"{elapsed:.2f} s"),
        "tokens_per_s_extrapolated": round(done / (elapsed * wl.layers), 4),
    }


def copy_probe(wl, dev, reps):
    """Copy blocks [0, NB/2) onto [NB/2, NB) in both caches, ``reps`` times.

    Each launch reads and writes exactly ``copy_bytes(NB/2, ...) / 2`` bytes;
    the HBM byte counters of this launch calibrate those of the decode kernel.
    """
    import torch

    import paged_kv_cache_382_amd as pa
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    kc = torch.zeros(shape, dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    half = wl.num_blocks // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).to(
        device=dev, dtype=torch.int32).contiguous()
    n = copy_bytes(half, wl.block_size, wl.num_kv_heads, wl.head_dim)
    pa.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        pa.pa_copy_blocks(kc, vc, pairs)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    print(json.dumps({"copy_probe": wl.name, "read_bytes": n // 2, "write_bytes": n // 2,
                      "launches": reps + 1, "us_per_launch": round(ms * 1e3, 3),
                      "gbps_read_plus_write": round(n / (ms * 1e-3) / 1e9, 2)}), flush=True)


def compaction_probe(wl, dev, reps):
    """Defragment a scattered pool and time the copies that compaction needs.

    The pool of ``wl`` is scattered by the seeded add/append/free trace, then
    every other surviving sequence is freed; the C++ allocator plans the
    compaction (timed on the host) and one many-pair ``pa_copy_blocks`` call
    moves the blocks of one layer's caches (timed with HIP events, ``reps``
    launches).  Each launch reads and writes ``copy_bytes(pairs, ...) / 2``
    bytes.
    """
    import torch

    import paged_kv_cache_382_amd as pa
    alloc = pa.Allocator(wl.num_blocks, wl.block_size, wl.max_blocks_per_seq,
                         W.free_order(wl.num_blocks, wl.seed))
    live = W.fragment_pool(alloc, wl.seed + 200, n_ops=10000,
                           max_tokens=min(8192, wl.max_blocks_per_seq * wl.block_size))
    for seq in live[::2]:
        alloc.free_seq(seq)
    used = alloc.stats()["used_blocks"]
    t0 = time.perf_counter()
    pairs = alloc.compact()
    host_ms = (time.perf_counter() - t0) * 1e3
    shape = (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)
    kc = torch.zeros(shape, dtype=torch.float16, device=dev)
    vc = torch.zeros_like(kc)
    pairs_dev = torch.from_numpy(np.ascontiguousarray(pairs)).to(dev)
    n = copy_bytes(len(pairs), wl.block_size, wl.num_kv_heads, wl.head_dim)
    pa.pa_copy_blocks(kc, vc, pairs_dev)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        pa.pa_copy_blocks(kc, vc, pairs_dev)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    gbps = n / (ms * 1e-3) / 1e9
    print(json.dumps({
        "compaction": wl.name, "used_blocks": used, "pairs": len(pairs),
        "host_plan_ms": round(host_ms, 3), "bytes_per_launch": n, "launches": reps + 1,
        "us_per_launch": round(ms * 1e3, 3), "gbps_read_plus_write": round(gbps, 2),
        "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mha")
    ap.add_argument("--splits", type=int, default=0,
                    help="pieces the decode work is cut into (0 = library default)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured as one HIP graph (reported under 'graph')")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run pa_copy_blocks over half the pool of one layer (a plain copy "
                         "of known size, for scaling the HBM byte counters) and exit")
    ap.add_argument("--compaction", action="store_true",
                    help="only plan a compaction of the scattered pool and time its block "
                         "copies for one layer, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus must be 1 (the library has no "
              "multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_382_amd as pa

    wl = workload_by_name(args.workload)
    layers = args.layers or wl.layers
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(wl, dev, max(args.steps, 1))
        return
    if args.compaction:
        compaction_probe(wl, dev, max(args.steps, 1))
        return

    alloc = pa.Allocator(wl.num_blocks, wl.block_size, wl.max_blocks_per_seq,
                         W.free_order(wl.num_blocks, wl.seed))
    plan = W.plan_for(wl, alloc)
    stats = alloc.stats()
    B = len(plan.seq_ids)
    lens = [int(x) for x in plan.context_lens]
    max_ctx = max(lens)
    hkv, hq, d, bs = wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.block_size

    shape = (wl.num_blocks, bs, hkv, d)
    caches = []
    for layer in range(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(wl.seed * 100000 + layer)
        kc = torch.randn(shape, generator=g, device=dev, dtype=torch.float16)
        vc = torch.randn(shape, generator=g, device=dev, dtype=torch.float16)
        caches.append((kc, vc))
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    q = torch.randn((layers, B, hq, d), generator=g, device=dev, dtype=torch.float16)
    k_new = torch.randn((layers, B, hkv, d), generator=g, device=dev, dtype=torch.float16)
    v_new = torch.randn((layers, B, hkv, d), generator=g, device=dev, dtype=torch.float16)
    out = torch.empty_like(q)
    tables = torch.from_numpy(np.ascontiguousarray(plan.block_tables, dtype=np.int32)).to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    slots = torch.tensor(list(plan.step_slots), dtype=torch.int32, device=dev)
    cows = torch.tensor([list(c) for c in plan.cow_pairs], dtype=torch.int32,
                        device=dev).reshape(-1, 2)
    desc = pa.CacheDesc(*shape)
    splits = args.splits                 # 0: the library's choice for this batch
    ws = pa.decode_workspace(desc, B, hq, splits, dev)

    def step(events=None):
        for layer in range(layers):
            kc, vc = caches[layer]
            if cows.numel():
                pa.pa_copy_blocks(kc, vc, cows)
            pa.pa_store_kvcache(k_new[layer], v_new[layer], slots, kc, vc)
            if events is not None:
                events[layer][0].record()
            pa.pa_decode(q[layer], kc, vc, tables, lens_d, wl.scale, out=out[layer],
                         max_context_len=max_ctx, num_splits=splits, workspace=ws)
            if events is not None:
                events[layer][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(layers)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(events[k])
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / args.steps
    dec_ms = [e[0].elapsed_time(e[1]) for row in events for e in row]
    dec_avg_ms = float(np.mean(dec_ms))

    graph = None
    if args.graph:
        g = pa.DecodeStepGraph(caches, q, k_new, v_new, slots, tables, lens_d, wl.scale, out,
                               cow_pairs=cows, max_context_len=max_ctx, num_splits=splits)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(args.steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        graph = gs.elapsed_time(ge) / args.steps

    n_dec = decode_bytes(lens, hq, hkv, d, bs)
    n_step = layers * (n_dec + store_bytes(B, hkv, d) + copy_bytes(len(plan.cow_pairs), bs, hkv, d))
    value = n_step / (step_ms * 1e-3) / 1e9
    achieved = n_dec / (dec_avg_ms * 1e-3) / 1e9
    traffic = counter_traffic(wl.name)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": describe(wl, plan),
            "batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": d, "block_size": bs,
            "context_min": min(lens), "context_max": max_ctx, "context_sum": sum(lens),
            "layers": layers, "num_splits": splits or "auto", "pool_blocks": wl.num_blocks,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "decode_tokens_per_s": round(B / (step_ms * 1e-3), 2),
        "decode_us_per_layer": round(dec_avg_ms * 1e3, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode (balanced split kernel + merge kernel)",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": n_dec,
            "flops_per_launch": decode_flops(lens, hq, d),
        },
        "allocator": {"utilisation": round(float(stats["utilisation"]), 4),
                      "internal_fragmentation": round(float(stats["internal_fragmentation"]), 5),
                      "shared_blocks": int(stats["shared_blocks"]),
                      "cow_pairs_this_step": len(plan.cow_pairs)},
        "host_step_us": host_step_cost(wl),
    }
    if graph is not None:
        result["graph"] = {"ms_per_step": round(graph, 4),
                           "value": round(n_step / (graph * 1e-3) / 1e9, 2),
                           "decode_tokens_per_s": round(B / (graph * 1e-3), 2)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, plan, caches[0][0], caches[0][1], q[0],
                                              args.cpu_budget)
    print(json.dumps(result, default=lambda o: o.item() if hasattr(o, "item") else str(o)),
          flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of one paged-decode step on one MI355X.

A step is the whole hot path for one batch, over every layer: copy-on-write
block copies (when the allocator asked for any), the store of the step's new
K/V rows, and paged decode attention (a balanced split kernel plus a merge
kernel, or one workgroup per (sequence, KV head) pair when that fills the
device or the contexts are short).  The
block tables, slot mapping and context lengths come from the library's C++
allocator; its per-step host cost is timed separately (``host_step_us``) since
it runs on the CPU ahead of the GPU work.

Inputs are synthetic and resident in HBM before timing starts; every layer has
its own K/V cache so that the 256 MB last-level cache cannot serve re-reads.

Prints one JSON line.  ``value`` is the step's algorithmic HBM traffic divided
by its time (GB/s); ``roofline`` reports the decode call alone, timed with
HIP events around each call inside the timed region; ``cpu_baseline`` is the
fp64 CPU oracle on a bounded sample of the same workload; ``graph`` times the
same step replayed as one captured HIP graph (``--no-graph`` skips it).

    python bench.py [--steps K] [--warmup W] [--workload mha|mix|prefix|long_bs16|...]

Other modes, each printing its own JSON line: ``--workload prefill_mha`` or
``prefill_gqa`` (chunked prefill: per layer the store of the chunk's rows and
causal chunk attention; ``roofline`` against the fp16 matrix peak),
``--compaction`` (block copies of a compaction plan) and ``--copy-probe``
(a plain copy of known size, for scaling the HBM byte counters).
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
PEAK_FP16_TFLOPS = 2500.0        # MI355X dense fp16 matrix peak, AMD specification
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_382_amd", "csrc", "decode.hip")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_382_amd", "csrc", "prefill.hip")


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


def prefill_flops(context_lens, chunk_lens, num_q_heads, head_dim):
    """Causal chunk attention: row j of a chunk of n rows in a context of L
    tokens sees L - n + j + 1 keys; 2 flops a key and dim for Q K^T and 2 for
    P V, per query head."""
    keys = 0
    for L, n in zip(context_lens, chunk_lens):
        L, n = int(L), int(n)
        keys += n * (L - n) + n * (n + 1) // 2
    return 4 * keys * num_q_heads * head_dim


def prefill_kv_bytes(context_lens, num_kv_heads, head_dim):
    """K and V rows of every context token, read once."""
    return sum(int(L) for L in context_lens) * num_kv_heads * head_dim * 2 * 2


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


def source_digest(path=None):
    with open(path or DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(wl_name, kind="decode"):
    """HBM bytes per launch of the ``kind`` kernel from committed rocprofv3
    counter runs, or None when that kernel's source changed since they were
    taken."""
    stem = wl_name if wl_name.startswith(kind + "_") else f"{kind}_{wl_name}"
    path = os.path.join(ROOT, "profiles", f"{stem}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = DECODE_SRC if kind == "decode" else PREFILL_SRC
    if rec.get(f"{kind}_source_sha256_16") != source_digest(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def counter_lds_conflicts(wl_name):
    """Share of the decode split kernel's LDS-active cycles stalled on bank
    conflicts, from the committed rocprofv3 counter pass, or None when the
    decode source changed since it was taken (or no pass exists)."""
    path = os.path.join(ROOT, "profiles", f"decode_{wl_name}_lds_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("decode_source_sha256_16") != source_digest(DECODE_SRC):
        return None
    return rec.get("lds_bank_conflict_share")


LAYOUT_NAMES = {"slot": "slot-major [block][token][head][dim]",
                "head": "head-major [block][head][token][dim]"}


def cache_shape(wl, layout):
    """Shape of one layer's K (or V) cache tensor in ``layout``."""
    if layout == "head":
        return (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    return (wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim)


def counter_stem(wl_name, layout):
    """Workload stem of the committed counter files for a layout (slot-major
    files carry no suffix)."""
    return wl_name if layout == "slot" else f"{wl_name}_head"


def pcts(xs):
    """p10 / median / p90 of a list of timings."""
    return {"p10": round(float(np.percentile(xs, 10)), 4), "median": round(float(np.median(xs)), 4),
            "p90": round(float(np.percentile(xs, 90)), 4)}


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


# The numerics bar of the decode output against the fp64 oracle (the tests
# assert it; here it is reported beside the measured errors).
PARITY_BAR = {"max_abs": 4e-3, "mean_abs": 5e-4, "rel_l2": 1e-3}


def parity_summary(diffs, refs):
    """max-abs, mean-abs and relative L2 of the GPU rows against the oracle's."""
    d = np.concatenate([x.ravel() for x in diffs])
    r = np.concatenate([x.ravel() for x in refs])
    out = {"max_abs": float(np.abs(d).max()), "mean_abs": float(np.abs(d).mean()),
           "rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-30))}
    out["within_bar"] = all(out[k] <= PARITY_BAR[k] for k in PARITY_BAR)
    out["bar"] = PARITY_BAR
    return out


def cpu_model():
    """The host CPU's model name (first ``model name`` line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, plan, kc0, vc0, q0, budget_s, out0=None, layout="slot", full_pass=False):
    """The fp64 oracle on the host cores: one layer, sequences taken in batch
    order until about ``budget_s`` seconds of work.  With ``out0`` (the GPU's
    output of the same layer) the first pass over the batch is also compared
    with it, row by row, and reported under ``parity``."""
    from threadpoolctl import threadpool_limits

    from oracle import decode_ref
    cores = len(os.sched_getaffinity(0))
    # The box grants one GPU's share of the host (16 cores) whatever the
    # affinity mask shows; the oracle's BLAS threads stay within that share.
    threads = min(cores, 16)
    kh = kc0.cpu().numpy()
    vh = vc0.cpu().numpy()
    qh = q0.cpu().numpy()
    gpu = out0.float().cpu().numpy().astype(np.float64) if out0 is not None else None
    diffs, refs = [], []
    tables = np.asarray(plan.block_tables, dtype=np.int32)
    lens = np.asarray(plan.context_lens, dtype=np.int32)
    done, tokens, nbytes, elapsed = 0, 0, 0, 0.0
    with threadpool_limits(limits=threads):
        while (elapsed < budget_s or (full_pass and done < len(lens))) and done < 64 * len(lens):
            s = done % len(lens)
            t0 = time.perf_counter()
            ref = decode_ref(qh[s:s + 1], kh, vh, tables[s:s + 1], lens[s:s + 1], wl.scale,
                             layout=layout)
            elapsed += time.perf_counter() - t0
            if gpu is not None and done < len(lens):
                diffs.append(gpu[s] - ref[0])
                refs.append(ref[0])
            done += 1
            tokens += int(lens[s])
            nbytes += decode_bytes(lens[s:s + 1], wl.num_q_heads, wl.num_kv_heads,
                                   wl.head_dim, wl.block_size)
    result = {
        "value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
        "affinity_cores": cores, "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, one layer of the same workload: {done} sequence "
                   f"decodes ({tokens} context tokens, batch order, repeating) in "
                   f"{elapsed:.2f} s"),
        "tokens_per_s_extrapolated": round(done / (elapsed * wl.layers), 4),
        "seconds_per_layer_extrapolated": round(elapsed / done * len(lens), 4),
    }
    if diffs:
        result["parity"] = dict(parity_summary(diffs, refs), sequences=len(diffs),
                                compared="layer 0 output of the timed steps, fp16, against the oracle")
    return result


def read_ceiling(buffers, reps):
    """The streaming-read rate of the device on the given resident buffers:
    ``pa_read_probe`` over each, ``reps`` times, timed with HIP events; the
    median launch is reported."""
    import torch

    from paged_kv_cache_382_amd import probe
    sink = torch.zeros(1, dtype=torch.int32, device=buffers[0].device)
    for b in buffers:
        probe.pa_read_probe(b, sink)
    torch.cuda.synchronize()
    times, nbytes = [], []
    for _ in range(reps):
        for b in buffers:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            probe.pa_read_probe(b, sink)
            e1.record()
            times.append((e0, e1))
            nbytes.append(b.numel() * b.element_size())
    torch.cuda.synchronize()
    rates = [n / (a.elapsed_time(b) * 1e-3) / 1e9 for n, (a, b) in zip(nbytes, times)]
    return {"gbps": round(float(np.median(rates)), 2), "bytes_per_launch": int(nbytes[0]),
            "launches": len(rates), "kernel": "read_probe_kernel (pa_read_probe: 16-byte "
            "non-temporal loads, one contiguous range per workgroup)"}


def mfma_ceiling(dev, reps):
    """The fp16 matrix-core rate the device sustains: ``pa_mfma_probe`` with
    two 8-wave workgroups per compute unit (all resident), ``reps`` launches
    timed with HIP events; the median launch is reported, with the check that
    every product ran (the probe's sink stays 0)."""
    import torch

    from paged_kv_cache_382_amd import probe
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 8192
    probe.pa_mfma_probe(sink, wgs, iters)
    torch.cuda.synchronize()
    times, flops = [], 0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = probe.pa_mfma_probe(sink, wgs, iters)
        e1.record()
        times.append((e0, e1))
    torch.cuda.synchronize()
    rates = [flops / (a.elapsed_time(b) * 1e-3) / 1e12 for a, b in times]
    return {"tflops": round(float(np.median(rates)), 2), "flops_per_launch": flops, "launches": reps,
            "products_checked": int(sink.item()) == 0,
            "kernel": (f"mfma_probe_kernel (pa_mfma_probe: {wgs} workgroups x 8 waves, four "
                       "independent v_mfma_f32_32x32x16_f16 chains per wave)")}


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


def prefill_cpu_baseline(wl, kc, vc, q, tables, lens, chunk, budget_s, out0=None, layout="slot"):
    """The oracle timed on the host: causal rows of the first sequence's
    chunk, each row being single-query attention over its prefix (the
    reduction the prefill oracle is pinned to), until ``budget_s`` passes.
    With ``out0`` (the GPU's output rows of the same layer) every computed row
    is also compared with it and reported under ``parity``."""
    import torch

    from oracle import prefill_ref
    threads = torch.get_num_threads()
    bs = wl.block_size
    L = int(lens[0])
    nb = -(-L // bs)
    row = np.asarray(tables[0][:nb], dtype=np.int64)
    k_host = kc[torch.from_numpy(row).to(kc.device)].cpu().numpy()
    v_host = vc[torch.from_numpy(row).to(vc.device)].cpu().numpy()
    q_host = q[:chunk].cpu().numpy()
    local = np.arange(nb, dtype=np.int32)[None, :]
    gpu = out0[:chunk].float().cpu().numpy().astype(np.float64) if out0 is not None else None
    diffs, refs = [], []
    done, flops, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < chunk:
        j = done
        pos = L - chunk + j
        ref = prefill_ref(q_host[j:j + 1], k_host, v_host, local, [pos + 1], [0, 1], wl.scale,
                          layout=layout)
        flops += 4 * (pos + 1) * wl.num_q_heads * wl.head_dim
        if gpu is not None:
            diffs.append(gpu[j] - ref[0])
            refs.append(ref[0])
        done += 1
    elapsed = time.perf_counter() - t0
    result = {
        "value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
        "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: {done} causal rows (all {wl.num_q_heads} query heads) "
                   f"of one sequence's chunk, one layer, in {elapsed:.2f} s"),
    }
    if diffs:
        result["parity"] = dict(parity_summary(diffs, refs), rows=len(diffs),
                                compared="layer 0 output rows of the timed steps, fp16, against the oracle")
    return result


def prefill_main(args, wl, dev):
    """Chunked prefill step: per layer, store the chunk's K/V rows, then causal
    attention of every chunk row over its context."""
    import torch

    import paged_kv_cache_382_amd as pa
    layers = args.layers or wl.layers
    chunk, ctx = W.PREFILL_CHUNK, W.PREFILL_CONTEXT
    B, hq, hkv, d, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    alloc = pa.Allocator(wl.num_blocks, bs, wl.max_blocks_per_seq,
                         W.free_order(wl.num_blocks, wl.seed))
    slots = []
    for s in range(B):
        sl = alloc.add_seq(s, ctx)
        slots += list(sl[ctx - chunk:])
    tables_h, lens_h = alloc.export(list(range(B)), wl.max_blocks_per_seq)
    shape = cache_shape(wl, args.layout)
    caches = []
    for layer in range(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(wl.seed * 100000 + layer)
        caches.append((torch.randn(shape, generator=g, device=dev, dtype=torch.float16),
                       torch.randn(shape, generator=g, device=dev, dtype=torch.float16)))
    T = B * chunk
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    q = torch.randn((layers, T, hq, d), generator=g, device=dev, dtype=torch.float16)
    k_new = torch.randn((layers, T, hkv, d), generator=g, device=dev, dtype=torch.float16)
    v_new = torch.randn((layers, T, hkv, d), generator=g, device=dev, dtype=torch.float16)
    out = torch.empty_like(q)
    tables = torch.from_numpy(np.ascontiguousarray(tables_h)).to(dev)
    lens_d = torch.from_numpy(np.ascontiguousarray(lens_h)).to(dev)
    starts = torch.arange(0, T + 1, chunk, dtype=torch.int32, device=dev)
    slots_d = torch.tensor(slots, dtype=torch.int32, device=dev)

    def step(events=None):
        for layer in range(layers):
            kc, vc = caches[layer]
            pa.pa_store_kvcache(k_new[layer], v_new[layer], slots_d, kc, vc, layout=args.layout)
            if events is not None:
                events[layer][0].record()
            pa.pa_prefill(q[layer], kc, vc, tables, lens_d, starts, wl.scale, out=out[layer],
                          max_query_len=chunk, max_context_len=ctx, layout=args.layout)
            if events is not None:
                events[layer][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(layers)] for _ in range(args.steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for k in range(args.steps):
        step(events[k])
        marks[k + 1].record()
    torch.cuda.synchronize()
    step_ms = marks[0].elapsed_time(marks[-1]) / args.steps
    step_each = [marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)]
    pf_each = [e[0].elapsed_time(e[1]) for row in events for e in row]
    pf_ms = float(np.mean(pf_each))
    lens = [int(x) for x in lens_h]
    flops = prefill_flops(lens, [chunk] * B, hq, d)
    value = layers * flops / (step_ms * 1e-3) / 1e12
    achieved = flops / (pf_ms * 1e-3) / 1e12
    result = {
        "metric": "chunked-prefill attention TFLOP/s (causal, fp16 in, fp32 accumulate)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
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
            "workload": (f"{wl.name}: {B} sequences, each prefilling the last {chunk}-token chunk "
                         f"of a {ctx}-token prompt; {hq}/{hkv} heads, head_dim {d}, block {bs}"),
            "chunk": chunk, "context": ctx, "layers": layers, "pool_blocks": wl.num_blocks,
            "cache_layout": LAYOUT_NAMES[args.layout],
            "parallelism": "single GPU",
        },
        "prefill_tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "prefill_us_per_layer": round(pf_ms * 1e3, 3),
        "step_ms_percentiles": pcts(step_each),
        "prefill_us_percentiles": pcts([x * 1e3 for x in pf_each]),
        "roofline": {
            "bound": "mfma",
            "kernel": "pa_prefill ({})".format("prefill_lds_kernel" if bs >= 16 else "prefill_kernel"),
            "achieved": round(achieved, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
            "traffic": counter_traffic(counter_stem(wl.name, args.layout), "prefill"),
            "flops_per_launch": flops,
            "algorithmic_bytes_per_launch": prefill_kv_bytes(lens, hkv, d) + 2 * T * hq * d * 2,
        },
    }
    if not args.no_mfma_ceiling:
        ceiling = mfma_ceiling(dev, 5)
        result["mfma_ceiling"] = ceiling
        result["roofline"]["frac_of_mfma_ceiling"] = round(achieved / ceiling["tflops"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(wl, caches[0][0], caches[0][1], q[0],
                                                      tables_h, lens_h, chunk, args.cpu_budget,
                                                      out0=out[0], layout=args.layout)
    print(json.dumps(result), flush=True)


def unique_kv_rows(block_tables, lens, block_size):
    """Distinct (physical block, row) cache slots the batch attends to."""
    seen = set()
    for row, L in zip(block_tables, lens):
        L = int(L)
        for p in range(L):
            seen.add(int(row[p // block_size]) * block_size + p % block_size)
    return len(seen)


def time_decode_only(wl, st, layout, splits, steps, warmup):
    """pa_decode alone over every layer, ``steps`` times, HIP events around
    each call; for comparing partitions of the same batch."""
    import torch

    import paged_kv_cache_382_amd as pa
    caches, q, out = st["caches"], st["q"], st["out"]
    desc = st["desc"]
    B = q.shape[1]
    ws = pa.decode_workspace(desc, B, q.shape[2], splits, q.device)
    max_ctx = max(st["lens"])

    def run(ev=None):
        for layer, (kc, vc) in enumerate(caches):
            if ev is not None:
                ev[layer][0].record()
            pa.pa_decode(q[layer], kc, vc, st["tables"], st["lens_d"], wl.scale, out=out[layer],
                         max_context_len=max_ctx, num_splits=splits, workspace=ws, layout=layout)
            if ev is not None:
                ev[layer][1].record()

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in caches] for _ in range(steps)]
    for k in range(steps):
        run(evs[k])
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for row in evs for a, b in row]
    n_dec = decode_bytes(st["lens"], wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size)
    achieved = n_dec / (float(np.mean(ms)) * 1e-3) / 1e9
    return {"num_splits": {0: "auto", -1: "whole pairs"}.get(splits, splits),
            "decode_us_percentiles": pcts([x * 1e3 for x in ms]),
            "achieved": round(achieved, 2), "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "kernel": decode_kernel_label(splits, B, max_ctx)}


def run_decode(wl, dev, layout="slot", splits_arg=0, steps=20, warmup=3, layers=None,
               do_graph=True, do_ceiling=True, cpu_budget=15.0):
    """One decode workload: plan with the C++ allocator, build the caches,
    time ``steps`` steps of every layer (HIP events around each step and each
    pa_decode call), then the optional graph replay, read ceiling and CPU
    oracle.  Returns the result dict (the JSON line's fields) and the state
    the caller may reuse."""
    import torch

    import paged_kv_cache_382_amd as pa
    layers = layers or wl.layers
    alloc = pa.Allocator(wl.num_blocks, wl.block_size, wl.max_blocks_per_seq,
                         W.free_order(wl.num_blocks, wl.seed))
    plan = W.plan_for(wl, alloc)
    stats = alloc.stats()
    B = len(plan.seq_ids)
    lens = [int(x) for x in plan.context_lens]
    max_ctx = max(lens)
    hkv, hq, d, bs = wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.block_size

    shape = cache_shape(wl, layout)
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
    desc = pa.cache_desc(caches[0][0], layout)
    # 0: the library's own partition for this batch.  No hint is passed for
    # equal lengths: one workgroup per pair (-1) measured slower on mha than
    # the default of two workgroups a compute unit, each taking two whole pairs.
    splits = splits_arg
    ws = pa.decode_workspace(desc, B, hq, splits, dev)

    def step(events=None):
        for layer in range(layers):
            kc, vc = caches[layer]
            if cows.numel():
                pa.pa_copy_blocks(kc, vc, cows, layout=layout)
            pa.pa_store_kvcache(k_new[layer], v_new[layer], slots, kc, vc, layout=layout)
            if events is not None:
                events[layer][0].record()
            pa.pa_decode(q[layer], kc, vc, tables, lens_d, wl.scale, out=out[layer],
                         max_context_len=max_ctx, num_splits=splits, workspace=ws,
                         layout=layout)
            if events is not None:
                events[layer][1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(layers)] for _ in range(steps)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for k in range(steps):
        step(events[k])
        marks[k + 1].record()
    torch.cuda.synchronize()
    step_ms = marks[0].elapsed_time(marks[-1]) / steps
    step_each = [marks[k].elapsed_time(marks[k + 1]) for k in range(steps)]
    dec_ms = [e[0].elapsed_time(e[1]) for row in events for e in row]
    dec_avg_ms = float(np.mean(dec_ms))

    graph = None
    if do_graph:
        g = pa.DecodeStepGraph(caches, q, k_new, v_new, slots, tables, lens_d, wl.scale, out,
                               cow_pairs=cows, num_splits=splits,
                               layout=layout)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        graph = gs.elapsed_time(ge) / steps

    ceiling = None
    if do_ceiling:
        # Caches smaller than 1 GiB would be read from the 256 MB last-level
        # cache: probe a dedicated 2 GiB buffer instead.
        big = caches[0][0].numel() * 2 >= 1 << 30
        probe_bufs = list(caches[0]) if big else [torch.empty(1 << 30, dtype=torch.float16, device=dev)]
        ceiling = read_ceiling(probe_bufs, 5)
        ceiling["buffers"] = "layer 0's K and V caches" if big else "a dedicated 2 GiB buffer"
        del probe_bufs

    n_dec = decode_bytes(lens, hq, hkv, d, bs)
    n_step = layers * (n_dec + store_bytes(B, hkv, d) + copy_bytes(len(plan.cow_pairs), bs, hkv, d))
    value = n_step / (step_ms * 1e-3) / 1e9
    achieved = n_dec / (dec_avg_ms * 1e-3) / 1e9
    traffic = counter_traffic(counter_stem(wl.name, layout))
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
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
            "layers": layers,
            "num_splits": {0: "auto", -1: "whole pairs"}.get(splits, splits),
            "pool_blocks": wl.num_blocks,
            "cache_layout": LAYOUT_NAMES[layout],
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "decode_tokens_per_s": round(B / (step_ms * 1e-3), 2),
        "decode_us_per_layer": round(dec_avg_ms * 1e3, 3),
        "step_ms_percentiles": pcts(step_each),
        "decode_us_percentiles": pcts([x * 1e3 for x in dec_ms]),
        "roofline": {
            "bound": "hbm",
            "kernel": decode_kernel_label(splits, B, max_ctx),
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
    if traffic is not None:
        result["roofline"]["traffic_over_algorithmic"] = round(traffic / n_dec, 4)
    lds = counter_lds_conflicts(counter_stem(wl.name, layout))
    if lds is not None:
        result["roofline"]["lds_bank_conflict_share"] = lds
    if ceiling is not None:
        result["read_ceiling"] = ceiling
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbps"], 4)
    if graph is not None:
        result["graph"] = {"ms_per_step": round(graph, 4),
                           "value": round(n_step / (graph * 1e-3) / 1e9, 2),
                           "decode_tokens_per_s": round(B / (graph * 1e-3), 2)}
    if cpu_budget != 0:
        # cpu_budget < 0: one pass over the batch only (every sequence's rows
        # compared with the oracle), no timing budget beyond it.
        result["cpu_baseline"] = cpu_baseline(wl, plan, caches[0][0], caches[0][1], q[0],
                                              max(cpu_budget, 0.0), out0=out[0], layout=layout,
                                              full_pass=True)
    if wl.name == "prefix":
        # Shared prefix blocks are read by every sequence but stored once:
        # report the bytes the method names (every attended row, "logical")
        # beside the bytes of distinct cache rows ("unique") and a rate for each.
        uniq = unique_kv_rows(plan.block_tables, lens, bs)
        n_unique = (uniq * hkv * d * 2 * 2 + 2 * B * hq * d * 2
                    + sum(-(-L // bs) for L in lens) * 4 + 4 * B)
        result["prefix_bytes"] = {
            "logical_bytes_per_launch": n_dec, "unique_bytes_per_launch": n_unique,
            "logical_gbps": round(achieved, 2),
            "unique_gbps": round(n_unique / (dec_avg_ms * 1e-3) / 1e9, 2),
            "distinct_rows": int(uniq), "attended_rows": int(sum(lens)),
            "note": "logical: every attended K/V row counted once per sequence (the method's bytes); "
                    "unique: each distinct cache row counted once (the shared blocks are re-read "
                    "from the last-level cache)"}
    return result, {"caches": caches, "q": q, "out": out, "tables": tables, "lens_d": lens_d,
                    "lens": lens, "plan": plan, "splits": splits, "ws": ws, "desc": desc}

# Longest context for which the library's automatic choice (num_splits 0) runs
# one workgroup per (sequence, KV head) pair, for batches of at most 64.
WHOLE_PAIR_MAX_TOKENS = 512


def decode_kernel_label(splits, batch, max_ctx):
    """Which decode kernels one pa_decode call launches for this partition."""
    whole = splits == -1 or (splits == 0 and batch <= 64 and max_ctx <= WHOLE_PAIR_MAX_TOKENS)
    if whole:
        return "pa_decode (one workgroup per (sequence, KV head) pair; no merge kernel)"
    return "pa_decode (balanced split kernel + merge kernel)"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mha")
    ap.add_argument("--layout", choices=sorted(LAYOUT_NAMES), default="slot",
                    help="cache layout: slot-major [block][token][head][dim] (default) or "
                         "head-major [block][head][token][dim]")
    ap.add_argument("--splits", type=int, default=0,
                    help="pieces the decode work is cut into (0 = library default)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read probe on layer 0's caches")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="prefill: skip timing the matrix-core probe")
    ap.add_argument("--no-whole-pair", dest="with_whole_pair", action="store_false",
                    help="with mha at the default partition, skip timing one workgroup per pair beside it")
    ap.add_argument("--no-mix", dest="with_mix", action="store_false",
                    help="with the default mha workload, skip the second measured configuration "
                         "(mixed context lengths, reported under 'mix')")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip timing the step captured as one HIP graph (reported under 'graph')")
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

    dev = torch.device("cuda", 0)
    if args.workload in W.PREFILLS:
        torch.cuda.set_device(dev)
        prefill_main(args, W.PREFILLS[args.workload], dev)
        return
    wl = workload_by_name(args.workload)
    layers = args.layers or wl.layers
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(wl, dev, max(args.steps, 1))
        return
    if args.compaction:
        compaction_probe(wl, dev, max(args.steps, 1))
        return

    result, st = run_decode(wl, dev, args.layout, args.splits, args.steps, args.warmup, layers,
                            args.graph, not args.no_read_ceiling,
                            0.0 if args.no_cpu_baseline else args.cpu_budget)
    if wl.name == "mha" and args.splits == 0 and args.with_whole_pair:
        # The headline runs the library's own partition; beside it, the same
        # batch with one workgroup per pair (-1, which equal contexts allow).
        result["whole_pair_partition"] = time_decode_only(
            wl, st, args.layout, -1, max(args.steps // 2, 5), args.warmup)
    if wl.name == "mha" and args.with_mix:
        # The second configuration the target names: mixed context lengths.
        del st
        torch.cuda.empty_cache()
        mix_res, mst = run_decode(W.MIX, dev, args.layout, 0, args.steps, args.warmup, None,
                                  False, False, 0.0 if args.no_cpu_baseline else -1.0)
        keep = ["config", "ms_per_step", "value", "pct_of_peak", "decode_tokens_per_s",
                "decode_us_per_layer", "decode_us_percentiles", "roofline", "allocator",
                "cpu_baseline"]
        result["mix"] = {k: mix_res[k] for k in keep if k in mix_res}
        del mst
        torch.cuda.empty_cache()
    print(json.dumps(result, default=lambda o: o.item() if hasattr(o, "item") else str(o)),
          flush=True)


if __name__ == "__main__":
    main()

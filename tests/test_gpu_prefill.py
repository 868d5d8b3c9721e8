"""Chunked-prefill attention on the device against the oracle.

Every problem stores each sequence's whole context (earlier tokens and the
chunk) with pa_store_kvcache into caches whose other slots hold NaN
patterns, then runs pa_prefill on the packed chunks.  The oracle receives
host copies of the inputs only (the rows, slots, queries, tables) and
computes every row in float64.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_382_amd as pa
import workloads as W
from oracle import decode_ref, prefill_ref, store_ref
from tests.gpu_problems import DEV, check_close, host_u16, say

pytestmark = pytest.mark.gpu


def make(hq, hkv, d, bs, lens, chunks, seed, num_blocks=None, order_seed=None):
    """Device problem + host copies of its inputs."""
    need = sum(-(-L // bs) for L in lens)
    nb = num_blocks or need + 7
    m = max(-(-L // bs) for L in lens)
    alloc = pa.Allocator(nb, bs, m, W.free_order(nb, seed if order_seed is None else order_seed))
    slots = []
    for s, L in enumerate(lens):
        slots += list(alloc.add_seq(s, L))
    tables, lens_arr = alloc.export(list(range(len(lens))), m)
    shape = (nb, bs, hkv, d)
    kc = W.nan_sentinel_fp16(shape, DEV)
    vc = kc.clone()
    pre = host_u16(kc)
    k_rows = W.normal_fp16((len(slots), hkv, d), 1000 + seed, DEV)
    v_rows = W.normal_fp16((len(slots), hkv, d), 2000 + seed, DEV)
    slots_t = torch.tensor(slots, dtype=torch.int32, device=DEV)
    say(f"prefill: store {len(slots)} rows (Hkv={hkv} D={d} bs={bs})")
    pa.pa_store_kvcache(k_rows, v_rows, slots_t, kc, vc)
    starts = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = W.normal_fp16((int(starts[-1]), hq, d), 3000 + seed, DEV)
    kh, vh = store_ref(host_u16(k_rows).view(np.float16), host_u16(v_rows).view(np.float16),
                       slots, pre, pre.copy())
    return {
        "q": q, "kc": kc, "vc": vc,
        "tables": torch.from_numpy(np.ascontiguousarray(tables)).to(DEV),
        "lens": torch.from_numpy(np.ascontiguousarray(lens_arr)).to(DEV),
        "starts": torch.from_numpy(starts).to(DEV),
        "max_q": int(max(chunks)) if len(chunks) else 0,
        "host": {"q": host_u16(q).view(np.float16), "k": kh.view(np.float16),
                 "v": vh.view(np.float16), "tables": np.asarray(tables), "lens": np.asarray(lens_arr),
                 "starts": starts},
    }


def run(p, scale):
    say(f"prefill: pa_prefill T={p['q'].shape[0]} Hq={p['q'].shape[1]} D={p['q'].shape[2]} "
        f"max_q={p['max_q']}")
    out = pa.pa_prefill(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], p["starts"], scale,
                        max_query_len=p["max_q"])
    torch.cuda.synchronize()
    return out


def oracle(p, scale):
    h = p["host"]
    return prefill_ref(h["q"], h["k"], h["v"], h["tables"], h["lens"], h["starts"], scale)


# (name, hq, hkv, d, bs, lens, chunks)
CASES = [
    ("mha_d128", 4, 4, 128, 16, [300, 77, 1000, 40], [256, 77, 1, 0]),
    ("gqa4_d128", 8, 2, 128, 16, [290, 129, 33], [200, 129, 33]),
    ("gqa8_d128", 16, 2, 128, 8, [150, 64], [37, 64]),
    ("gqa3_d128", 6, 2, 128, 32, [95, 260], [95, 17]),
    ("mha_d64", 4, 4, 64, 16, [333, 20], [170, 20]),
    ("gqa2_d64_bs64", 4, 2, 64, 64, [500, 129], [129, 64]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, hq, hkv, d, bs, lens, chunks = case
    scale = float(np.float32(1.0 / np.sqrt(d)))
    p = make(hq, hkv, d, bs, lens, chunks, seed=len(name))
    out = run(p, scale)
    check_close(out, oracle(p, scale), f"prefill {name}")


def test_prefill_is_deterministic_and_placement_invariant():
    lens, chunks = [400, 90], [256, 90]
    a = make(8, 2, 128, 16, lens, chunks, seed=4)
    b = make(8, 2, 128, 16, lens, chunks, seed=4, num_blocks=200, order_seed=99)
    assert not torch.equal(a["tables"], b["tables"])
    scale = 0.0883883
    o1, o2 = run(a, scale), run(a, scale)
    o3 = run(b, scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_peaky_scores_stay_accurate():
    """Large scores: the reference max moves many times inside a row."""
    lens, chunks = [700], [160]
    p = make(4, 4, 128, 16, lens, chunks, seed=8)
    # queries aligned with a few keys give very large, growing scores
    p["q"].mul_(4.0)
    p["host"]["q"] = host_u16(p["q"]).view(np.float16)
    scale = 0.25
    out = run(p, scale)
    check_close(out, oracle(p, scale), "prefill peaky")


def test_single_token_prompt_returns_value_row():
    p = make(4, 2, 128, 16, [1, 1], [1, 1], seed=3)
    out = run(p, 0.1)
    h = p["host"]
    for s in range(2):
        blk = h["tables"][s][0]
        for head in range(4):
            v = h["v"][blk, 0, head // 2]
            assert np.array_equal(host_u16(out[s, head]).view(np.float16), v.astype(np.float16))


FULL = [
    ("prefill_mha", W.PREFILL_MHA),
    ("prefill_gqa", W.PREFILL_GQA),
]


@pytest.mark.parametrize("name,wl", FULL, ids=[f[0] for f in FULL])
def test_prefill_full_size_sampled(name, wl):
    """The benchmarked shape; sampled rows against single-query attention
    over each row's causal prefix (the reduction the oracle is pinned to)."""
    lens = [W.PREFILL_CONTEXT] * wl.num_seqs
    chunks = [W.PREFILL_CHUNK] * wl.num_seqs
    p = make(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, lens, chunks,
             seed=wl.seed, num_blocks=wl.num_blocks)
    out = run(p, wl.scale)
    h = p["host"]
    rng = np.random.default_rng(5)
    got, ref = [], []
    for s in rng.choice(wl.num_seqs, size=4, replace=False):
        for j in [0, 1, 31, 127, 128, 200, W.PREFILL_CHUNK - 1]:
            t = int(h["starts"][s]) + j
            pos = int(h["lens"][s]) - W.PREFILL_CHUNK + j
            r = decode_ref(h["q"][t:t + 1], h["k"], h["v"], h["tables"][s:s + 1], [pos + 1], wl.scale)
            got.append(out[t])
            ref.append(r[0])
    check_close(torch.stack(got), np.stack(ref), f"{name} sampled")


def test_prefill_cache_larger_than_4gib():
    """A pool whose caches exceed 4 GiB, with the sequences' blocks at its top:
    the kernel must address them with 64-bit offsets.  The oracle runs on a
    compact host cache built from the same input rows."""
    hq, hkv, d, bs = 8, 2, 128, 16
    block_bytes = bs * hkv * d * 2
    nb = (1 << 32) // block_bytes + 64
    lens, chunks = [300, 77], [256, 77]
    order = np.arange(nb - 1, -1, -1, dtype=np.int32)          # highest blocks first
    alloc = pa.Allocator(nb, bs, 32, order)
    slots = []
    for s, L in enumerate(lens):
        slots += list(alloc.add_seq(s, L))
    tables, lens_arr = alloc.export([0, 1], 32)
    assert int(tables[0][0]) * block_bytes >= 1 << 32
    say(f"prefill: caches of {nb * block_bytes / 2**30:.2f} GiB each")
    kc = torch.empty((nb, bs, hkv, d), dtype=torch.float16, device=DEV)
    vc = torch.empty_like(kc)
    k_rows = W.normal_fp16((len(slots), hkv, d), 71, DEV)
    v_rows = W.normal_fp16((len(slots), hkv, d), 72, DEV)
    pa.pa_store_kvcache(k_rows, v_rows, torch.tensor(slots, dtype=torch.int32, device=DEV), kc, vc)
    starts = np.array([0, 256, 333], dtype=np.int32)
    q = W.normal_fp16((333, hq, d), 73, DEV)
    out = pa.pa_prefill(q, kc, vc, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens_arr).to(DEV),
                        torch.from_numpy(starts).to(DEV), 0.0883883, max_query_len=256)
    torch.cuda.synchronize()
    # compact oracle cache: used block i of the tables becomes block i
    used = sorted({int(b) for row, L in zip(tables, lens_arr) for b in row[:-(-int(L) // bs)]})
    remap = {b: i for i, b in enumerate(used)}
    small_tables = np.array([[remap.get(int(b), 0) for b in row] for row in tables], dtype=np.int32)
    small_slots = [remap[s // bs] * bs + s % bs for s in slots]
    shape = (len(used), bs, hkv, d)
    kh, vh = store_ref(host_u16(k_rows).view(np.float16), host_u16(v_rows).view(np.float16), small_slots,
                       np.zeros(shape, np.uint16), np.zeros(shape, np.uint16))
    ref = prefill_ref(host_u16(q).view(np.float16), kh.view(np.float16), vh.view(np.float16),
                      small_tables, lens_arr, starts, 0.0883883)
    check_close(out, ref, "prefill > 4 GiB pool")
    del kc, vc
    torch.cuda.empty_cache()


def test_prefill_many_short_chunks():
    """100 sequences with chunks of 1..40 rows over contexts of up to 200
    tokens, grouped heads."""
    rng = np.random.default_rng(23)
    lens = [int(x) for x in rng.integers(1, 200, size=100)]
    chunks = [int(min(L, x)) for L, x in zip(lens, rng.integers(1, 41, size=100))]
    chunks[3] = 0
    p = make(8, 2, 128, 16, lens, chunks, seed=23)
    out = run(p, 0.0883883)
    check_close(out, oracle(p, 0.0883883), "prefill many short chunks")


def test_prefill_long_context_sampled():
    """Two 32768-token contexts with 256-row chunks (block ids past the first
    thousand table entries), sampled rows against single-query attention over
    each row's prefix."""
    lens, chunks = [32768, 30001], [256, 256]
    p = make(8, 2, 128, 16, lens, chunks, seed=41)
    out = run(p, 0.0883883)
    h = p["host"]
    got, ref = [], []
    for s in range(2):
        for j in [0, 77, 255]:
            t = int(h["starts"][s]) + j
            pos = int(h["lens"][s]) - 256 + j
            r = decode_ref(h["q"][t:t + 1], h["k"], h["v"], h["tables"][s:s + 1], [pos + 1], 0.0883883)
            got.append(out[t])
            ref.append(r[0])
    check_close(torch.stack(got), np.stack(ref), "prefill long context")


def random_prefill_configs(n=12, seed=47):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        bs = int(rng.choice([4, 8, 16, 32, 64, 128]))
        b = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.integers(1, 500, size=b)]
        chunks = [int(rng.integers(0, L + 1)) for L in lens]
        if b > 1:
            chunks[0] = lens[0]                        # a whole prompt
        if b > 2:
            chunks[1] = 1                              # a single new row
        if b > 3:
            chunks[2] = 0                              # no rows this step
        out.append((i, d, g, hkv, bs, lens, chunks))
    return out


@pytest.mark.parametrize("cfg", random_prefill_configs(), ids=lambda c: f"r{c[0]}_d{c[1]}_g{c[2]}_bs{c[4]}")
def test_prefill_random_configurations(cfg):
    """Seeded random shapes: head dim, group (odd ones too), KV heads, block
    size, batch, ragged contexts and chunks (whole prompts, single rows, empty)."""
    i, d, g, hkv, bs, lens, chunks = cfg
    scale = float(np.float32(1.0 / np.sqrt(d)))
    p = make(g * hkv, hkv, d, bs, lens, chunks, seed=200 + i)
    out = run(p, scale)
    check_close(out, oracle(p, scale), f"prefill random config {i}")

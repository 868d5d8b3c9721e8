"""GPU parity of pa_decode against the fp64 oracle.

Tolerance (fp16 output, fp32 accumulation): max-abs 4e-3 and mean-abs 5e-4,
plus relative L2 1e-3 (fp16 output rounding alone is at most 2^-11 relative).
Placement and sharing invariances are checked bitwise on the GPU output.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_382_amd as pa
import workloads as W
from oracle import decode_ref, store_ref
from tests.gpu_problems import (DEV, build, check_close, host_u16, oracle_caches, oracle_out,
                                run_step, say)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": W.TINY,
    "tiny_d128_g4": W.shrink(W.TINY, name="tiny_d128_g4", num_q_heads=16, num_kv_heads=4,
                             head_dim=128),
    "tiny_d64_g8": W.shrink(W.TINY, name="tiny_d64_g8", num_q_heads=16, num_kv_heads=2),
    "tiny_bs8_g2": W.shrink(W.TINY, name="tiny_bs8_g2", block_size=8, num_blocks=128,
                            max_blocks_per_seq=8, num_q_heads=6, num_kv_heads=3, head_dim=128),
    "tiny_bs32": W.shrink(W.TINY, name="tiny_bs32", block_size=32, num_blocks=32,
                          max_blocks_per_seq=4, num_q_heads=8, num_kv_heads=8, head_dim=128),
    "tiny_bs64_g4": W.shrink(W.TINY, name="tiny_bs64_g4", block_size=64, num_blocks=16,
                             max_blocks_per_seq=2, num_q_heads=8, num_kv_heads=2, head_dim=64),
}

# Several partitions, several chunks per wave and ragged tails everywhere.
MEDIUM = W.shrink(W.MIX, name="medium", num_seqs=6, num_blocks=1024, max_blocks_per_seq=256,
                  num_q_heads=16, num_kv_heads=4)
MEDIUM_LENS = [1, 17, 200, 1000, 2049, 3333]


def medium_plan(wl=MEDIUM, lens=MEDIUM_LENS):
    return lambda a: W._plain_plan(a, wl, lens)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_small_matches_oracle(name):
    wl = SMALL[name]
    p = build(wl, plan_fn=lambda a: W.tiny_plan(a, wl))
    out = run_step(p)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), name)


# 1: one split walks every pair; 5, 37: ranges end mid-pair; 1000: more
# splits than workgroups (the queue hands out the rest); 2000: about one chunk
# per split; 4000: more splits than chunks (empty ranges between a pair's
# owners); 0: the device default.
@pytest.mark.parametrize("N", [1, 5, 37, 256, 1000, 2000, 4000, 0])
def test_decode_split_sizes_match_oracle(N):
    p = build(MEDIUM, plan_fn=medium_plan())
    out = run_step(p, num_splits=N)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"N={N}")


@pytest.mark.parametrize("bs", [8, 32, 64])
def test_decode_block_sizes_medium(bs):
    wl = W.shrink(MEDIUM, name=f"medium_bs{bs}", block_size=bs,
                  num_blocks=1024 * 16 // bs, max_blocks_per_seq=4096 // bs)
    p = build(wl, plan_fn=medium_plan(wl))
    out = run_step(p, num_splits=97)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"bs={bs}")


def test_decode_is_deterministic_and_placement_invariant():
    p = build(MEDIUM, plan_fn=medium_plan())
    out1 = run_step(p, num_splits=300)
    say("decode again")
    out2 = pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], MEDIUM.scale,
                        max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    nb = MEDIUM.num_blocks
    pi = torch.from_numpy(np.random.default_rng(4).permutation(nb)).to(DEV)
    k2, v2 = torch.empty_like(p["kc"]), torch.empty_like(p["vc"])
    k2[pi], v2[pi] = p["kc"], p["vc"]
    t2 = torch.where(p["tables"] >= 0, pi[p["tables"].clamp(min=0).long()].int(), p["tables"])
    say("decode on permuted placement")
    out3 = pa.pa_decode(p["q"], k2, v2, t2.contiguous(), p["lens"], MEDIUM.scale,
                        max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


SMALL_PREFIX = W.shrink(W.PREFIX, name="small_prefix", num_seqs=8, num_blocks=256,
                        max_blocks_per_seq=64)


def small_prefix_plan(a):
    return W.prefix_plan(a, SMALL_PREFIX, prefix_tokens=496, suffix_range=(5, 60))


def test_shared_prefix_equals_private_copies_bitwise():
    p = build(SMALL_PREFIX, plan_fn=small_prefix_plan)
    out_shared = run_step(p, num_splits=50)
    kc, vc = oracle_caches(p)
    check_close(out_shared, oracle_out(p, kc, vc), "prefix")
    # private copies of every shared block, made on the device
    tables = p["tables"].cpu().numpy()
    lens = p["lens"].cpu().numpy()
    bs = SMALL_PREFIX.block_size
    owners = {}
    for s, row in enumerate(tables):
        for b in row[:-(-int(lens[s]) // bs)]:
            owners.setdefault(int(b), []).append(s)
    shared = {b for b, o in owners.items() if len(o) > 1}
    assert len(shared) >= 31
    extra = sum(len(owners[b]) for b in shared)
    nb = SMALL_PREFIX.num_blocks
    k2 = torch.cat([p["kc"], torch.zeros((extra,) + p["kc"].shape[1:], dtype=torch.float16,
                                         device=DEV)])
    v2 = torch.cat([p["vc"], torch.zeros_like(k2[:extra])])
    t2 = tables.copy()
    nxt = nb
    for s in range(len(tables)):
        for j in range(-(-int(lens[s]) // bs)):
            b = int(tables[s, j])
            if b in shared:
                k2[nxt], v2[nxt] = p["kc"][b], p["vc"][b]
                t2[s, j] = nxt
                nxt += 1
    say("decode on private copies")
    out_private = pa.pa_decode(p["q"], k2, v2, torch.from_numpy(t2).to(DEV), p["lens"],
                               SMALL_PREFIX.scale, max_context_len=p["max_ctx"],
                               num_splits=50)
    torch.cuda.synchronize()
    assert torch.equal(out_shared.view(torch.int16), out_private.view(torch.int16))


def test_garbage_in_unused_slots_does_not_leak():
    """NaN-filled vs zero-filled unused slots and table padding: same bits."""
    p = build(MEDIUM, plan_fn=medium_plan())
    out_nan = run_step(p, num_splits=300)
    assert torch.isfinite(out_nan.float()).all()
    mask = np.zeros(MEDIUM.num_blocks * MEDIUM.block_size, dtype=bool)
    from tests.gpu_problems import used_slot_mask
    mask = used_slot_mask(MEDIUM, p["plan"].block_tables, p["plan"].context_lens)
    unused = torch.from_numpy(~mask).to(DEV)
    k0, v0 = p["kc"].clone(), p["vc"].clone()
    k0.view(-1, MEDIUM.num_kv_heads, MEDIUM.head_dim)[unused] = 0
    v0.view(-1, MEDIUM.num_kv_heads, MEDIUM.head_dim)[unused] = 0
    t0 = p["tables"].clone()
    t0[t0 < 0] = 7          # padding entries now point at a real block
    say("decode with zeroed unused slots")
    out_zero = pa.pa_decode(p["q"], k0, v0, t0, p["lens"], MEDIUM.scale,
                            max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    assert torch.equal(out_nan.view(torch.int16), out_zero.view(torch.int16))


def test_single_token_context_returns_value_row_exactly():
    wl = SMALL["tiny_d128_g4"]
    p = build(wl, plan_fn=lambda a: W.tiny_plan(a, wl))
    out = run_step(p)
    s = W.TINY_LENS.index(1)
    v_new = p["v_new"][s]                                 # [Hkv, D]
    expect = v_new.repeat_interleave(wl.group, dim=0)
    assert torch.equal(out[s].view(torch.int16), expect.view(torch.int16))


def test_empty_context_gives_zero_rows():
    p = build(MEDIUM, plan_fn=medium_plan())
    run_step(p, num_splits=300)         # caches now hold the step's tokens
    lens = p["lens"].clone()
    lens[2] = 0
    out = torch.full_like(p["q"], float("nan"))
    say("decode with an empty context")
    pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], lens, MEDIUM.scale, out=out,
                 max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[2]).item() == 0
    kc, vc = oracle_caches(p)
    r = p["ref"]
    ref = decode_ref(r["q"], kc.view(np.float16), vc.view(np.float16), r["tables"],
                     lens.cpu().numpy(), MEDIUM.scale)
    keep = [0, 1, 3, 4, 5]
    check_close(out[keep], ref[keep], "empty-context batch")


def test_peaky_queries():
    """q = 2 K[p*]: the softmax concentrates on one token; out ~ V[p*]."""
    p = build(MEDIUM, plan_fn=medium_plan())
    run_step(p, num_splits=300)          # caches now hold the step's tokens
    kc, vc = oracle_caches(p)
    r = p["ref"]
    rng = np.random.default_rng(17)
    q = np.zeros_like(r["q"])
    from oracle import gather_sequence
    for s, L in enumerate(r["lens"]):
        K = gather_sequence(kc.view(np.float16), r["tables"][s], int(L))
        for h in range(MEDIUM.num_q_heads):
            star = int(rng.integers(int(L)))
            q[s, h] = (K[star, h // MEDIUM.group].astype(np.float32) * 2).astype(np.float16)
    qd = torch.from_numpy(q).to(DEV)
    say("decode with peaky queries")
    out = pa.pa_decode(qd, p["kc"], p["vc"], p["tables"], p["lens"], MEDIUM.scale,
                       max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    ref = decode_ref(q, kc.view(np.float16), vc.view(np.float16), r["tables"], r["lens"],
                     MEDIUM.scale)
    check_close(out, ref, "peaky")


def test_out_of_range_table_entry_is_skipped_not_read():
    """Without validation a bad entry must not fault: its block counts as empty."""
    p = build(MEDIUM, plan_fn=medium_plan())
    run_step(p, num_splits=300)
    s = 4                                           # 2049 tokens: last block holds 1 token
    L = int(p["plan"].context_lens[s])
    last = (L - 1) // MEDIUM.block_size
    bad = p["tables"].clone()
    bad[s, last] = MEDIUM.num_blocks + 1000
    say("decode with an out-of-range table entry")
    out = pa.pa_decode(p["q"], p["kc"], p["vc"], bad, p["lens"], MEDIUM.scale,
                       max_context_len=p["max_ctx"], num_splits=300)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(p)
    r = p["ref"]
    lens = r["lens"].copy()
    lens[s] = last * MEDIUM.block_size
    ref = decode_ref(r["q"], kc.view(np.float16), vc.view(np.float16), r["tables"], lens,
                     MEDIUM.scale)
    check_close(out, ref, "bad entry")
    prev = pa.pa_set_validate(True)
    try:
        with pytest.raises(pa.PaError) as e:
            pa.pa_decode(p["q"], p["kc"], p["vc"], bad, p["lens"], MEDIUM.scale,
                         max_context_len=p["max_ctx"], num_splits=300)
        assert e.value.code == "RANGE"
        with pytest.raises(pa.PaError) as e:
            pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], MEDIUM.scale,
                         max_context_len=100, num_splits=300)
        assert e.value.code == "RANGE"
    finally:
        pa.pa_set_validate(prev)


@pytest.mark.parametrize("bs", [8, 16])
def test_out_of_range_entries_inside_a_context_drop_their_tokens(bs):
    """Bad entries at an even and an odd block index of a long context (at
    block size 8 the first and the second block of a 16-token chunk): their
    tokens drop out of the softmax, which the oracle reproduces by leaving the
    two blocks out of the table (attention over a set of rows does not depend
    on their order)."""
    wl = W.shrink(MEDIUM, name=f"medium_bad_bs{bs}", block_size=bs,
                  num_blocks=1024 * 16 // bs, max_blocks_per_seq=4096 // bs)
    p = build(wl, plan_fn=medium_plan(wl))
    run_step(p)
    s = 5                                           # 3333 tokens
    L = int(p["plan"].context_lens[s])
    nblk = -(-L // bs)
    drop = [40, 101]
    assert max(drop) < nblk - 1
    bad = p["tables"].clone()
    for i in drop:
        bad[s, i] = -1 if i % 2 else wl.num_blocks + 5
    for n_split in (0, 300):
        say(f"decode with out-of-range entries, block size {bs}, {n_split} splits")
        out = pa.pa_decode(p["q"], p["kc"], p["vc"], bad, p["lens"], wl.scale,
                           max_context_len=p["max_ctx"], num_splits=n_split)
        torch.cuda.synchronize()
        kc, vc = oracle_caches(p)
        r = p["ref"]
        tables = r["tables"].copy()
        keep = [i for i in range(tables.shape[1]) if i not in drop]
        tables[s] = np.concatenate([tables[s, keep], np.full(len(drop), -1, tables.dtype)])
        lens = r["lens"].copy()
        lens[s] = L - len(drop) * bs
        ref = decode_ref(r["q"], kc.view(np.float16), vc.view(np.float16), tables, lens, wl.scale)
        check_close(out, ref, f"bad entries bs={bs} N={n_split}")


# Full-size workloads in the launch configuration the benchmark times (the
# library's default partition), and mha also on one workgroup per pair (-1);
# every sequence is compared except in prefix, where 6 of 64 share one prefix.
FULL = [("mha", None, 0), ("mha", None, -1), ("mix", None, 0), ("prefix", [0, 15, 31, 47, 62, 63], 0),
        ("long_bs16", None, 0), ("long_bs8", None, 0), ("long_bs64", None, 0)]


@pytest.mark.parametrize("name,seqs,n_split", FULL, ids=[f"{f[0]}_N{f[2]}" for f in FULL])
def test_decode_full_size(name, seqs, n_split):
    wl = W.ALL.get(name) or W.long_workload(int(name.split("bs")[1]))
    p = build(wl, fill="random")
    out = run_step(p, num_splits=n_split)
    kc, vc = oracle_caches(p)
    ref = oracle_out(p, kc, vc, seqs)
    check_close(out if seqs is None else out[seqs], ref, name)


@pytest.mark.parametrize("N", [64, 200])
def test_decode_head_group_and_plain_orders_in_one_call(N):
    """Slot-major, 4 query heads per KV head, 4 KV heads: a sequence takes the
    head-group order while its groups span at most about 32 splits
    (4 * chunks * N <= 30 * U; here U = 4 * 341 chunks).  At N = 64 the
    4 000-token sequence (250 chunks) runs the plain order and the others the
    head-group order; at N = 200 the 1 000-token one (63 chunks) also runs the
    plain order.  Every row against the oracle; the same call with the plain
    order's workspace (every sequence plain) too."""
    lens = [4000, 100, 300, 17, 1000]
    wl = W.shrink(MEDIUM, name="orders", num_seqs=len(lens))
    p = build(wl, plan_fn=medium_plan(wl, lens))
    out = run_step(p, num_splits=N)
    kc, vc = oracle_caches(p)
    ref = oracle_out(p, kc, vc)
    check_close(out, ref, f"mixed orders N={N}")
    B = p["q"].shape[0]
    desc_h = pa.cache_desc(p["kc"])                  # same sizes, head-major: plain order only
    desc_h.layout = pa.LAYOUTS["head"]
    plain = pa.decode_workspace(desc_h, B, wl.num_q_heads, N, DEV)
    assert plain.numel() < pa.pa_decode_workspace_bytes(pa.cache_desc(p["kc"]), B, wl.num_q_heads, N)
    say(f"orders: plain-order workspace, N={N}")
    out_p = pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], wl.scale,
                         max_context_len=p["max_ctx"], num_splits=N, workspace=plain)
    torch.cuda.synchronize()
    check_close(out_p, ref, f"plain order N={N}")


def test_decode_full_size_mix_head_major():
    """The mixed-length workload with the head-major cache: bitwise equal to
    the slot-major call in the same (plain) order, which slot-major runs when
    given the plain order's workspace (same arithmetic, other addresses); the
    head-major result and the slot-major result in its default head-group
    order both within the bar of the oracle for every sequence."""
    wl = W.MIX
    p = build(wl, fill="random")
    out_sd = run_step(p)                       # default workspace: head-group order
    nb, bs, hkv, d = p["kc"].shape
    kh = p["kc"].transpose(1, 2).contiguous()
    vh = p["vc"].transpose(1, 2).contiguous()
    B = p["q"].shape[0]
    plain = pa.decode_workspace(pa.cache_desc(kh, "head"), B, wl.num_q_heads, 0, DEV)
    say("mix slot-major, plain order: pa_decode")
    out_s = pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], wl.scale,
                         max_context_len=p["max_ctx"], workspace=plain)
    say("mix head-major: pa_decode")
    out_h = pa.pa_decode(p["q"], kh, vh, p["tables"], p["lens"], wl.scale,
                         max_context_len=p["max_ctx"], layout="head")
    torch.cuda.synchronize()
    assert torch.equal(out_h.view(torch.int16), out_s.view(torch.int16))
    kc, vc = oracle_caches(p)
    ref = oracle_out(p, kc, vc)
    check_close(out_h, ref, "mix head-major")
    check_close(out_sd, ref, "mix slot-major, head-group order")


GROUPS = [(g, bs, d) for g, bs, d in [(3, 16, 128), (3, 8, 64), (5, 16, 64), (5, 8, 128), (6, 32, 128),
                                      (6, 8, 64), (7, 16, 128), (7, 64, 64), (9, 16, 128),
                                      (12, 8, 64), (12, 16, 128), (16, 16, 128), (16, 8, 64)]]


@pytest.mark.parametrize("g,bs,d", GROUPS, ids=[f"g{g}_bs{bs}_d{d}" for g, bs, d in GROUPS])
@pytest.mark.parametrize("n_split", [0, 23])
def test_decode_any_group_size(g, bs, d, n_split):
    """Query groups other than 1, 2, 4, 8: 3 to 7 run padded on matrix cores
    (block >= 16) or on the vector kernel (block 8); groups above 8 run as
    groups of their largest divisor up to 8.  Ragged lengths, a single-token
    context, the default split and 23 splits (pairs across splits)."""
    rng = np.random.default_rng(1000 + 31 * g + bs + d)
    hkv = 2
    lens = [int(x) for x in rng.integers(1, 600, size=7)]
    lens[3] = 1
    m = max(-(-L // bs) for L in lens)
    nb = sum(-(-L // bs) for L in lens) + 8
    wl = W.shrink(W.MIX, name=f"group{g}", num_seqs=len(lens), num_q_heads=g * hkv,
                  num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=nb,
                  max_blocks_per_seq=m, seed=500 + g)
    p = build(wl, lambda a: W._plain_plan(a, wl, lens))
    out = run_step(p, num_splits=n_split)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"group {g} bs {bs} d {d}")


LARGE_BATCH = W.shrink(W.MIX, name="large_batch", num_seqs=150, num_blocks=4096, max_blocks_per_seq=32,
                       num_q_heads=16, num_kv_heads=4)
# The same batch with 6 query heads per KV head (two row sets of the matrix-core kernel).
LARGE_BATCH_G6 = W.shrink(LARGE_BATCH, name="large_batch_g6", num_q_heads=24)


def large_batch_lens():
    rng = np.random.default_rng(17)
    lens = [int(x) for x in rng.integers(1, 400, size=LARGE_BATCH.num_seqs)]
    lens[5] = lens[77] = 1               # single-token contexts
    lens[140] = 400                      # a table row filled to the last block
    return lens


@pytest.mark.parametrize("N", [0, 7, 333])
@pytest.mark.parametrize("wl", [LARGE_BATCH, LARGE_BATCH_G6], ids=["g4", "g6"])
def test_decode_batch_larger_than_a_wave(N, wl):
    """More than 64 sequences: context lengths no longer fit one wave's
    registers, so the split kernel and the merge kernel scan them from memory.
    Every row is checked against the oracle."""
    lens = large_batch_lens()
    p = build(wl, lambda a: W._plain_plan(a, wl, lens))
    out = run_step(p, num_splits=N)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"large batch N={N}")


def random_configs(n=16, seed=31):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        bs = int(rng.choice([8, 16, 32, 64]))
        b = int(rng.integers(1, 20))
        lens = [int(x) for x in rng.integers(1, 700, size=b)]
        if b > 2:
            lens[int(rng.integers(b))] = 1
        n_split = int(rng.choice([0, 0, 1, 3, 64, 999]))
        out.append((i, d, g, hkv, bs, lens, n_split))
    return out


@pytest.mark.parametrize("cfg", random_configs(), ids=lambda c: f"r{c[0]}_d{c[1]}_g{c[2]}_bs{c[4]}")
def test_decode_random_configurations(cfg):
    """Seeded random shapes: head dim, group, KV heads, block size, batch,
    ragged lengths (with single-token contexts) and split counts."""
    i, d, g, hkv, bs, lens, n_split = cfg
    m = max(-(-L // bs) for L in lens)
    nb = sum(-(-L // bs) for L in lens) + 16
    wl = W.shrink(W.MIX, name=f"random{i}", num_seqs=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv,
                  head_dim=d, block_size=bs, num_blocks=nb, max_blocks_per_seq=m, seed=100 + i)
    p = build(wl, lambda a: W._plain_plan(a, wl, lens))
    out = run_step(p, num_splits=n_split)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"random config {i}")


def test_store_copy_decode_cache_larger_than_4gib():
    """A pool whose caches exceed 4 GiB with the sequences' blocks at its top:
    the store, a block copy between two top blocks and decode all address past
    4 GiB.  The oracle runs on a compact host cache holding the same rows."""
    hq, hkv, d, bs = 16, 4, 128, 16
    block_bytes = bs * hkv * d * 2
    nb = (1 << 32) // block_bytes + 256
    lens = [300, 77, 1000]
    m = 64
    order = np.arange(nb - 1, -1, -1, dtype=np.int32)          # highest blocks first
    alloc = pa.Allocator(nb, bs, m, order)
    slots = []
    for s, L in enumerate(lens):
        slots += list(alloc.add_seq(s, L))
    tables, lens_arr = alloc.export(list(range(len(lens))), m)
    assert min(int(x) // bs for x in slots) * block_bytes >= 1 << 32
    say(f"decode: caches of {nb * block_bytes / 2**30:.2f} GiB each")
    kc = torch.empty((nb, bs, hkv, d), dtype=torch.float16, device=DEV)
    vc = torch.empty_like(kc)
    k_rows = W.normal_fp16((len(slots), hkv, d), 81, DEV)
    v_rows = W.normal_fp16((len(slots), hkv, d), 82, DEV)
    say("decode > 4 GiB: store")
    pa.pa_store_kvcache(k_rows, v_rows, torch.tensor(slots, dtype=torch.int32, device=DEV), kc, vc)
    # copy the first block of sequence 2 onto a free block near the top, and
    # point sequence 2's table at the copy
    src = int(tables[2][0])
    dst = int(alloc.free_list()[0])
    assert dst * block_bytes >= 1 << 32
    say(f"decode > 4 GiB: copy block {src} -> {dst}")
    pa.pa_copy_blocks(kc, vc, torch.tensor([[src, dst]], dtype=torch.int32, device=DEV))
    tables = np.array(tables, dtype=np.int32)
    tables[2][0] = dst
    q = W.normal_fp16((len(lens), hq, d), 83, DEV)
    say("decode > 4 GiB: decode")
    out = pa.pa_decode(q, kc, vc, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens_arr).to(DEV),
                       0.0883883, max_context_len=max(lens))
    torch.cuda.synchronize()
    assert torch.equal(kc[dst].view(torch.int16), kc[src].view(torch.int16))
    assert torch.equal(vc[dst].view(torch.int16), vc[src].view(torch.int16))
    # compact oracle cache: used block i of the tables becomes block i
    used = sorted({int(b) for row, L in zip(tables, lens_arr) for b in row[:-(-int(L) // bs)]} | {src})
    remap = {b: i for i, b in enumerate(used)}
    small_tables = np.array([[remap.get(int(b), 0) for b in row] for row in tables], dtype=np.int32)
    small_slots = [remap[s // bs] * bs + s % bs for s in slots]
    shape = (len(used), bs, hkv, d)
    kh, vh = store_ref(host_u16(k_rows).view(np.float16), host_u16(v_rows).view(np.float16), small_slots,
                       np.zeros(shape, np.uint16), np.zeros(shape, np.uint16))
    kh[remap[dst]] = kh[remap[src]]
    vh[remap[dst]] = vh[remap[src]]
    ref = decode_ref(host_u16(q).view(np.float16), kh.view(np.float16), vh.view(np.float16),
                     small_tables, lens_arr, 0.0883883)
    check_close(out, ref, "decode > 4 GiB pool")
    del kc, vc
    torch.cuda.empty_cache()


SHORT_LENS = [1, 16, 17, 200, 512, 33, 64, 300]


def test_whole_pairs_short_contexts_with_empty_ones():
    """Contexts of at most 512 tokens and the default split: one workgroup per
    (sequence, KV head) pair and no merge launch.  Empty contexts still get
    zero rows and every other row is written (the output starts as NaN)."""
    p = build(MEDIUM, plan_fn=medium_plan(lens=SHORT_LENS))
    out0 = run_step(p)                  # caches now hold the step's tokens
    kc, vc = oracle_caches(p)
    check_close(out0, oracle_out(p, kc, vc), "whole pairs")
    lens = p["lens"].clone()
    lens[1] = 0
    lens[6] = 0
    out = torch.full_like(p["q"], float("nan"))
    say("whole pairs with empty contexts")
    pa.pa_decode(p["q"], p["kc"], p["vc"], p["tables"], lens, MEDIUM.scale, out=out,
                 max_context_len=p["max_ctx"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[1]).item() == 0 and torch.count_nonzero(out[6]).item() == 0
    r = p["ref"]
    ref = decode_ref(r["q"], kc.view(np.float16), vc.view(np.float16), r["tables"],
                     lens.cpu().numpy(), MEDIUM.scale)
    keep = [0, 2, 3, 4, 5, 7]
    check_close(out[keep], ref[keep], "whole pairs, empty contexts")


def test_whole_pairs_agree_with_split_path_and_repeat_bitwise():
    p = build(MEDIUM, plan_fn=medium_plan(lens=SHORT_LENS))
    run_step(p)
    args = (p["q"], p["kc"], p["vc"], p["tables"], p["lens"], MEDIUM.scale)
    say("whole pairs twice, then 7 explicit splits")
    a = pa.pa_decode(*args, max_context_len=p["max_ctx"])
    b = pa.pa_decode(*args, max_context_len=p["max_ctx"])
    c = pa.pa_decode(*args, max_context_len=p["max_ctx"], num_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    kc, vc = oracle_caches(p)
    ref = oracle_out(p, kc, vc)
    check_close(a, ref, "whole pairs")
    check_close(c, ref, "split path")


@pytest.mark.parametrize("lens", [MEDIUM_LENS, [1500] * 6], ids=["ragged", "equal"])
def test_whole_pairs_requested_for_long_contexts(lens):
    """num_splits = -1: one workgroup per pair whatever the context lengths."""
    p = build(MEDIUM, plan_fn=medium_plan(lens=lens))
    out = run_step(p, num_splits=-1)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), "whole pairs requested")


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("n_split", [300, 5000])
def test_merge_rounds_head_dim_64(g, n_split):
    """Head dim 64 with pairs spanning many more splits than one merge round
    holds (300: about 40-100 splits a pair; 5000: more splits than chunks, so
    many splits are empty and must be skipped by index)."""
    lens = [1, 300, 777, 1200, 64]
    hkv = 2
    m = max(-(-L // 16) for L in lens)
    nb = sum(-(-L // 16) for L in lens) + 16
    wl = W.shrink(W.MIX, name=f"merge64_g{g}", num_seqs=len(lens), num_q_heads=g * hkv, num_kv_heads=hkv,
                  head_dim=64, block_size=16, num_blocks=nb, max_blocks_per_seq=m, seed=200 + g)
    p = build(wl, lambda a: W._plain_plan(a, wl, lens))
    out = run_step(p, num_splits=n_split)
    kc, vc = oracle_caches(p)
    check_close(out, oracle_out(p, kc, vc), f"head dim 64, group {g}, {n_split} splits")

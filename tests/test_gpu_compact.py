"""Compaction and prefix caching on the device.

Compaction: the allocator renumbers the blocks of a fragmented pool, the
library applies the returned copy list with one many-pair pa_copy_blocks, and
then (a) both caches equal the oracle's copy of the same list, byte for byte,
and (b) decode through the new tables equals decode through the old ones bit
for bit (the decode kernel's result does not depend on where blocks sit).

Prefix caching: sequences registered by token ids share the cached full
blocks of a common prefix and store only the tokens past it; decode over the
shared layout must equal the oracle's decode of each sequence's own K/V rows,
and equal, bit for bit, the library's decode over a private layout where
every token is stored.
"""

import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_382_amd as pa
import workloads as W
from oracle import AllocatorModel, copy_blocks_ref, decode_ref, store_ref
from tests.gpu_problems import DEV, build, check_close, host_u16, oracle_caches, run_step, say

pytestmark = pytest.mark.gpu

FRAG = W.shrink(W.MIX, name="compact_mix", num_seqs=12, num_blocks=4096, max_blocks_per_seq=256)
FRAG_LENS = [1, 15, 16, 17, 300, 999, 1024, 2000, 2900, 31, 64, 700]


def frag_plan(a):
    """A pool scattered by a seeded add/append/free trace, the step's
    sequences in what is left, then every other sequence of the trace freed
    (the rest stay live and move with the compaction)."""
    live = W.fragment_pool(a, seed=5, n_ops=600, max_tokens=3000, append_max=64)
    need = sum(-(-L // FRAG.block_size) for L in FRAG_LENS) + len(FRAG_LENS)
    while a.num_free() < need:
        a.free_seq(live.pop(0))
    plan = W._plain_plan(a, FRAG, FRAG_LENS)
    for s in live[::2]:
        a.free_seq(s)
    return plan


def test_compaction_copy_matches_oracle_and_keeps_decode_bitwise():
    p = build(FRAG, frag_plan)
    out_before = run_step(p)
    kc_ref, vc_ref = oracle_caches(p)
    check_close(out_before, decode_ref(p["ref"]["q"], kc_ref.view(np.float16), vc_ref.view(np.float16),
                                       p["ref"]["tables"], p["ref"]["lens"], FRAG.scale),
                "compact: before")

    pairs = p["alloc"].compact()
    pairs_ref = p["model"].compact()
    assert [tuple(x) for x in pairs] == [tuple(x) for x in pairs_ref]
    assert len(pairs) > 100, "the trace should leave a fragmented pool"
    say(f"compact: pa_copy_blocks x{len(pairs)}")
    pa.pa_copy_blocks(p["kc"], p["vc"], torch.from_numpy(np.ascontiguousarray(pairs)).to(DEV))
    torch.cuda.synchronize()
    kc_ref, vc_ref = copy_blocks_ref(kc_ref, vc_ref, np.asarray(pairs_ref, dtype=np.int32).reshape(-1, 2))
    assert np.array_equal(host_u16(p["kc"]), kc_ref)
    assert np.array_equal(host_u16(p["vc"]), vc_ref)

    seqs = p["plan"].seq_ids
    tables, lens = p["alloc"].export(seqs, FRAG.max_blocks_per_seq)
    tables_ref, lens_ref = p["model"].export(seqs, FRAG.max_blocks_per_seq)
    assert np.array_equal(tables, np.asarray(tables_ref)) and list(lens) == list(lens_ref)
    used = sum(1 for r in p["model"].refcounts if r > 0)
    assert int(np.max(tables)) < used
    say("compact: pa_decode through the compacted tables")
    out_after = pa.pa_decode(p["q"], p["kc"], p["vc"], torch.from_numpy(tables).to(DEV),
                             torch.from_numpy(lens).to(DEV), FRAG.scale,
                             max_context_len=p["max_ctx"])
    torch.cuda.synchronize()
    assert torch.equal(out_after.view(torch.int16), out_before.view(torch.int16))


# --------------------------------------------------------------------------
# prefix caching
# --------------------------------------------------------------------------

PWL = W.shrink(W.PREFIX, name="prefix_cache", num_seqs=6, num_blocks=512, max_blocks_per_seq=64)


def token_lists():
    rng = np.random.default_rng(11)
    shared = [int(x) for x in rng.integers(0, 32000, size=300)]
    lists = {
        0: shared + [int(x) for x in rng.integers(0, 32000, size=41)],
        1: shared + [int(x) for x in rng.integers(0, 32000, size=7)],
        2: shared[:160] + [int(x) for x in rng.integers(0, 32000, size=90)],
        3: shared[:300],                                # ends on a block edge past 288
        4: [int(x) for x in rng.integers(0, 32000, size=129)],
    }
    late = shared[:250] + [int(x) for x in rng.integers(0, 32000, size=33)]
    return lists, late


def rows_for(tokens, hkv, d):
    """K and V rows of every position: a function of the token prefix up to
    and including that position (as a causal model's K/V are)."""
    k = np.empty((len(tokens), hkv, d), dtype=np.float16)
    v = np.empty_like(k)
    for pos in range(len(tokens)):
        seed = zlib.crc32(np.asarray(tokens[:pos + 1], dtype=np.int32).tobytes())
        r = np.random.default_rng(seed).standard_normal((2, hkv, d)).astype(np.float16)
        k[pos], v[pos] = r[0], r[1]
    return k, v


def test_prefix_cache_shared_layout_matches_private_layout():
    hkv, d, bs = PWL.num_kv_heads, PWL.head_dim, PWL.block_size
    lists, late = token_lists()
    shape = (PWL.num_blocks, bs, hkv, d)
    kc = W.nan_sentinel_fp16(shape, DEV)
    vc = kc.clone()
    alloc = pa.Allocator(PWL.num_blocks, bs, PWL.max_blocks_per_seq)
    model = AllocatorModel(PWL.num_blocks, bs, PWL.max_blocks_per_seq)
    rows = {s: rows_for(t, hkv, d) for s, t in list(lists.items()) + [(5, late)]}

    def add(seq, toks):
        slots, n_cached = alloc.add_seq_tokens(seq, toks)
        slots_ref, cached_ref = model.add_seq_tokens(seq, toks)
        assert list(slots) == list(slots_ref) and n_cached == cached_ref
        k, v = rows[seq]
        if n_cached < len(toks):
            say(f"prefix cache: store seq {seq} tokens {n_cached}..{len(toks)}")
            pa.pa_store_kvcache(torch.from_numpy(np.ascontiguousarray(k[n_cached:])).to(DEV),
                                torch.from_numpy(np.ascontiguousarray(v[n_cached:])).to(DEV),
                                torch.from_numpy(np.ascontiguousarray(slots[n_cached:])).to(DEV),
                                kc, vc)
        return n_cached

    cached = {s: add(s, t) for s, t in lists.items()}
    assert cached == {0: 0, 1: 288, 2: 160, 3: 288, 4: 0}
    alloc.free_seq(0)
    model.free_seq(0)
    pairs = alloc.compact()
    assert [tuple(x) for x in pairs] == [tuple(x) for x in model.compact()]
    if len(pairs):
        say(f"prefix cache: compaction copies x{len(pairs)}")
        pa.pa_copy_blocks(kc, vc, torch.from_numpy(np.ascontiguousarray(pairs)).to(DEV))
    assert add(5, late) == 240                          # still cached through seqs 1-3
    assert alloc.prefix_stats() == model.prefix_stats()

    live = [1, 2, 3, 4, 5]
    toks = {s: (late if s == 5 else lists[s]) for s in live}
    tables, lens = alloc.export(live, PWL.max_blocks_per_seq)
    q = W.normal_fp16((len(live), PWL.num_q_heads, d), 21, DEV)
    say("prefix cache: pa_decode over the shared layout")
    out_shared = pa.pa_decode(q, kc, vc, torch.from_numpy(tables).to(DEV),
                              torch.from_numpy(lens).to(DEV), PWL.scale,
                              max_context_len=int(max(lens)))

    # private layout: every sequence holds its own blocks and every row is stored
    priv = AllocatorModel(PWL.num_blocks, bs, PWL.max_blocks_per_seq)
    kp = W.nan_sentinel_fp16(shape, DEV)
    vp = kp.clone()
    all_slots, k_all, v_all = [], [], []
    for s in live:
        all_slots += priv.add_seq(s, len(toks[s]))
        k_all.append(rows[s][0])
        v_all.append(rows[s][1])
    k_all, v_all = np.concatenate(k_all), np.concatenate(v_all)
    say("prefix cache: private layout store + decode")
    pa.pa_store_kvcache(torch.from_numpy(k_all).to(DEV), torch.from_numpy(v_all).to(DEV),
                        torch.tensor(all_slots, dtype=torch.int32, device=DEV), kp, vp)
    ptables, plens = priv.export(live, PWL.max_blocks_per_seq)
    out_private = pa.pa_decode(q, kp, vp, torch.from_numpy(np.asarray(ptables, dtype=np.int32)).to(DEV),
                               torch.tensor(plens, dtype=torch.int32, device=DEV), PWL.scale,
                               max_context_len=int(max(plens)))
    torch.cuda.synchronize()
    assert torch.equal(out_shared.view(torch.int16), out_private.view(torch.int16))

    # the oracle, from the rows themselves (never from a device cache)
    kr = np.zeros(shape, dtype=np.uint16)
    vr = np.zeros_like(kr)
    kr, vr = store_ref(k_all, v_all, all_slots, kr, vr)
    ref = decode_ref(host_u16(q).view(np.float16), kr.view(np.float16), vr.view(np.float16),
                     np.asarray(ptables, dtype=np.int32), np.asarray(plens, dtype=np.int32), PWL.scale)
    check_close(out_shared, ref, "prefix cache: shared layout")

"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* brute force: a scalar-loop second coding on tiny inputs;
* a library routine: with a contiguous (identity) block table, paged decode is
  ``torch.nn.functional.scaled_dot_product_attention`` in float64;
* invariants the pages state: placement of physical blocks does not change the
  result; shared prefix blocks give the same result as private copies;
* closed forms: one token, constant values, zero query, equal keys;
* the split-K merge identity;
* raw-bit store semantics, including NaN payloads.

A final test plants plausible mistakes in the oracle and checks that the pins
catch each one.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import (AllocatorModel, copy_blocks_ref, decode_bruteforce, decode_ref,
                    decode_splitk_ref, gather_sequence, store_bruteforce, store_ref, prefill_ref)
from tests.oracle_problems import after_step, build_problem

TINY_GQA = W.shrink(W.TINY, name="tiny_gqa", num_q_heads=8, num_kv_heads=2)
TINY_BS8 = W.shrink(W.TINY, name="tiny_bs8", block_size=8, num_blocks=128,
                    max_blocks_per_seq=8, num_q_heads=6, num_kv_heads=3, head_dim=32)
SMALL_PREFIX = W.shrink(W.PREFIX, name="small_prefix", num_seqs=6, num_q_heads=4,
                        num_kv_heads=2, head_dim=32, num_blocks=96,
                        max_blocks_per_seq=16)


def tiny_problem(wl):
    return build_problem(wl, plan_fn=lambda a: W.tiny_plan(a, wl))


def prefix_problem(wl=SMALL_PREFIX):
    return build_problem(wl, plan_fn=lambda a: W.prefix_plan(
        a, wl, prefix_tokens=48, suffix_range=(5, 30)))


def decoded(problem, fn=decode_ref, **kw):
    kc, vc = after_step(problem)
    return fn(problem["q"], kc.view(np.float16), vc.view(np.float16),
              problem["tables"], problem["lens"], problem["scale"], **kw)


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("wl", [W.TINY, TINY_GQA, TINY_BS8], ids=lambda w: w.name)
def test_bruteforce_matches_vectorised(wl):
    p = tiny_problem(wl)
    ref = decoded(p)
    brute = np.asarray(decoded(p, decode_bruteforce))
    assert ref.shape == brute.shape
    assert np.max(np.abs(ref - brute)) <= 1e-12


@pytest.mark.parametrize("wl", [W.TINY, TINY_BS8], ids=lambda w: w.name)
def test_store_bruteforce_matches(wl):
    p = tiny_problem(wl)
    a = store_ref(p["k_new"], p["v_new"], p["slots"], p["pre_k"], p["pre_v"])
    b = store_bruteforce(p["k_new"], p["v_new"], p["slots"], p["pre_k"], p["pre_v"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# library routine: contiguous layout == dense attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv,bs", [(4, 4, 16), (8, 2, 16), (6, 3, 8), (4, 1, 32)])
def test_identity_table_equals_sdpa(hq, hkv, bs):
    rng = np.random.default_rng(11)
    d, lens = 32, [1, 5, bs, 3 * bs + 1, 50]
    nblk = [-(-L // bs) for L in lens]
    NB = sum(nblk)
    kc = rng.standard_normal((NB, bs, hkv, d)).astype(np.float16)
    vc = rng.standard_normal((NB, bs, hkv, d)).astype(np.float16)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float16)
    M = max(nblk)
    tables = np.full((len(lens), M), -1, np.int32)
    start = 0
    for s, n in enumerate(nblk):            # sequence s owns a contiguous run
        tables[s, :n] = np.arange(start, start + n)
        start += n
    scale = 0.173
    out = decode_ref(q, kc, vc, tables, lens, scale)
    flat_k = torch.from_numpy(kc.astype(np.float64)).reshape(NB * bs, hkv, d)
    flat_v = torch.from_numpy(vc.astype(np.float64)).reshape(NB * bs, hkv, d)
    start = 0
    for s, L in enumerate(lens):
        kk = flat_k[start * bs:start * bs + L].permute(1, 0, 2).unsqueeze(0)
        vv = flat_v[start * bs:start * bs + L].permute(1, 0, 2).unsqueeze(0)
        qq = torch.from_numpy(q[s].astype(np.float64)).reshape(1, hq, 1, d)
        dense = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, scale=float(np.float32(scale)), enable_gqa=True)
        assert np.max(np.abs(dense.reshape(hq, d).numpy() - out[s])) <= 1e-12
        start += nblk[s]


# --------------------------------------------------------------------------
# invariants stated by the pages
# --------------------------------------------------------------------------

def permute_placement(kc, vc, tables, seed):
    """Move every physical block b to pi[b] and rewrite the tables to match."""
    NB = kc.shape[0]
    pi = np.random.default_rng(seed).permutation(NB)
    k2, v2 = np.empty_like(kc), np.empty_like(vc)
    k2[pi], v2[pi] = kc, vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    return k2, v2, t2


@pytest.mark.parametrize("wl", [W.TINY, TINY_GQA, TINY_BS8], ids=lambda w: w.name)
def test_placement_invariance_bitwise(wl):
    p = tiny_problem(wl)
    kc, vc = after_step(p)
    base = decode_ref(p["q"], kc.view(np.float16), vc.view(np.float16), p["tables"],
                      p["lens"], p["scale"])
    for seed in range(3):
        k2, v2, t2 = permute_placement(kc, vc, p["tables"], seed)
        moved = decode_ref(p["q"], k2.view(np.float16), v2.view(np.float16), t2,
                           p["lens"], p["scale"])
        assert np.array_equal(base, moved)


def unshare(kc, vc, tables, lens, block_size):
    """Give every sequence private copies of the blocks it shares."""
    owners = {}
    for s, row in enumerate(tables):
        for b in row[:-(-int(lens[s]) // block_size)]:
            owners.setdefault(int(b), []).append(s)
    shared = [b for b, o in owners.items() if len(o) > 1]
    extra = sum(len(owners[b]) for b in shared)
    NB = kc.shape[0]
    k2 = np.concatenate([kc, np.zeros((extra,) + kc.shape[1:], kc.dtype)])
    v2 = np.concatenate([vc, np.zeros((extra,) + vc.shape[1:], vc.dtype)])
    t2 = tables.copy()
    nxt = NB
    for s in range(len(tables)):
        for j in range(-(-int(lens[s]) // block_size)):
            b = int(tables[s, j])
            if b in shared:
                k2[nxt], v2[nxt] = kc[b], vc[b]
                t2[s, j] = nxt
                nxt += 1
    return k2, v2, t2, len(shared)


def test_shared_prefix_equals_private_copies():
    p = prefix_problem()
    kc, vc = after_step(p)
    k2, v2, t2, n_shared = unshare(kc, vc, p["tables"], p["lens"],
                                   SMALL_PREFIX.block_size)
    assert n_shared >= 2           # the prefix blocks really are shared
    a = decode_ref(p["q"], kc.view(np.float16), vc.view(np.float16), p["tables"],
                   p["lens"], p["scale"])
    b = decode_ref(p["q"], k2.view(np.float16), v2.view(np.float16), t2,
                   p["lens"], p["scale"])
    assert np.array_equal(a, b)


def test_prefix_plan_copy_on_write_happens_once():
    p = prefix_problem()
    assert p["cow_pairs"].shape == (1, 2)
    src, dst = p["cow_pairs"][0]
    kc, _ = after_step(p)
    # the copy holds the shared rows; the forked sequence's new token went
    # into the old block, the other sequence's new token into the copy
    n = SMALL_PREFIX.num_seqs
    bs = SMALL_PREFIX.block_size
    s62, s63 = p["slots"][n - 2], p["slots"][n - 1]
    assert s62 // bs == dst and s63 // bs == src
    assert s62 % bs == s63 % bs
    filled = s62 % bs
    assert np.array_equal(kc[dst, :filled], kc[src, :filled])


def test_softmax_weights_sum_to_one():
    p = tiny_problem(TINY_GQA)
    _, weights = decoded(p, return_weights=True)
    for s, w in enumerate(weights):
        assert w.shape[1] == p["lens"][s]
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
        assert np.all(w >= 0)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def _single_seq(L, hq=4, hkv=2, d=16, bs=16, seed=5):
    rng = np.random.default_rng(seed)
    nb = -(-L // bs) + 2
    kc = rng.standard_normal((nb, bs, hkv, d)).astype(np.float16)
    vc = rng.standard_normal((nb, bs, hkv, d)).astype(np.float16)
    q = rng.standard_normal((1, hq, d)).astype(np.float16)
    table = rng.permutation(nb)[None, :].astype(np.int32)
    return q, kc, vc, table, np.array([L], np.int32)


def test_single_token_returns_its_value_exactly():
    q, kc, vc, table, lens = _single_seq(1)
    out = decode_ref(q, kc, vc, table, lens, 0.25)
    v0 = vc[table[0, 0], 0].astype(np.float64)        # [Hkv, D]
    for h in range(4):
        assert np.array_equal(out[0, h], v0[h // 2])


def test_constant_values_give_that_value():
    q, kc, vc, table, lens = _single_seq(45)
    row = np.random.default_rng(1).standard_normal((2, 16)).astype(np.float16)
    vc[:] = row
    out = decode_ref(q, kc, vc, table, lens, 0.3)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - row[h // 2].astype(np.float64))) <= 1e-12


@pytest.mark.parametrize("zero", ["query", "keys"])
def test_uniform_scores_give_mean_value(zero):
    q, kc, vc, table, lens = _single_seq(37)
    if zero == "query":
        q[:] = 0
    else:
        kc[:] = np.float16(0.5)
    out = decode_ref(q, kc, vc, table, lens, 0.3)
    V = gather_sequence(vc, table[0], 37).astype(np.float64)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - V[:, h // 2].mean(axis=0))) <= 1e-12


def test_empty_context_gives_zeros():
    q, kc, vc, table, _ = _single_seq(5)
    out = decode_ref(q, kc, vc, table, np.array([0], np.int32), 0.3)
    assert np.array_equal(out, np.zeros_like(out))


# --------------------------------------------------------------------------
# split-K merge identity
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 16, 512])
def test_splitk_merge_matches_single_pass(chunk):
    q, kc, vc, table, lens = _single_seq(1200, hq=8, hkv=2, d=32, seed=9)
    q = (q.astype(np.float32) * 3).astype(np.float16)   # sharper softmax
    ref = decode_ref(q, kc, vc, table, lens, 0.2)
    split = decode_splitk_ref(q, kc, vc, table, lens, 0.2, chunk)
    assert np.max(np.abs(split - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# --------------------------------------------------------------------------
# store semantics
# --------------------------------------------------------------------------

def _store_case(seed=3):
    rng = np.random.default_rng(seed)
    NB, bs, hkv, d = 6, 4, 2, 8
    kc = W.nan_sentinel_fp16((NB, bs, hkv, d)).numpy().view(np.uint16)
    vc = kc.copy() ^ 0x0001
    k = rng.standard_normal((5, hkv, d)).astype(np.float16)
    v = rng.standard_normal((5, hkv, d)).astype(np.float16)
    return kc, vc, k, v, bs


def test_store_writes_rows_and_nothing_else():
    kc, vc, k, v, bs = _store_case()
    slots = np.array([0, 7, -1, 23, 9], np.int32)
    k2, v2 = store_ref(k, v, slots, kc, vc)
    touched = np.zeros(kc.shape[:2], bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), bs)
        touched[b, o] = True
        assert np.array_equal(k2[b, o], k[t].view(np.uint16))
        assert np.array_equal(v2[b, o], v[t].view(np.uint16))
    assert np.array_equal(k2[~touched], kc[~touched])      # NaN payloads kept
    assert np.array_equal(v2[~touched], vc[~touched])


def test_store_rejects_bad_slots():
    kc, vc, k, v, _ = _store_case()
    with pytest.raises(ValueError):
        store_ref(k[:2], v[:2], np.array([3, 3]), kc, vc)
    with pytest.raises(ValueError):
        store_ref(k[:1], v[:1], np.array([kc.shape[0] * kc.shape[1]]), kc, vc)


def test_store_then_gather_round_trip():
    """Rows stored at the allocator's slots read back in logical order."""
    alloc = AllocatorModel(20, 4, 10, W.free_order(20, 8))
    slots = alloc.add_seq(0, 13)
    kc, vc, _, _, _ = _store_case()
    kc = np.zeros((20, 4, 2, 8), np.uint16)
    rows = np.random.default_rng(2).standard_normal((13, 2, 8)).astype(np.float16)
    k2, _ = store_ref(rows, rows, slots, kc, kc)
    table, lens = alloc.export([0], 10)
    back = gather_sequence(k2, table[0], lens[0])
    assert np.array_equal(back, rows.view(np.uint16))


def test_copy_blocks_copies_whole_blocks_in_order():
    kc, vc, _, _, _ = _store_case()
    k2, v2 = copy_blocks_ref(kc, vc, [(1, 4), (4, 5)])
    assert np.array_equal(k2[4], kc[1]) and np.array_equal(k2[5], kc[1])
    assert np.array_equal(v2[5], vc[1])
    assert np.array_equal(k2[:4], kc[:4])


# --------------------------------------------------------------------------
# the pins catch plausible mistakes planted in the oracle
# --------------------------------------------------------------------------

def _mutant_gathers():
    real = oracle.attention.gather_sequence

    def drop_last(cache, row, L, block_size=None):
        rows = real(cache, row, L, block_size).copy()
        if L >= 2:                      # off by one: position L-2 read twice
            rows[-1] = rows[-2]
        return rows

    def swapped_offset(cache, row, L, block_size=None):
        nb, bs = cache.shape[:2]
        n = -(-L // bs)
        rows = cache[np.asarray(row[:n])].transpose(1, 0, 2, 3).reshape(n * bs, *cache.shape[2:])
        return rows[:L]

    def reversed_in_block(cache, row, L, block_size=None):
        nb, bs = cache.shape[:2]
        n = -(-L // bs)
        return cache[np.asarray(row[:n])][:, ::-1].reshape(n * bs, *cache.shape[2:])[:L]

    def heads_swapped(cache, row, L, block_size=None):
        return real(cache, row, L, block_size)[:, ::-1]

    return {"drop_last": drop_last, "swapped_offset": swapped_offset,
            "reversed_in_block": reversed_in_block, "heads_swapped": heads_swapped}


@pytest.mark.parametrize("name", sorted(_mutant_gathers()))
def test_pins_catch_planted_mistake(name, monkeypatch):
    mutant = _mutant_gathers()[name]
    p = tiny_problem(TINY_GQA)
    brute = np.asarray(decoded(p, decode_bruteforce))
    monkeypatch.setattr(oracle.attention, "gather_sequence", mutant)
    with np.errstate(invalid="ignore"):
        bad = decoded(p)
        diff = np.abs(bad - brute)
    assert np.isnan(diff).any() or diff.max() > 1e-3


def _head_major(c):
    return np.ascontiguousarray(np.swapaxes(c, 1, 2))


def test_head_major_store_puts_each_head_in_its_block_run():
    """Brute force on positions: token t's head h lands at [slot // bs, h,
    slot % bs] of a head-major cache, and nothing else changes."""
    rng = np.random.default_rng(21)
    NB, bs, H, D = 5, 4, 3, 8
    kc = rng.integers(0, 1 << 16, size=(NB, H, bs, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, H, bs, D), dtype=np.uint16)
    slots = [7, -1, 0, 19, 12]
    k = rng.integers(0, 1 << 16, size=(len(slots), H, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(len(slots), H, D), dtype=np.uint16)
    k2, v2 = store_ref(k, v, slots, kc, vc, layout="head")
    expect_k, expect_v = kc.copy(), vc.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(H):
            for d in range(D):
                expect_k[s // bs, h, s % bs, d] = k[t, h, d]
                expect_v[s // bs, h, s % bs, d] = v[t, h, d]
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    # The same writes seen slot-major: storing into the transposed cache.
    ks, vs = store_ref(k, v, slots, np.swapaxes(kc, 1, 2), np.swapaxes(vc, 1, 2))
    assert np.array_equal(_head_major(ks), k2) and np.array_equal(_head_major(vs), v2)


def test_layouts_give_identical_attention():
    """The layout only moves rows: decode and prefill over a head-major copy
    of the caches equal the slot-major results bit for bit."""
    rng = np.random.default_rng(22)
    NB, bs, Hkv, D, G = 12, 8, 2, 16, 2
    kc = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    vc = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    tables = [[4, 9, 1, 0], [11, 2, 7, 3]]
    lens = [29, 17]
    q = rng.standard_normal((2, Hkv * G, D)).astype(np.float16)
    a = decode_ref(q, kc, vc, tables, lens, 0.25)
    b = decode_ref(q, _head_major(kc), _head_major(vc), tables, lens, 0.25, layout="head")
    assert np.array_equal(a, b)
    qp = rng.standard_normal((7, Hkv * G, D)).astype(np.float16)
    starts = [0, 4, 7]
    a = prefill_ref(qp, kc, vc, tables, lens, starts, 0.25)
    b = prefill_ref(qp, _head_major(kc), _head_major(vc), tables, lens, starts, 0.25, layout="head")
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        decode_ref(q, kc, vc, tables, lens, 0.25, layout="diagonal")

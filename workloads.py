"""Seeded synthetic workloads for paged KV-cache decode.

This module is the only code shared by the oracle side and the HIP side.  It
holds no attention, store or allocator arithmetic: it draws random numbers,
fixes shapes and sizes, and sequences allocator *calls* (which block a
sequence receives is decided by whichever allocator is driven).

Workloads (sizes follow the scope of the build; seeds are fixed readings):

tiny    fp16, 4 sequences with context lengths {1, 7, 16, 33}, 4 query heads =
        4 KV heads, head_dim 64, block 16, 64 blocks in a seeded shuffled
        order.  The L-1 earlier tokens of each sequence are stored first; the
        step then stores 4 new tokens and decodes.
mha     fp16, 32 sequences x 2048 tokens, 32 query = 32 KV heads, head_dim 128,
        block 16, 8192 blocks shuffled.
mix     fp16 GQA 32/8, head_dim 128, 32 sequences with lengths U{1..8192},
        at most 512 blocks per sequence, 32768 blocks fragmented by a seeded
        trace of 10 000 add / append / free calls.
prefix  fp16 GQA 32/8, head_dim 128, 64 sequences sharing one 2000-token
        prefix (125 blocks) plus private suffixes U{50..200}; sequence 63 is a
        fork of sequence 62 taken on a partly filled block, so the step's
        append by 62 triggers one copy-on-write.  1024 blocks.
long    fp16 GQA 32/8, head_dim 128, 4 sequences x 131072 tokens, block 16
        (also 8 and 64), a pool of 1.25x the blocks needed, shuffled.
"""

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    seed: int
    layers: int = 32

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))


TINY = Workload("tiny", 4, 4, 4, 64, 16, 64, 4, seed=0, layers=1)
MHA = Workload("mha", 32, 32, 32, 128, 16, 8192, 128, seed=1)
MIX = Workload("mix", 32, 32, 8, 128, 16, 32768, 512, seed=2)
PREFIX = Workload("prefix", 64, 32, 8, 128, 16, 1024, 144, seed=3)
_LONG_TOKENS = 131072


def long_workload(block_size=16):
    seed = {16: 4, 8: 5, 64: 6}.get(block_size, 7)
    per_seq = _LONG_TOKENS // block_size
    return Workload("long_bs%d" % block_size, 4, 32, 8, 128, block_size,
                    num_blocks=(per_seq * 4 * 5) // 4, max_blocks_per_seq=per_seq,
                    seed=seed)


LONG = long_workload(16)
# Chunked prefill: every sequence prefills the last chunk (256 tokens, the
# pages' prefill chunk size) of a 2048-token prompt; MHA and grouped heads.
PREFILL_CHUNK = 256
PREFILL_CONTEXT = 2048
PREFILL_MHA = Workload("prefill_mha", 32, 32, 32, 128, 16, 4160, 128, seed=5)
PREFILL_GQA = Workload("prefill_gqa", 32, 32, 8, 128, 16, 4160, 128, seed=6)
PREFILLS = {w.name: w for w in (PREFILL_MHA, PREFILL_GQA)}
ALL = {w.name: w for w in (TINY, MHA, MIX, PREFIX, LONG)}

TINY_LENS = (1, 7, 16, 33)
PREFIX_TOKENS = 2000
PREFIX_HOLDER = 1 << 40      # sequence id of the request that owns the prefix
BACKGROUND_BASE = 1 << 41    # sequence ids of the fragmenting trace


# --------------------------------------------------------------------------
# random numbers
# --------------------------------------------------------------------------

def free_order(num_blocks, seed):
    """Seeded permutation of block numbers: the initial free-list order."""
    return np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)


def normal_fp16(shape, seed, device="cpu"):
    """N(0, 1) drawn in float32 by a seeded torch generator, rounded to fp16."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.float16)


def nan_sentinel_fp16(shape, device="cpu"):
    """fp16 array of assorted NaN bit patterns (quiet and signalling, +/-)."""
    import torch
    n = int(np.prod(shape))
    i = torch.arange(n, device=device, dtype=torch.int32)
    payload = 1 + (i % 1023)                  # mantissa never 0: always NaN
    sign = ((i // 1023) % 2) << 15
    bits = (0x7C00 | payload | sign).to(torch.int32)
    bits = torch.where(bits >= 32768, bits - 65536, bits).to(torch.int16)
    return bits.view(torch.float16).reshape(tuple(shape))


def value_seed(workload, stream):
    """Distinct generator seed per (workload, tensor role)."""
    roles = {"q": 1, "k_new": 2, "v_new": 3, "k_cache": 4, "v_cache": 5,
             "k_prior": 6, "v_prior": 7}
    return workload.seed * 1000 + roles[stream]


# --------------------------------------------------------------------------
# allocator call sequences (work with any allocator exposing add_seq, fork,
# append_slot, free_seq, export; failures raise an exception whose ``code``
# attribute names the failure)
# --------------------------------------------------------------------------

@dataclass
class StepPlan:
    seq_ids: list            # batch order
    prior_slots: dict        # seq id -> slots of tokens stored before the step
    prior_rows: dict         # seq id -> [(value source key, row index)] per prior slot
    step_slots: list         # slot of the step's new token, batch order
    cow_pairs: list          # [(src, dst)] copies to do before the step's store
    context_lens: list       # after the step
    block_tables: list       # after the step, rows padded with -1
    trace_stats: dict = None


def _code(exc):
    return getattr(exc, "code", None)


def _append_step(alloc, seq_ids):
    slots, cows = [], []
    for s in seq_ids:
        slot, src, dst = alloc.append_slot(s)
        slots.append(slot)
        if src >= 0:
            cows.append((src, dst))
    return slots, cows


def _plain_plan(alloc, workload, lens):
    seq_ids = list(range(len(lens)))
    prior, rows = {}, {}
    for s, L in zip(seq_ids, lens):
        prior[s] = list(alloc.add_seq(s, L - 1))
        rows[s] = [(s, p) for p in range(L - 1)]
    step_slots, cows = _append_step(alloc, seq_ids)
    tables, out_lens = alloc.export(seq_ids, workload.max_blocks_per_seq)
    return StepPlan(seq_ids, prior, rows, step_slots, cows, list(out_lens), tables)


def tiny_plan(alloc, workload=TINY):
    return _plain_plan(alloc, workload, TINY_LENS)


def uniform_plan(alloc, workload, context_len):
    return _plain_plan(alloc, workload, [context_len] * workload.num_seqs)


def mix_lengths(workload=MIX):
    rng = np.random.default_rng(workload.seed + 100)
    return [int(x) for x in rng.integers(1, 8192 + 1, size=workload.num_seqs)]


def fragment_pool(alloc, seed, n_ops=10000, max_tokens=8192, append_max=256):
    """Seeded trace of add / append / free calls that scatters the free list.

    Each call is add (35 %), append a run of tokens to a random live sequence
    (35 %) or free a random live sequence (30 %).  A call that runs out of
    blocks becomes a free of a random live sequence.  Returns the live
    sequence ids, oldest first.
    """
    rng = np.random.default_rng(seed)
    live, next_id = [], BACKGROUND_BASE
    for _ in range(n_ops):
        r = rng.random()
        try:
            if r < 0.35 or not live:
                n = int(rng.integers(1, max_tokens + 1))
                alloc.add_seq(next_id, n)
                live.append(next_id)
                next_id += 1
            elif r < 0.70:
                seq = live[int(rng.integers(len(live)))]
                for _ in range(int(rng.integers(1, append_max + 1))):
                    try:
                        alloc.append_slot(seq)
                    except Exception as exc:  # noqa: BLE001
                        if _code(exc) == "SEQ_LIMIT":
                            break
                        raise
            else:
                alloc.free_seq(live.pop(int(rng.integers(len(live)))))
        except Exception as exc:  # noqa: BLE001
            if _code(exc) != "OUT_OF_BLOCKS":
                raise
            if live:
                alloc.free_seq(live.pop(int(rng.integers(len(live)))))
    return live


def _retry_freeing(alloc, live, fn):
    while True:
        try:
            return fn()
        except Exception as exc:  # noqa: BLE001
            if _code(exc) != "OUT_OF_BLOCKS" or not live:
                raise
            alloc.free_seq(live.pop(0))


def mix_plan(alloc, workload=MIX, n_ops=10000):
    live = fragment_pool(alloc, workload.seed + 200, n_ops=n_ops)
    lens = mix_lengths(workload)
    seq_ids = list(range(workload.num_seqs))
    prior, rows = {}, {}
    for s, L in zip(seq_ids, lens):
        prior[s] = list(_retry_freeing(alloc, live, lambda s=s, L=L: alloc.add_seq(s, L - 1)))
        rows[s] = [(s, p) for p in range(L - 1)]
    step_slots, cows = [], []
    for s in seq_ids:
        slot, src, dst = _retry_freeing(alloc, live, lambda s=s: alloc.append_slot(s))
        step_slots.append(slot)
        if src >= 0:
            cows.append((src, dst))
    tables, out_lens = alloc.export(seq_ids, workload.max_blocks_per_seq)
    return StepPlan(seq_ids, prior, rows, step_slots, cows, list(out_lens), tables,
                    trace_stats={"background_seqs": len(live)})


def prefix_suffix_lengths(workload=PREFIX, suffix_range=(50, 200)):
    lo, hi = suffix_range
    rng = np.random.default_rng(workload.seed + 300)
    lens = [int(x) for x in rng.integers(lo, hi + 1, size=workload.num_seqs - 1)]
    while lens[-1] % workload.block_size == 0:       # the forked sequence ends mid-block
        lens[-1] = int(rng.integers(lo, hi + 1))
    return lens


def prefix_plan(alloc, workload=PREFIX, prefix_tokens=PREFIX_TOKENS,
                suffix_range=(50, 200)):
    """All sequences share a prefix; the last is a fork of the one before it,
    taken while that one's last block is partly filled."""
    n = workload.num_seqs
    suffix = prefix_suffix_lengths(workload, suffix_range)
    prior, rows = {}, {}
    holder_slots = list(alloc.add_seq(PREFIX_HOLDER, prefix_tokens))
    for s in range(n - 1):
        alloc.fork(PREFIX_HOLDER, s)
        own = [alloc.append_slot(s) for _ in range(suffix[s])]
        if any(src >= 0 for _, src, _ in own):
            raise AssertionError("a suffix append copied a shared block")
        prior[s] = holder_slots + [slot for slot, _, _ in own]
        rows[s] = [("prefix", p) for p in range(prefix_tokens)] + \
                  [(s, p) for p in range(suffix[s])]
    alloc.fork(n - 2, n - 1)
    prior[n - 1] = []           # shares every prior row with sequence n-2
    rows[n - 1] = []
    alloc.free_seq(PREFIX_HOLDER)
    seq_ids = list(range(n))
    step_slots, cows = _append_step(alloc, seq_ids)
    tables, out_lens = alloc.export(seq_ids, workload.max_blocks_per_seq)
    return StepPlan(seq_ids, prior, rows, step_slots, cows, list(out_lens), tables)


def plan_for(workload, alloc):
    if workload.name == "tiny":
        return tiny_plan(alloc, workload)
    if workload.name == "mha":
        return uniform_plan(alloc, workload, 2048)
    if workload.name == "mix":
        return mix_plan(alloc, workload)
    if workload.name == "prefix":
        return prefix_plan(alloc, workload)
    if workload.name.startswith("long"):
        return uniform_plan(alloc, workload, _LONG_TOKENS)
    raise KeyError(workload.name)


def prior_scatter(plan):
    """Flatten the plan's earlier tokens into (slots, row keys, distinct keys).

    ``keys[i]`` names the value row that belongs in ``slots[i]``; rows shared
    by several sequences (the common prefix) appear once in ``distinct``.
    """
    slots, keys, owner = [], [], {}
    for s in plan.seq_ids:
        for slot, key in zip(plan.prior_slots[s], plan.prior_rows[s]):
            if slot in owner:               # a shared block: stored once
                if owner[slot] != key:
                    raise AssertionError("two rows planned for one slot")
                continue
            owner[slot] = key
            slots.append(slot)
            keys.append(key)
    distinct, index = [], {}
    for key in keys:
        if key not in index:
            index[key] = len(distinct)
            distinct.append(key)
    return slots, [index[k] for k in keys], distinct


def shrink(workload, **kw):
    """A copy of ``workload`` with some sizes changed (for small test cases)."""
    return replace(workload, **kw)

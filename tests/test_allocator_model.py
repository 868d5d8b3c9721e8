"""Pins of the oracle's block-manager model (``oracle.AllocatorModel``).

Checked against what the pages state (golden fixtures under tests/golden/),
against closed forms, and against invariants that must hold after every
operation of a random trace.
"""

import json
import os
from collections import Counter

import pytest
from hypothesis import given, settings, strategies as st

import workloads as W
from oracle import AllocatorModel, AllocError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_invariants(m):
    """Every block is either free or referenced; counts match the tables."""
    refs = Counter()
    for blocks, n in m.seqs.values():
        assert len(blocks) == -(-n // m.block_size)
        assert len(blocks) <= m.max_blocks_per_seq
        refs.update(blocks)
    free = list(m.free)
    assert len(free) == len(set(free))
    for b in range(m.num_blocks):
        assert m.refcounts[b] == refs.get(b, 0)
        assert (m.refcounts[b] == 0) == (b in set(free))
    assert len(free) + sum(1 for r in m.refcounts if r > 0) == m.num_blocks


def snapshot(m):
    return (list(m.free), list(m.refcounts),
            {k: (list(v[0]), v[1]) for k, v in m.seqs.items()}, m.cow_copies)


# --------------------------------------------------------------------------
# the pages' printed values
# --------------------------------------------------------------------------

def test_128k_context_takes_8192_blocks():
    g = golden("blocks_128k.json")
    m = AllocatorModel(g["blocks"], g["block_size"], g["blocks"])
    m.add_seq(0, g["context_tokens"])
    assert len(m.seq_blocks(0)) == g["blocks"]
    assert m.num_free() == 0
    with pytest.raises(AllocError) as e:           # the next token needs a block
        m.append_slot(0)
    assert e.value.code == "SEQ_LIMIT"


def test_abc_scenario():
    """A and B share the system prompt, C does not; B finishes first."""
    g = golden("abc_scenario.json")
    facts, read = g["page_facts"], g["readings"]
    bs = read["block_size"]
    trad_blocks = 3 * facts["traditional_prealloc_tokens_per_request"] // bs
    m = AllocatorModel(trad_blocks, bs, trad_blocks, W.free_order(trad_blocks, 5))
    SYS = 99
    m.add_seq(SYS, read["system_prompt_tokens"])
    m.fork(SYS, "A")
    m.fork(SYS, "B")
    m.free_seq(SYS)
    m.add_seq("C", read["question_tokens"]["C"])
    prefix_blocks = m.seq_blocks("A")
    assert prefix_blocks == m.seq_blocks("B")
    assert all(m.refcount(b) == 2 for b in prefix_blocks)
    peak = 0
    for name in ("A", "B", "C"):
        n_new = read["question_tokens"][name] if name != "C" else 0
        n_new += facts["generated_tokens"][name]
        for _ in range(n_new):
            m.append_slot(name)
            check_invariants(m)
            peak = max(peak, m.num_blocks - m.num_free())
    # only the partly filled prefix block is ever copied, by the first writer
    assert m.cow_copies == 1
    a_blocks = m.seq_blocks("A")
    b_only = set(m.seq_blocks("B")) - set(a_blocks)
    m.free_seq("B")                    # B finishes first ...
    check_invariants(m)
    assert all(b in m.free for b in b_only)
    assert all(m.refcount(b) == 1 for b in a_blocks)   # ... A keeps its pages
    assert m.seq_blocks("A") == a_blocks
    assert peak < facts["paged_total_below_fraction_of_traditional"] * trad_blocks


def test_shared_page_survives_one_sharer_finishing():
    """Reference counts stop one sharer from releasing another's pages."""
    m = AllocatorModel(32, 4, 16)
    m.add_seq("x", 10)
    m.fork("x", "y")
    shared = m.seq_blocks("x")
    m.free_seq("x")
    assert not any(b in m.free for b in shared)
    m.free_seq("y")
    assert all(b in m.free for b in shared)
    check_invariants(m)


def test_finished_request_returns_all_blocks_in_order():
    m = AllocatorModel(10, 4, 10, list(range(9, -1, -1)))
    m.add_seq(1, 9)                      # takes 9, 8, 7
    m.add_seq(2, 4)                      # takes 6
    assert m.seq_blocks(1) == [9, 8, 7]
    m.free_seq(1)
    assert list(m.free) == [5, 4, 3, 2, 1, 0, 9, 8, 7]


# --------------------------------------------------------------------------
# closed forms and exact semantics
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bs", [1, 4, 16])
@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 100])
def test_blocks_and_slots_closed_form(bs, n):
    m = AllocatorModel(200, bs, 200, W.free_order(200, 3))
    slots = m.add_seq(0, n)
    blocks = m.seq_blocks(0)
    assert len(blocks) == -(-n // bs)
    assert slots == [blocks[p // bs] * bs + p % bs for p in range(n)]
    assert len(set(slots)) == n


def test_append_takes_new_block_only_when_full():
    m = AllocatorModel(8, 4, 8)
    m.add_seq(0, 3)
    assert m.append_slot(0) == (3, -1, -1)          # fills block 0
    assert m.num_free() == 7
    assert m.append_slot(0) == (4, -1, -1)          # block 1 taken now
    assert m.num_free() == 6


def test_copy_on_write_first_writer_copies_last_writes_in_place():
    m = AllocatorModel(8, 4, 8)
    m.add_seq("p", 6)                  # blocks 0 (full) and 1 (2 of 4 filled)
    m.fork("p", "c")
    slot, src, dst = m.append_slot("c")
    assert (src, dst) == (1, 2)        # the writer moves to a fresh block
    assert slot == 2 * 4 + 2
    assert m.seq_blocks("c") == [0, 2] and m.seq_blocks("p") == [0, 1]
    assert m.append_slot("p") == (1 * 4 + 2, -1, -1)   # now sole owner
    assert m.refcount(0) == 2 and m.refcount(1) == 1 and m.refcount(2) == 1
    check_invariants(m)


def test_full_shared_block_is_never_copied():
    m = AllocatorModel(8, 4, 8)
    m.add_seq("p", 8)
    m.fork("p", "c")
    assert m.append_slot("c")[1:] == (-1, -1)
    assert m.append_slot("p")[1:] == (-1, -1)
    assert m.cow_copies == 0


@pytest.mark.parametrize("op", ["add_big", "add_limit", "append_oob", "cow_oob",
                                "unknown", "exists", "fork_unknown", "free_twice"])
def test_failed_operation_leaves_state_unchanged(op):
    m = AllocatorModel(6, 4, 3)
    m.add_seq("a", 6)
    m.fork("a", "b")
    m.add_seq("c", 12)                 # pool now has 6 - 2 - 3 = 1 free block
    m.add_seq("d", 4)                  # and now none
    before = snapshot(m)
    calls = {
        "add_big": (lambda: m.add_seq("e", 5), "OUT_OF_BLOCKS"),
        "add_limit": (lambda: m.add_seq("e", 13), "SEQ_LIMIT"),
        "append_oob": (lambda: m.append_slot("d"), "OUT_OF_BLOCKS"),
        "cow_oob": (lambda: m.append_slot("a"), "OUT_OF_BLOCKS"),
        "unknown": (lambda: m.append_slot("zz"), "UNKNOWN_SEQ"),
        "exists": (lambda: m.add_seq("a", 1), "SEQ_EXISTS"),
        "fork_unknown": (lambda: m.fork("zz", "e"), "UNKNOWN_SEQ"),
        "free_twice": (lambda: (m.free_seq("d"), m.free_seq("d")), "UNKNOWN_SEQ"),
    }
    fn, code = calls[op]
    with pytest.raises(AllocError) as e:
        fn()
    assert e.value.code == code
    if op != "free_twice":
        assert snapshot(m) == before
    check_invariants(m)


def test_stats_closed_form():
    m = AllocatorModel(10, 4, 10)
    m.add_seq(0, 5)                    # 2 blocks, 5 of 8 slots filled
    m.add_seq(1, 4)                    # 1 block, full
    m.fork(0, 2)                       # shares both blocks
    st_ = m.stats()
    assert st_["used_blocks"] == 3 and st_["shared_blocks"] == 2
    assert st_["utilisation"] == pytest.approx(0.3)
    assert st_["internal_fragmentation"] == pytest.approx(3 / 12)
    assert st_["logical_tokens"] == 14 and st_["stored_tokens"] == 9


def test_export_pads_with_minus_one_and_checks_stride():
    m = AllocatorModel(10, 4, 10, list(range(10)))
    m.add_seq(7, 9)
    tables, lens = m.export([7], 5)
    assert tables == [[0, 1, 2, -1, -1]] and lens == [9]
    with pytest.raises(AllocError) as e:
        m.export([7], 2)
    assert e.value.code == "SHAPE"


def test_bad_initial_order_rejected():
    with pytest.raises(AllocError):
        AllocatorModel(4, 4, 4, [0, 1, 1, 3])


# --------------------------------------------------------------------------
# invariants under random traces
# --------------------------------------------------------------------------

ops = st.lists(st.tuples(st.sampled_from(["add", "fork", "append", "free"]),
                         st.integers(0, 7), st.integers(0, 7), st.integers(0, 40)),
               max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4, 8]), seed=st.integers(0, 5))
def test_random_trace_keeps_invariants(ops, bs, seed):
    m = AllocatorModel(24, bs, 6, W.free_order(24, seed))
    for kind, a, b, n in ops:
        before = snapshot(m)
        try:
            if kind == "add":
                m.add_seq(a, n)
            elif kind == "fork":
                m.fork(a, b)
            elif kind == "append":
                m.append_slot(a)
            else:
                m.free_seq(a)
        except AllocError:
            assert snapshot(m) == before
        check_invariants(m)


def test_fragmenting_trace_is_deterministic():
    def run():
        m = AllocatorModel(4096, 16, 512, W.free_order(4096, 2))
        live = W.fragment_pool(m, seed=7, n_ops=300)
        return live, list(m.free)
    assert run() == run()

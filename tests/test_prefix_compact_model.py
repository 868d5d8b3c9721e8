"""Pins of the oracle model's prefix cache and compaction.

The hash is pinned to FNV-1a's published test vectors.  Prefix sharing and
compaction are pinned through what they must preserve: a simulated cache in
which every stored token writes its id into its slot must, gathered through
any live sequence's block table, give back exactly that sequence's tokens —
whatever was shared, copied on write or moved.  Hit counts are pinned to a
brute force over the live sequences' token lists.
"""

from collections import Counter

import pytest
from hypothesis import given, settings, strategies as st

from oracle import AllocatorModel, AllocError, block_hash, fnv1a64


# --------------------------------------------------------------------------
# FNV-1a, 64-bit: the published test vectors of its authors' test suite
# --------------------------------------------------------------------------

@pytest.mark.parametrize("data,expect", [
    (b"", 0xCBF29CE484222325),
    (b"a", 0xAF63DC4C8601EC8C),
    (b"foobar", 0x85944171F73967E8),
])
def test_fnv1a64_published_vectors(data, expect):
    assert fnv1a64(data) == expect


def test_block_hash_byte_layout():
    # parent hash as 8 little-endian bytes, then 4 little-endian bytes a token
    data = (0x0102030405060708).to_bytes(8, "little") + (7).to_bytes(4, "little") \
        + (0xFFFFFFFF).to_bytes(4, "little")
    assert block_hash(0x0102030405060708, [7, -1]) == fnv1a64(data)
    assert block_hash(0, [1, 2]) != block_hash(0, [2, 1])
    assert block_hash(1, [1, 2]) != block_hash(0, [1, 2])


# --------------------------------------------------------------------------
# a content simulation: slot -> token id written there
# --------------------------------------------------------------------------

class Sim:
    """Drives a model and a fake cache.  ``tokens[s]`` is what sequence s
    holds logically; ``reg[s]`` the token list it was registered with (a fork
    inherits its parent's), used by the brute-force hit count."""

    def __init__(self, num_blocks, block_size, max_blocks):
        self.m = AllocatorModel(num_blocks, block_size, max_blocks)
        self.content = {}
        self.tokens = {}
        self.reg = {}

    def add(self, seq, toks):
        slots, n_cached = self.m.add_seq_tokens(seq, toks)
        for p in range(n_cached, len(toks)):        # only uncached tokens are stored
            self.content[slots[p]] = toks[p]
        self.tokens[seq] = list(toks)
        self.reg[seq] = list(toks)
        return slots, n_cached

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])
        self.reg[child] = list(self.reg[parent])

    def append(self, seq, tok):
        slot, src, dst = self.m.append_slot(seq)
        if src >= 0:
            self.copy_block(src, dst)
        self.content[slot] = tok
        self.tokens[seq].append(tok)

    def free(self, seq):
        self.m.free_seq(seq)
        del self.tokens[seq], self.reg[seq]

    def copy_block(self, src, dst):
        bs = self.m.block_size
        for o in range(bs):
            if src * bs + o in self.content:
                self.content[dst * bs + o] = self.content[src * bs + o]

    def compact(self):
        pairs = self.m.compact()
        for src, dst in pairs:                      # disjoint, so any order works
            self.copy_block(src, dst)
        return pairs

    def check(self):
        bs = self.m.block_size
        for seq, toks in self.tokens.items():
            blocks, n = self.m.seqs[seq]
            assert n == len(toks)
            got = [self.content.get(blocks[p // bs] * bs + p % bs) for p in range(n)]
            assert got == toks, seq
        refs = Counter(b for blocks, _ in self.m.seqs.values() for b in blocks)
        assert all(self.m.refcounts[b] == refs.get(b, 0) for b in range(self.m.num_blocks))
        assert sorted(self.m.free) == [b for b in range(self.m.num_blocks) if refs.get(b, 0) == 0]
        for h, b in self.m.index.items():           # cached blocks are live and hold their key
            assert self.m.refcounts[b] > 0 and self.m.block_key[b][0] == h
            assert [self.content.get(b * bs + o) for o in range(bs)] == list(self.m.block_key[b][2])

    def expected_hits(self, toks):
        """Full blocks of ``toks`` that equal the start of a live sequence's
        registered token list, block for block from the first."""
        bs = self.m.block_size
        best = 0
        for reg in self.reg.values():
            j = 0
            while (j + 1) * bs <= min(len(toks), len(reg)) and \
                    toks[:(j + 1) * bs] == reg[:(j + 1) * bs]:
                j += 1
            best = max(best, j)
        return best * bs


def test_shared_prefix_reuses_blocks_and_counts_hits():
    s = Sim(32, 4, 8)
    _, c1 = s.add(1, list(range(10)))               # blocks 0,1 full, 2 partial
    _, c2 = s.add(2, list(range(8)) + [50, 51, 52])
    _, c3 = s.add(3, [0, 1, 2, 9] + list(range(4, 10)))   # differs in block 0
    assert (c1, c2, c3) == (0, 8, 0)
    b1, b2, b3 = (s.m.seqs[k][0] for k in (1, 2, 3))
    assert b2[:2] == b1[:2] and b2[2] != b1[2]
    assert not set(b3) & set(b1)
    assert [s.m.refcounts[b] for b in b1] == [2, 2, 1]
    assert s.m.prefix_stats() == (31, 8, 4)         # blocks 0,1 of seq 1 and 3's two
    s.check()


def test_second_block_needs_its_parent_to_match():
    s = Sim(32, 2, 8)
    s.add(1, [1, 2, 3, 4])
    _, c = s.add(2, [9, 9, 3, 4])                   # same second block, other parent
    assert c == 0
    assert s.m.seqs[2][0][1] != s.m.seqs[1][0][1]
    s.check()


def test_cached_block_dies_with_its_last_user():
    s = Sim(16, 2, 8)
    s.add(1, [5, 6, 7])
    s.add(2, [5, 6, 8])                             # shares block 0
    s.free(1)
    _, c = s.add(3, [5, 6])                         # still cached through seq 2
    assert c == 2
    s.free(2)
    s.free(3)
    assert s.m.prefix_stats()[2] == 0
    _, c = s.add(4, [5, 6])
    assert c == 0
    s.check()


def test_whole_sequence_cached_and_appends_copy_nothing_shared():
    s = Sim(16, 4, 8)
    s.add(1, list(range(8)))
    _, c = s.add(2, list(range(8)))
    assert c == 8 and s.m.seqs[2][0] == s.m.seqs[1][0]
    s.append(2, 100)                                # starts a block of its own
    s.append(1, 200)
    assert s.m.cow_copies == 0
    s.check()


def test_failed_add_leaves_state_unchanged():
    s = Sim(4, 2, 8)
    s.add(1, [1, 2, 3, 4, 5])                       # 3 blocks
    before = (list(s.m.free), list(s.m.refcounts), dict(s.m.index), s.m.prefix_stats())
    with pytest.raises(AllocError) as e:
        s.m.add_seq_tokens(2, [1, 2, 3, 4, 7, 8, 9])  # 2 hits, needs 2 new, 1 free
    assert e.value.code == "OUT_OF_BLOCKS"
    assert (list(s.m.free), list(s.m.refcounts), dict(s.m.index), s.m.prefix_stats()) == before
    _, c = s.add(2, [1, 2, 3, 4, 7])                # 2 hits + 1 new fits
    assert c == 4
    s.check()


def test_compaction_moves_only_high_blocks_into_holes():
    s = Sim(12, 2, 8)
    for k in range(4):
        s.add(k, [k] * 5)                           # 3 blocks each: the pool is full
    s.free(0)
    s.free(2)
    used = sum(1 for r in s.m.refcounts if r > 0)
    high = [b for b in range(used, 12) if s.m.refcounts[b] > 0]
    holes = [b for b in range(used) if s.m.refcounts[b] == 0]
    pairs = s.compact()
    assert pairs == list(zip(high, holes))
    assert all(src >= used > dst for src, dst in pairs)
    assert list(s.m.free) == list(range(used, 12))
    assert all(b < used for blocks, _ in s.m.seqs.values() for b in blocks)
    s.check()
    assert s.compact() == []                        # already compact


def test_compaction_keeps_shared_blocks_shared_and_cached():
    s = Sim(16, 2, 8)
    s.add(9, [0] * 12)                              # occupies the low blocks
    s.add(1, [1, 2, 3, 4, 5])
    s.fork(1, 2)
    _, c = s.add(3, [1, 2, 3, 4, 6])
    assert c == 4
    s.free(9)
    pairs = s.compact()
    assert len(pairs) == 4                          # 3 of seq 1 (shared) + seq 3's last
    shared = s.m.seqs[1][0]
    assert s.m.seqs[2][0] == shared and s.m.seqs[3][0][:2] == shared[:2]
    assert s.m.refcounts[shared[0]] == 3
    _, c = s.add(4, [1, 2, 3, 4])                   # the cache follows the move
    assert c == 4 and s.m.seqs[4][0] == shared[:2]
    s.append(2, 77)                                 # copy-on-write after the move
    s.check()


ops = st.lists(st.tuples(st.sampled_from(["add", "add", "fork", "append", "free", "compact"]),
                         st.integers(0, 5), st.integers(0, 5),
                         st.lists(st.integers(0, 2), max_size=14)),
               max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4]))
def test_random_trace_content_and_hits(ops, bs):
    s = Sim(24, bs, 8)
    for kind, a, b, toks in ops:
        try:
            if kind == "add":
                if a in s.m.seqs:
                    continue
                want = s.expected_hits(toks)
                _, c = s.add(a, toks)
                assert c == want
            elif kind == "fork" and a in s.m.seqs and b not in s.m.seqs:
                s.fork(a, b)
            elif kind == "append" and a in s.m.seqs:
                s.append(a, toks[0] if toks else 3)
            elif kind == "free" and a in s.m.seqs:
                s.free(a)
            elif kind == "compact":
                s.compact()
        except AllocError as e:
            assert e.code in ("OUT_OF_BLOCKS", "SEQ_LIMIT")
        s.check()

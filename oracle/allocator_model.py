"""Oracle model of the host-side block manager (free list, tables, refcounts).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

What the pages fix:

* [PA-mem] section "PagedAttention: the operating system's memory wisdom":
  the block manager keeps a list of free physical blocks and, per sequence, a
  table from logical to physical blocks.  A new request first receives its
  initial blocks; while it generates, a fresh block is taken from the free list
  each time the current block fills, and the table is updated.
* [PA-mem] section "Continuous batching and memory management working
  together": a finished request returns all of its blocks to the free list.
* [vLLM-core] section 2 ("KV Cache management"): pages holding a common prefix
  may be shared by several requests; a shared page is copied only when one of
  its sharers modifies it (copy-on-write, as with ``fork``); shared pages carry
  a reference count so that one sharer finishing cannot release a page another
  still uses.

Readings where the pages are silent:

* the free list is FIFO: blocks are taken from the front, returned to the
  back, and a finished sequence returns its blocks in logical order;
* ``initial_free_order`` (a permutation of the block numbers) sets the first
  order of the free list, which is how a "shuffled" or "fragmented" pool is
  built;
* copy-on-write fires in ``append_slot`` when the sequence's last block is
  partly filled and has a reference count above one: the appending sequence
  moves to a fresh block and the caller must copy the old block into it;
* a full shared block is never written again, so it is never copied;
* every operation either succeeds completely or raises ``AllocError`` with the
  state unchanged.
"""

from collections import deque

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data):
    """64-bit FNV-1a (Fowler, Noll, Vo): start from the offset basis; for each
    byte, xor it in, then multiply by the FNV prime modulo 2**64."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent_hash, tokens):
    """Content hash of one full block: FNV-1a over the parent block's hash
    (8 bytes, little-endian) followed by the block's token ids (4 bytes each,
    little-endian, two's complement).  The first block of a sequence has
    parent hash 0."""
    data = int(parent_hash & MASK64).to_bytes(8, "little")
    data += b"".join(int(t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


class AllocError(Exception):
    """Raised by a failed operation; ``code`` names the failure."""

    def __init__(self, code, msg=""):
        super().__init__(f"{code}: {msg}" if msg else code)
        self.code = code


class AllocatorModel:
    def __init__(self, num_blocks, block_size, max_blocks_per_seq,
                 initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise AllocError("RANGE", "sizes must be positive")
        if initial_free_order is None:
            order = list(range(num_blocks))
        else:
            order = [int(b) for b in initial_free_order]
            if sorted(order) != list(range(num_blocks)):
                raise AllocError("RANGE", "initial order is not a permutation")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = deque(order)
        self.refcounts = [0] * num_blocks
        self.seqs = {}  # seq id -> [list of physical blocks, number of tokens]
        self.cow_copies = 0
        # Prefix cache: content hash -> block, and per registered block its
        # (hash, parent block or -1, token ids).
        self.index = {}
        self.block_key = {}
        self.prefix_queried = 0
        self.prefix_hits = 0

    # -- helpers -----------------------------------------------------------
    def _slot(self, blocks, pos):
        return blocks[pos // self.block_size] * self.block_size + pos % self.block_size

    def _get(self, seq):
        if seq not in self.seqs:
            raise AllocError("UNKNOWN_SEQ", str(seq))
        return self.seqs[seq]

    # -- operations --------------------------------------------------------
    def add_seq(self, seq, n_tokens):
        """Register a sequence holding ``n_tokens`` tokens; return their slots."""
        if seq in self.seqs:
            raise AllocError("SEQ_EXISTS", str(seq))
        if n_tokens < 0:
            raise AllocError("RANGE", "negative token count")
        need = -(-n_tokens // self.block_size)
        if need > self.max_blocks_per_seq:
            raise AllocError("SEQ_LIMIT", f"{need} blocks")
        if need > len(self.free):
            raise AllocError("OUT_OF_BLOCKS", f"need {need}, have {len(self.free)}")
        blocks = [self.free.popleft() for _ in range(need)]
        for b in blocks:
            self.refcounts[b] = 1
        self.seqs[seq] = [blocks, n_tokens]
        return [self._slot(blocks, p) for p in range(n_tokens)]

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent``, sharing all of its blocks."""
        blocks, n = self._get(parent)
        if child in self.seqs:
            raise AllocError("SEQ_EXISTS", str(child))
        for b in blocks:
            self.refcounts[b] += 1
        self.seqs[child] = [list(blocks), n]

    def append_slot(self, seq):
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow_src, cow_dst)``; the pair is ``(-1, -1)`` unless the
        caller must copy block ``cow_src`` into ``cow_dst`` before writing.
        """
        entry = self._get(seq)
        blocks, pos = entry
        cow = (-1, -1)
        if pos % self.block_size == 0:
            if len(blocks) >= self.max_blocks_per_seq:
                raise AllocError("SEQ_LIMIT", str(seq))
            if not self.free:
                raise AllocError("OUT_OF_BLOCKS", "append")
            b = self.free.popleft()
            self.refcounts[b] = 1
            blocks.append(b)
        else:
            last = blocks[-1]
            if self.refcounts[last] > 1:
                if not self.free:
                    raise AllocError("OUT_OF_BLOCKS", "copy-on-write")
                fresh = self.free.popleft()
                self.refcounts[last] -= 1
                self.refcounts[fresh] = 1
                blocks[-1] = fresh
                cow = (last, fresh)
                self.cow_copies += 1
        entry[1] = pos + 1
        return self._slot(blocks, pos), cow[0], cow[1]

    def free_seq(self, seq):
        """Drop a finished sequence; blocks whose count reaches 0 become free
        (and leave the prefix cache)."""
        blocks, _ = self._get(seq)
        for b in blocks:
            self.refcounts[b] -= 1
            if self.refcounts[b] == 0:
                self.free.append(b)
                key = self.block_key.pop(b, None)
                if key is not None and self.index.get(key[0]) == b:
                    del self.index[key[0]]
        del self.seqs[seq]

    def add_seq_tokens(self, seq, tokens):
        """Register a sequence by its token ids, reusing cached full blocks.

        Automatic prefix sharing ([vLLM-core] section 2, pages of a common
        prefix are shared; [PA-mem] "Architectural limits" and [nano-KV]
        "Engineering: configuration and monitoring", prefix caching and its hit
        rate).  Reading: each full block is keyed by the hash chain of
        ``block_hash``; a leading run of full blocks whose hash, tokens and
        parent block match a live registered block is shared (reference count
        + 1) instead of allocated; the first miss ends the run.  Every newly
        allocated full block is registered; a partial last block never is.
        Only live blocks are found: a block leaves the cache when it is freed.

        Returns ``(slots, n_cached)``: the slot of every token and how many
        leading tokens already hold their K/V (whole shared blocks).
        """
        if seq in self.seqs:
            raise AllocError("SEQ_EXISTS", str(seq))
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        bs = self.block_size
        need_total = -(-n // bs)
        if need_total > self.max_blocks_per_seq:
            raise AllocError("SEQ_LIMIT", f"{need_total} blocks")
        hits, hashes, parent, h = [], [], -1, 0
        for j in range(n // bs):
            toks = tuple(tokens[j * bs:(j + 1) * bs])
            h = block_hash(h, toks)
            hashes.append(h)
            if len(hits) == j:
                b = self.index.get(h)
                if b is not None and self.block_key[b][1] == parent and self.block_key[b][2] == toks:
                    hits.append(b)
                    parent = b
        need_new = need_total - len(hits)
        if need_new > len(self.free):
            raise AllocError("OUT_OF_BLOCKS", f"need {need_new}, have {len(self.free)}")
        blocks = list(hits)
        for b in hits:
            self.refcounts[b] += 1
        parent = hits[-1] if hits else -1
        for j in range(len(hits), need_total):
            b = self.free.popleft()
            self.refcounts[b] = 1
            blocks.append(b)
            if j < n // bs:
                h = hashes[j]
                if h not in self.index:
                    self.index[h] = b
                    self.block_key[b] = (h, parent, tuple(tokens[j * bs:(j + 1) * bs]))
                parent = b
        self.seqs[seq] = [blocks, n]
        self.prefix_queried += n
        self.prefix_hits += len(hits) * bs
        return [self._slot(blocks, p) for p in range(n)], len(hits) * bs

    def compact(self):
        """Move every used block below the count of used blocks.

        Defragmentation by block remapping ([PA-mem] "Continuous batching and
        memory management working together": memory compaction, weighed against
        its migration cost).  Reading: with ``u`` blocks in use, each used block
        numbered ``u`` or above moves, in increasing order, to the lowest free
        block below ``u`` not yet taken; every table, reference count and
        prefix-cache entry follows; the free list becomes ``u .. NB-1`` in
        increasing order.  Returns the ``(src, dst)`` copies (increasing src)
        the caller must apply to every cache before using the new tables.
        """
        used = sum(1 for r in self.refcounts if r > 0)
        holes = [b for b in range(used) if self.refcounts[b] == 0]
        movers = [b for b in range(used, self.num_blocks) if self.refcounts[b] > 0]
        remap = dict(zip(movers, holes))
        for entry in self.seqs.values():
            entry[0] = [remap.get(b, b) for b in entry[0]]
        for src, dst in remap.items():
            self.refcounts[dst] = self.refcounts[src]
            self.refcounts[src] = 0
        keys = {}
        for b, (h, parent, toks) in self.block_key.items():
            keys[remap.get(b, b)] = (h, remap.get(parent, parent), toks)
        self.block_key = keys
        self.index = {h: remap.get(b, b) for h, b in self.index.items()}
        self.free = deque(range(used, self.num_blocks))
        return sorted(remap.items())

    def prefix_stats(self):
        """(tokens asked for through add_seq_tokens, tokens found cached,
        blocks currently in the prefix cache)."""
        return self.prefix_queried, self.prefix_hits, len(self.index)

    def export(self, seq_ids, row_stride):
        """Block tables ``[n][row_stride]`` (padding -1) and context lengths."""
        tables, lens = [], []
        for seq in seq_ids:
            blocks, n = self._get(seq)
            if len(blocks) > row_stride:
                raise AllocError("SHAPE", "row stride too small")
            tables.append(list(blocks) + [-1] * (row_stride - len(blocks)))
            lens.append(n)
        return tables, lens

    # -- observation -------------------------------------------------------
    def refcount(self, block):
        return self.refcounts[block]

    def num_free(self):
        return len(self.free)

    def seq_blocks(self, seq):
        return list(self._get(seq)[0])

    def seq_len(self, seq):
        return self._get(seq)[1]

    def stats(self):
        """Block utilisation and internal fragmentation.

        [PA-mem] section "Monitoring and tuning": utilisation is allocated blocks
        over all blocks; internal fragmentation is the share of token slots
        inside allocated blocks that hold no token.  A shared block counts as
        filled up to the furthest token any of its sharers keeps in it.
        """
        bs = self.block_size
        fill = {}
        logical = 0
        for blocks, n in self.seqs.values():
            logical += n
            for j, b in enumerate(blocks):
                fill[b] = max(fill.get(b, 0), min(bs, n - j * bs))
        used = sum(1 for r in self.refcounts if r > 0)
        shared = sum(1 for r in self.refcounts if r > 1)
        filled = sum(fill.values())
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": shared,
            "cow_copies": self.cow_copies,
            "live_seqs": len(self.seqs),
            "logical_tokens": logical,
            "stored_tokens": filled,
            "utilisation": used / self.num_blocks,
            "internal_fragmentation": (used * bs - filled) / (used * bs) if used else 0.0,
        }

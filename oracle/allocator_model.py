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
        """Drop a finished sequence; blocks whose count reaches 0 become free."""
        blocks, _ = self._get(seq)
        for b in blocks:
            self.refcounts[b] -= 1
            if self.refcounts[b] == 0:
                self.free.append(b)
        del self.seqs[seq]

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

"""Oracle for single-query (decode) attention over a block-paged KV cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

What is computed is the plain definition, written out:

1. Paging.  [vLLM-core] section 1 ("PagedAttention: inspiration from virtual
   memory") and [PA-mem] section "PagedAttention: the operating system's memory
   wisdom": a sequence's KV cache is logically contiguous but stored in
   fixed-size physical blocks that may sit anywhere; a per-sequence table maps
   logical block ``j`` to a physical block.  So logical token ``p`` of sequence
   ``s`` lives at row ``p % bs`` of physical block ``table[s][p // bs]``.
   Only the first ``context_len`` logical tokens exist; nothing else is read.
2. Attention.  [nano-KV] section "Engineering: configuration and monitoring"
   names a plain ("standard") attention as the fallback for the fused decode
   kernel.  With the pages printing no formula, the plain reading is scaled
   dot-product attention of the one new query against every cached token:
   ``z_p = scale * q . K_p``, ``a = softmax(z)``, ``out = sum_p a_p V_p``.

Readings where the pages are silent (each is listed with its reason in the
design notes):

* grouped heads: query head ``h`` reads KV head ``h // (Hq // Hkv)``;
* ``scale`` is the float32 value the kernel receives, widened to float64;
* ``context_len == 0`` gives an all-zero output row;
* the output is left unrounded in float64.
"""

import numpy as np

from .store import slot_view


def gather_sequence(cache, table_row, context_len, block_size=None):
    """Logical rows ``[context_len, Hkv, D]`` of one sequence, in logical order.

    ``cache`` is ``[NB, bs, Hkv, D]`` (any dtype); ``table_row`` lists physical
    block numbers in logical order.  Table entries past the last block that
    holds a token are not touched.
    """
    num_blocks, bs, hkv, d = cache.shape
    if block_size is not None and block_size != bs:
        raise ValueError("block_size does not match the cache")
    L = int(context_len)
    if L < 0:
        raise ValueError("negative context length")
    n_used = -(-L // bs)
    phys = np.asarray(table_row[:n_used], dtype=np.int64)
    if phys.size != n_used:
        raise ValueError("block table row shorter than the context needs")
    if np.any(phys < 0) or np.any(phys >= num_blocks):
        raise ValueError("block table entry out of range")
    rows = cache[phys].reshape(n_used * bs, hkv, d)
    return rows[:L]


def decode_ref(q, k_cache, v_cache, block_tables, context_lens, scale,
               return_weights=False, layout="slot"):
    """fp64 decode attention for every (sequence, query head).

    q:             [B, Hq, D] float16
    k/v_cache:     [NB, bs, Hkv, D] float16 ([NB, Hkv, bs, D] with layout "head")
    block_tables:  [B, M] integers (logical -> physical block)
    context_lens:  [B] integers
    scale:         float (rounded to float32 first, as the kernel receives it)
    Returns out [B, Hq, D] float64, and with ``return_weights`` also a list of
    per-sequence [Hq, L] float64 softmax weights.
    """
    k_cache, v_cache = slot_view(k_cache, layout), slot_view(v_cache, layout)
    q = np.asarray(q)
    B, Hq, D = q.shape
    num_blocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("q, k_cache and v_cache disagree on shape")
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    weights = []
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            weights.append(np.zeros((Hq, 0)))
            continue
        K = gather_sequence(k_cache, block_tables[s], L).astype(np.float64)
        V = gather_sequence(v_cache, block_tables[s], L).astype(np.float64)
        w_seq = np.zeros((Hq, L))
        for h in range(Hq):
            g = h // group
            z = scale64 * (K[:, g, :] @ q[s, h].astype(np.float64))
            e = np.exp(z - z.max())
            a = e / e.sum()
            out[s, h] = a @ V[:, g, :]
            w_seq[h] = a
        weights.append(w_seq)
    if return_weights:
        return out, weights
    return out

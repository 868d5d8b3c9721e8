"""Oracle for chunked-prefill attention over a block-paged KV cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

What is computed, from the pages:

* [PA-mem] section "Deployable configuration parameters" sets a prefill chunk
  size (256 tokens): a prompt is prefilled a chunk at a time.
* [vLLM-core] section 3 ("Continuous batching"): the requests of one batch go
  through prefill and decode together, so a step may hold prompt chunks of
  several sequences of different lengths.
* [nano-KV] section "Engineering: configuration and monitoring": the prefill
  phase uses a variable-length attention routine and falls back to standard
  attention, which fixes the result: plain causal scaled dot-product attention.

Readings where the pages are silent (each is listed in the design notes):

* the chunk is the last ``n_s`` tokens of sequence ``s``'s context, whose K/V
  are already in the cache; ``context_lens[s]`` counts them;
* query token ``j`` of the chunk sits at logical position
  ``context_lens[s] - n_s + j`` and attends to positions ``0 ..`` that
  position, through the block table (causal mask);
* query rows of all sequences are packed: sequence ``s`` owns rows
  ``query_start[s] .. query_start[s+1]-1`` of ``q`` and of the output;
* grouped heads, the float32 ``scale`` and the unrounded float64 output
  follow the decode oracle.
"""

import numpy as np

from .store import slot_view

from .attention import gather_sequence


def prefill_ref(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                layout="slot"):
    """fp64 causal attention of every packed query row.

    q:             [T, Hq, D] float16, rows of all chunks, packed
    k/v_cache:     [NB, bs, Hkv, D] float16 ([NB, Hkv, bs, D] with layout "head")
    block_tables:  [B, M] integers
    context_lens:  [B] integers, context length including the chunk
    query_start:   [B + 1] integers, non-decreasing, query_start[0] == 0,
                   query_start[B] == T
    scale:         float (rounded to float32 first)
    Returns out [T, Hq, D] float64.
    """
    k_cache, v_cache = slot_view(k_cache, layout), slot_view(v_cache, layout)
    q = np.asarray(q)
    T, Hq, D = q.shape
    num_blocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("q, k_cache and v_cache disagree on shape")
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    starts = [int(x) for x in query_start]
    B = len(starts) - 1
    if starts[0] != 0 or starts[-1] != T or any(b < a for a, b in zip(starts, starts[1:])):
        raise ValueError("query_start must run from 0 to T without decreasing")
    group = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(B):
        n = starts[s + 1] - starts[s]
        L = int(context_lens[s])
        if n == 0:
            continue
        if n > L:
            raise ValueError("a chunk is longer than its sequence's context")
        K = gather_sequence(k_cache, block_tables[s], L).astype(np.float64)
        V = gather_sequence(v_cache, block_tables[s], L).astype(np.float64)
        for j in range(n):
            pos = L - n + j
            t = starts[s] + j
            for h in range(Hq):
                g = h // group
                z = scale64 * (K[:pos + 1, g, :] @ q[t, h].astype(np.float64))
                e = np.exp(z - z.max())
                out[t, h] = (e / e.sum()) @ V[:pos + 1, g, :]
    return out

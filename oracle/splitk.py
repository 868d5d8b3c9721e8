"""Oracle for decode attention computed over token chunks, then recombined.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The pages do not describe splitting a long context; they only say that decode
is limited by memory bandwidth ([vLLM-core] section 3, "Continuous batching",
the tuning anecdote about batch size and bandwidth).  Splitting the context of
one query into chunks and merging per-chunk softmax statistics is the published
"online softmax" identity (Milakov & Gimelshein, 2018), used for decode as
"flash-decoding" (Dao et al., 2023).  It reaches the plain result of
``attention.decode_ref`` up to rounding order, so this module exists to state,
in the simplest form, what a chunked kernel and its merge step must compute:

for chunk c of positions P_c:
    m_c = max_{p in P_c} z_p
    l_c = sum_{p in P_c} exp(z_p - m_c)
    o_c = sum_{p in P_c} exp(z_p - m_c) V_p
merge:
    m* = max_c m_c
    out = sum_c exp(m_c - m*) o_c / sum_c exp(m_c - m*) l_c
"""

import numpy as np

from .attention import gather_sequence


def chunk_partials(z, V, chunk_tokens):
    """Per-chunk (m, l, o) for scores ``z`` [L] and values ``V`` [L, D]."""
    parts = []
    for start in range(0, z.shape[0], chunk_tokens):
        zc = z[start:start + chunk_tokens]
        Vc = V[start:start + chunk_tokens]
        m = zc.max()
        e = np.exp(zc - m)
        parts.append((m, e.sum(), e @ Vc))
    return parts


def merge_partials(parts):
    """Combine per-chunk (m, l, o) into the normalised output vector."""
    m_star = max(m for m, _, _ in parts)
    num = sum(np.exp(m - m_star) * o for m, _, o in parts)
    den = sum(np.exp(m - m_star) * l for m, l, _ in parts)
    return num / den


def decode_splitk_ref(q, k_cache, v_cache, block_tables, context_lens, scale,
                      chunk_tokens):
    """Same contract as ``decode_ref``, computed chunk by chunk."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        K = gather_sequence(k_cache, block_tables[s], L).astype(np.float64)
        V = gather_sequence(v_cache, block_tables[s], L).astype(np.float64)
        for h in range(Hq):
            g = h // group
            z = scale64 * (K[:, g, :] @ q[s, h].astype(np.float64))
            out[s, h] = merge_partials(chunk_partials(z, V[:, g, :], chunk_tokens))
    return out

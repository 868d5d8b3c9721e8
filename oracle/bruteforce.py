"""A second, scalar-loop coding of the store and of decode attention.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Written independently of ``store.py`` and ``attention.py``: it addresses the
cache through flat slot numbers (``slot = table[p // bs] * bs + p % bs``, the
slot view of [nano-KV] section "Core mechanism of the paged KV cache") one
scalar at a time, with Python floats and ``math.exp``.  It is only usable for
tiny inputs; its purpose is to catch indexing slips (a swapped head, a wrong
block offset, an off-by-one context) in the vectorised oracle.
"""

import math

import numpy as np


def store_bruteforce(k, v, slot_mapping, k_cache, v_cache):
    """Scalar-loop store on flattened ``[NB*bs*Hkv*D]`` uint16 buffers."""
    kc = np.asarray(k_cache).view(np.uint16).reshape(-1).copy()
    vc = np.asarray(v_cache).view(np.uint16).reshape(-1).copy()
    num_blocks, bs, hkv, d = np.asarray(k_cache).shape
    row = hkv * d
    kin = np.asarray(k).view(np.uint16).reshape(-1)
    vin = np.asarray(v).view(np.uint16).reshape(-1)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        for i in range(row):
            kc[s * row + i] = kin[t * row + i]
            vc[s * row + i] = vin[t * row + i]
    return kc.reshape(num_blocks, bs, hkv, d), vc.reshape(num_blocks, bs, hkv, d)


def decode_bruteforce(q, k_cache, v_cache, block_tables, context_lens, scale):
    """Scalar-loop decode attention; returns a nested Python list [B][Hq][D]."""
    num_blocks, bs, hkv, d = k_cache.shape
    kflat = np.asarray(k_cache).reshape(num_blocks * bs, hkv, d)
    vflat = np.asarray(v_cache).reshape(num_blocks * bs, hkv, d)
    nseq, hq, _ = q.shape
    per_kv = hq // hkv
    sc = float(np.float32(scale))
    result = []
    for s in range(nseq):
        L = int(context_lens[s])
        seq_out = []
        for h in range(hq):
            kv = h // per_kv
            slots = [int(block_tables[s][p // bs]) * bs + p % bs for p in range(L)]
            scores = []
            for slot in slots:
                acc = 0.0
                for i in range(d):
                    acc += float(q[s, h, i]) * float(kflat[slot, kv, i])
                scores.append(sc * acc)
            if not scores:
                seq_out.append([0.0] * d)
                continue
            top = max(scores)
            ex = [math.exp(x - top) for x in scores]
            total = sum(ex)
            vec = []
            for i in range(d):
                num = 0.0
                for e, slot in zip(ex, slots):
                    num += e * float(vflat[slot, kv, i])
                vec.append(num / total)
            seq_out.append(vec)
        result.append(seq_out)
    return result

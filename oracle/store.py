"""Oracle for writing new K/V rows into the block-paged cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: [nano-KV] section "Core mechanism of the paged KV cache": each new
token's key and value row is written into the cache at the slot that a
per-token ``slot_mapping`` tensor names; the cache is viewed as a flat array of
token slots.  [PA-mem] section "PagedAttention: the operating system's memory
wisdom" fixes the blocking: the cache is cut into fixed-size blocks of
``block_size`` token slots.

Readings where the pages are silent:

* layout: ``cache[num_blocks][block_size][num_kv_heads][head_dim]`` fp16, so
  slot ``s`` is row ``s % block_size`` of physical block ``s // block_size``;
* a negative slot means "no write" (padding);
* a slot at or beyond ``num_blocks * block_size`` and a repeated non-negative
  slot are caller errors (raised here).

The copy is on raw 16-bit patterns, so NaN payloads survive bit for bit.

Source for ``copy_blocks_ref``: [vLLM-core] section 2 ("KV Cache management"),
copy-on-write item: a shared page is duplicated only when one of its sharers
is about to modify it.  Reading: the whole physical block (every slot, every
head, K and V) is copied from ``src`` to ``dst``.
"""

import numpy as np

# Cache layouts.  "slot" (the reading above): cache[num_blocks][block_size]
# [num_kv_heads][head_dim].  "head": cache[num_blocks][num_kv_heads]
# [block_size][head_dim] -- the same rows, each (block, KV head) run kept
# together; the pages fix no order inside a block (the slot numbering and the
# block table are the same in both).
LAYOUTS = ("slot", "head")


def slot_view(cache, layout="slot"):
    """``cache`` seen as [num_blocks][block_size][num_kv_heads][head_dim]
    (a numpy view: writes through it land in ``cache``)."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {LAYOUTS}")
    return cache if layout == "slot" else np.swapaxes(cache, 1, 2)


def _as_u16(a):
    a = np.asarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype == np.uint16:
        return a
    raise TypeError(f"expected float16 or uint16 array, got {a.dtype}")


def store_ref(k, v, slot_mapping, k_cache, v_cache, layout="slot"):
    """Return new (k_cache, v_cache) with each token's rows written to its slot.

    k, v:          [N, Hkv, D] float16 (or uint16 bit patterns)
    slot_mapping:  [N] integers; slot < 0 skips the token
    k_cache, v_cache: [NB, bs, Hkv, D] float16 (or uint16), or [NB, Hkv, bs, D]
                   with layout "head"; not modified
    Returns uint16 arrays (the exact bit patterns), in the caches' layout.
    """
    k16, v16 = _as_u16(k), _as_u16(v)
    kc_out = _as_u16(k_cache).copy()
    vc_out = _as_u16(v_cache).copy()
    kc, vc = slot_view(kc_out, layout), slot_view(vc_out, layout)
    num_blocks, block_size, hkv, d = kc.shape
    slots = np.asarray(slot_mapping).astype(np.int64).reshape(-1)
    if k16.shape != (slots.size, hkv, d) or v16.shape != k16.shape:
        raise ValueError("k/v must be [N, Hkv, D] matching the cache and slot_mapping")
    seen = set()
    for t in range(slots.size):
        s = int(slots[t])
        if s < 0:
            continue
        if s >= num_blocks * block_size:
            raise ValueError(f"slot {s} out of range")
        if s in seen:
            raise ValueError(f"slot {s} written twice")
        seen.add(s)
        block, offset = divmod(s, block_size)
        kc[block, offset] = k16[t]
        vc[block, offset] = v16[t]
    return kc_out, vc_out


def copy_blocks_ref(k_cache, v_cache, pairs):
    """Return new (k_cache, v_cache) with block ``dst`` replaced by block ``src``.

    pairs: [n, 2] integers (src, dst), applied in order.
    """
    kc = _as_u16(k_cache).copy()
    vc = _as_u16(v_cache).copy()
    num_blocks = kc.shape[0]
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks):
            raise ValueError(f"block pair ({src}, {dst}) out of range")
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc

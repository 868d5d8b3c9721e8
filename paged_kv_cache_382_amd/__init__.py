"""Paged KV-cache decode for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``lib/libpa.so``: the names match the C ABI in
``include/pa.h`` and every function only marshals arguments (tensor pointers,
shapes, the current HIP stream).  All work runs in the library's HIP kernels
or its C++ allocator; there is no Python or CPU fallback.  Importing the
package fails loudly when the library has not been built
(``python -m paged_kv_cache_382_amd.build``).

PyTorch is used only for device memory and streams.
"""

import ctypes
import os

import numpy as np

__all__ = [
    "PaError", "CacheDesc", "lib",
    "pa_store_kvcache", "pa_copy_blocks", "pa_decode", "pa_decode_noalloc", "pa_prefill",
    "pa_decode_workspace_bytes", "pa_decode_num_splits",
    "pa_set_validate", "pa_version", "Allocator", "decode_workspace", "DecodeStepGraph",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpa.so")

STATUS = {
    0: "OK", 1: "NULL", 2: "SHAPE", 3: "ALIGN", 4: "UNSUPPORTED", 5: "RANGE",
    6: "WORKSPACE", 7: "OUT_OF_BLOCKS", 8: "SEQ_LIMIT", 9: "UNKNOWN_SEQ",
    10: "SEQ_EXISTS", 11: "HIP", 12: "HOST",
}


class PaError(RuntimeError):
    """A failed library call; ``code`` is the status name (e.g. "OUT_OF_BLOCKS")."""

    def __init__(self, status, message):
        self.status = int(status)
        self.code = STATUS.get(self.status, str(status))
        super().__init__(f"{self.code}: {message}")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


# Cache layouts (pa_layout): "slot" = [num_blocks][block_size][num_kv_heads][head_dim]
# (the default), "head" = [num_blocks][num_kv_heads][block_size][head_dim].
LAYOUTS = {"slot": 0, "head": 1}


class AllocStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("used_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("cow_copies", ctypes.c_int64), ("live_seqs", ctypes.c_int64),
                ("logical_tokens", ctypes.c_int64), ("stored_tokens", ctypes.c_int64),
                ("utilisation", ctypes.c_double), ("internal_fragmentation", ctypes.c_double)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes): every symbol declared in include/pa.h
SIGNATURES = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
    "pa_set_validate": (ctypes.c_int, [ctypes.c_int]),
    "pa_store_kvcache": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, ctypes.POINTER(CacheDesc), _P]),
    "pa_copy_blocks": (ctypes.c_int, [_P, _P, ctypes.POINTER(CacheDesc), _P, _I32, _P]),
    "pa_decode": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(CacheDesc), _P, _I32, _P, _I32, _I32,
                                 _I32, ctypes.c_float, _P, _I32, _P, ctypes.c_size_t, _P]),
    "pa_decode_noalloc": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(CacheDesc), _P, _I32, _P, _I32,
                                         _I32, _I32, ctypes.c_float, _P, _I32, _P]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), _I32, _I32, _I32]),
    "pa_decode_num_splits": (_I32, [ctypes.POINTER(CacheDesc), _I32, _I32]),
    "pa_prefill": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(CacheDesc), _P, _I32, _P, _P, _I32,
                                  _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P]),
    "pa_alloc_create": (ctypes.c_int, [_I32, _I32, _I32, _PI32, ctypes.POINTER(_P)]),
    "pa_alloc_destroy": (None, [_P]),
    "pa_alloc_add_seq": (ctypes.c_int, [_P, _I64, _I32, _PI32]),
    "pa_alloc_fork": (ctypes.c_int, [_P, _I64, _I64]),
    "pa_alloc_append_slot": (ctypes.c_int, [_P, _I64, _PI32, _PI32, _PI32]),
    "pa_alloc_append_batch": (ctypes.c_int, [_P, _PI64, _I32, _PI32, _PI32, _PI32, _PI32]),
    "pa_alloc_free_seq": (ctypes.c_int, [_P, _I64]),
    "pa_alloc_export": (ctypes.c_int, [_P, _PI64, _I32, _I32, _PI32, _PI32]),
    "pa_alloc_stats": (ctypes.c_int, [_P, ctypes.POINTER(AllocStats)]),
    "pa_alloc_refcount": (_I32, [_P, _I32]),
    "pa_alloc_num_free": (_I32, [_P]),
    "pa_alloc_free_list": (_I32, [_P, _PI32, _I32]),
    "pa_alloc_seq_info": (ctypes.c_int, [_P, _I64, _PI32, _PI32]),
    "pa_alloc_add_seq_tokens": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32, _PI32]),
    "pa_alloc_compact": (ctypes.c_int, [_P, _PI32, _I32, _PI32]),
    "pa_alloc_prefix_stats": (ctypes.c_int, [_P, _PI64, _PI64, _PI32]),
}

_lib = None


def lib():
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        # PyTorch ships its own HIP runtime under another file name.  Loading
        # it first makes libpa.so bind to that same runtime (matched by
        # soname) instead of pulling a second copy into the process.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_382_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


lib()   # fail at import time, not at first call, when the library is missing


def _check(status):
    if status != 0:
        raise PaError(status, lib().pa_last_error().decode())


def pa_version():
    return lib().pa_version().decode()


def pa_set_validate(on):
    """Turn the library's validation mode on/off; returns the previous setting."""
    return bool(lib().pa_set_validate(1 if on else 0))


# --------------------------------------------------------------------------
# device calls
# --------------------------------------------------------------------------

def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def cache_desc(k_cache, layout="slot"):
    """Descriptor of a cache tensor whose dimensions are in ``layout`` order."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if layout == "slot":
        nb, bs, hkv, d = k_cache.shape
    else:
        nb, hkv, bs, d = k_cache.shape
    return CacheDesc(nb, bs, hkv, d, LAYOUTS[layout])


def pa_store_kvcache(k, v, slot_mapping, k_cache, v_cache, stream=None, layout="slot"):
    """Write k/v [N, Hkv, D] fp16 rows to the cache slots in slot_mapping [N] int32."""
    import torch
    if k_cache.shape != v_cache.shape or k.shape != v.shape:
        raise ValueError("k/v and k_cache/v_cache must have matching shapes")
    desc = cache_desc(k_cache, layout)
    n = k.shape[0]
    if k.dim() != 3 or tuple(k.shape[1:]) != (desc.num_kv_heads, desc.head_dim):
        raise ValueError("k must be [N, num_kv_heads, head_dim]")
    if slot_mapping.numel() != n:
        raise ValueError("slot_mapping must have one entry per token")
    _check(lib().pa_store_kvcache(
        _dev(k, torch.float16, "k"), _dev(v, torch.float16, "v"),
        _dev(slot_mapping, torch.int32, "slot_mapping"), n,
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"),
        ctypes.byref(desc), _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, src_dst, stream=None, layout="slot"):
    """Copy whole blocks src_dst[i][0] -> src_dst[i][1] in both caches."""
    import torch
    desc = cache_desc(k_cache, layout)
    n = src_dst.shape[0] if src_dst.numel() else 0
    if src_dst.numel() and (src_dst.dim() != 2 or src_dst.shape[1] != 2):
        raise ValueError("src_dst must be [n, 2]")
    _check(lib().pa_copy_blocks(
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"),
        ctypes.byref(desc), _dev(src_dst, torch.int32, "src_dst") if n else None, n,
        _stream(stream)))


def pa_decode_workspace_bytes(desc, num_seqs, num_q_heads, num_splits=0):
    return int(lib().pa_decode_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                               num_splits))


def pa_decode_num_splits(desc, num_q_heads, num_splits=0):
    return int(lib().pa_decode_num_splits(ctypes.byref(desc), num_q_heads, num_splits))


def decode_workspace(desc, num_seqs, num_q_heads, num_splits=0, device="cuda"):
    """A workspace for pa_decode with these shapes (contents irrelevant)."""
    import torch
    n = pa_decode_workspace_bytes(desc, num_seqs, num_q_heads, num_splits)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check_rows(q, out, desc, name):
    """q (and out, when given) must be [rows, Hq, head_dim] of one shape and dtype."""
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError(f"{name} must be [rows, num_q_heads, {desc.head_dim}] (got {tuple(q.shape)})")
    if q.shape[1] % desc.num_kv_heads != 0:
        raise ValueError(f"num_q_heads ({q.shape[1]}) must be a multiple of num_kv_heads "
                         f"({desc.num_kv_heads})")
    if out is not None and (tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype):
        raise ValueError(f"out must match {name} in shape and dtype (got {tuple(out.shape)}, {out.dtype})")


def _check_decode_shapes(q, k_cache, v_cache, desc, block_tables, context_lens, out):
    """Every size the kernels take from the tensors, checked before any launch:
    the C ABI sees raw pointers, so a mismatched tensor would be read or
    written past its end."""
    _check_rows(q, out, desc, "q")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must have k_cache's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != q.shape[0]:
        raise ValueError("block_tables must be [B, M] with B = q.shape[0]")
    if context_lens.numel() != q.shape[0]:
        raise ValueError("context_lens must be [B]")


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
              max_context_len=None, num_splits=0, workspace=None, stream=None, layout="slot"):
    """Single-query paged attention; returns ``out`` [B, Hq, D] fp16.

    ``max_context_len`` (host int) bounds ``context_lens``; by default the
    table width times the block size.  ``num_splits`` is the number of equal
    pieces (one workgroup each) the work is cut into (0: as many workgroups as
    the GPU holds at once).  ``workspace`` (a uint8 device tensor from
    ``decode_workspace``) is allocated when not given.
    """
    import torch
    desc = cache_desc(k_cache, layout)
    _check_decode_shapes(q, k_cache, v_cache, desc, block_tables, context_lens, out)
    B, hq, d = q.shape
    M = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = M * desc.block_size
    if out is None:
        out = torch.empty_like(q)
    need = pa_decode_workspace_bytes(desc, B, hq, num_splits) if B else 0
    if need and workspace is None:
        workspace = decode_workspace(desc, B, hq, num_splits, q.device)
    ws_ptr = _dev(workspace, torch.uint8, "workspace") if need else None
    ws_bytes = workspace.numel() if need else 0
    _check(lib().pa_decode(
        _dev(q, torch.float16, "q"), _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), ctypes.byref(desc),
        _dev(block_tables, torch.int32, "block_tables"), M,
        _dev(context_lens, torch.int32, "context_lens"), B, hq, int(max_context_len),
        float(scale), _dev(out, torch.float16, "out"), int(num_splits), ws_ptr, ws_bytes,
        _stream(stream)))
    return out


# Bytes of the device array that pa_decode_noalloc keeps its partial results in.
NOALLOC_SCRATCH_BYTES = 8 << 20


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                      max_context_len=None, num_splits=0, stream=None, layout="slot"):
    """pa_decode with the partial results in the library's own device array
    (no workspace, no allocation); ``out`` must be given.  Calls that overlap
    on one GPU share that array and must be serialised by the caller."""
    import torch
    desc = cache_desc(k_cache, layout)
    if out is None:
        raise ValueError("pa_decode_noalloc writes into a caller-provided out")
    _check_decode_shapes(q, k_cache, v_cache, desc, block_tables, context_lens, out)
    B, hq, d = q.shape
    M = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = M * desc.block_size
    _check(lib().pa_decode_noalloc(
        _dev(q, torch.float16, "q"), _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), ctypes.byref(desc),
        _dev(block_tables, torch.int32, "block_tables"), M,
        _dev(context_lens, torch.int32, "context_lens"), B, hq, int(max_context_len),
        float(scale), _dev(out, torch.float16, "out"), int(num_splits), _stream(stream)))
    return out


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, out=None,
               max_query_len=None, max_context_len=None, stream=None, layout="slot"):
    """Causal attention of packed prompt chunks; returns ``out`` [T, Hq, D] fp16.

    ``query_start`` (device int32 [B + 1]) splits the T rows of ``q`` into the
    sequences' chunks; each chunk is the last rows of its sequence's context
    (``context_lens``), already stored in the caches.  ``max_query_len`` (host
    int, at least every chunk's length) is read from ``query_start`` when not
    given, which synchronises; ``max_context_len`` defaults to the table
    width times the block size.
    """
    import torch
    desc = cache_desc(k_cache, layout)
    _check_rows(q, out, desc, "q")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("v_cache must have k_cache's shape")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, M]")
    T, hq, d = q.shape
    B, M = block_tables.shape
    if context_lens.numel() != B or query_start.numel() != B + 1:
        raise ValueError("context_lens must be [B] and query_start [B + 1]")
    if max_query_len is None:
        qs = query_start.to("cpu", torch.int64)
        max_query_len = int((qs[1:] - qs[:-1]).max().item()) if B else 0
    if max_context_len is None:
        max_context_len = M * desc.block_size
    if out is None:
        out = torch.empty_like(q)
    _check(lib().pa_prefill(
        _dev(q, torch.float16, "q"), _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), ctypes.byref(desc),
        _dev(block_tables, torch.int32, "block_tables"), M,
        _dev(context_lens, torch.int32, "context_lens"),
        _dev(query_start, torch.int32, "query_start"), B, T, hq, int(max_query_len),
        int(max_context_len), float(scale), _dev(out, torch.float16, "out"), _stream(stream)))
    return out


class DecodeStepGraph:
    """One decode step of every layer, captured once into a HIP graph.

    Source: [PA-mem] "Architectural limits and evolution" (graph capture turns
    many kernel launches into one executable graph) and [nano-KV] "Scheduling
    strategy and continuous batching" (the token-by-token decode loop is
    captured as a graph to remove launch and interpreter overhead).

    A step is, per layer: the copy-on-write block copies (if any), the store of
    the step's new K/V rows through ``slot_mapping``, and ``pa_decode``.  The
    launches are recorded once; ``replay()`` then issues the whole step with a
    single graph launch, without per-kernel launch cost.  As with any graph,
    the tensors are fixed: update their contents in place between replays
    (new rows, slots, tables, lengths, queries); shapes and the number of
    copy pairs cannot change.  The decode is captured with the table bound
    (max_blocks_per_seq * block_size) as its length bound, so lengths can grow
    in place up to what the tables hold; an explicit smaller
    ``max_context_len`` is refused.

    layers: list of (k_cache, v_cache); q, k_new, v_new, out: per-layer lists
    of tensors (q/out [B, Hq, D], k_new/v_new [N, Hkv, D]); the metadata is
    shared by all layers.
    """

    def __init__(self, layers, q, k_new, v_new, slot_mapping, block_tables, context_lens, scale,
                 out, cow_pairs=None, max_context_len=None, num_splits=0, layout="slot"):
        import torch
        self.layers = list(layers)
        self.args = (q, k_new, v_new, slot_mapping, block_tables, context_lens, out, cow_pairs)
        self.scale = float(scale)
        self.layout = layout
        kc0 = self.layers[0][0]
        desc = cache_desc(kc0, layout)
        # The bound is fixed at capture and lengths may grow between replays:
        # capture with the largest length the tables can hold, so that no
        # context is ever clamped.
        bound = block_tables.shape[1] * desc.block_size
        if max_context_len is not None and int(max_context_len) < bound:
            raise ValueError(f"max_context_len {max_context_len} is below the table bound {bound} "
                             "(max_blocks_per_seq * block_size); contexts that grow past it would be "
                             "clamped in replays")
        self.max_context_len = bound
        B, hq = q[0].shape[0], q[0].shape[1]
        self.num_splits = int(num_splits)
        self.workspace = decode_workspace(desc, B, hq, self.num_splits, kc0.device)
        # Kernels are loaded (and the pool primed) by one eager step on a side
        # stream before capture.
        side = torch.cuda.Stream(device=kc0.device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize(kc0.device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step()

    def _step(self):
        q, k_new, v_new, slots, tables, lens, out, cows = self.args
        for layer, (kc, vc) in enumerate(self.layers):
            if cows is not None and cows.numel():
                pa_copy_blocks(kc, vc, cows, layout=self.layout)
            pa_store_kvcache(k_new[layer], v_new[layer], slots, kc, vc, layout=self.layout)
            pa_decode(q[layer], kc, vc, tables, lens, self.scale, out=out[layer],
                      max_context_len=self.max_context_len, num_splits=self.num_splits,
                      workspace=self.workspace, layout=self.layout)

    def replay(self):
        self.graph.replay()


# --------------------------------------------------------------------------
# host allocator
# --------------------------------------------------------------------------

def _i32p(a):
    return a.ctypes.data_as(_PI32)


class Allocator:
    """The C++ block manager: FIFO free list, block tables, refcounts, CoW."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq, initial_free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.size != self.num_blocks:
                raise PaError(5, "initial order must list every block")
        h = ctypes.c_void_p()
        _check(lib().pa_alloc_create(self.num_blocks, self.block_size, self.max_blocks_per_seq,
                                     _i32p(order) if order is not None else None, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_alloc_destroy(h)
            self._h = None

    def add_seq(self, seq, n_tokens):
        slots = np.empty(max(int(n_tokens), 1), dtype=np.int32)
        _check(lib().pa_alloc_add_seq(self._h, int(seq), int(n_tokens), _i32p(slots)))
        return slots[:int(n_tokens)]

    def fork(self, parent, child):
        _check(lib().pa_alloc_fork(self._h, int(parent), int(child)))

    def append_slot(self, seq):
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_alloc_append_slot(self._h, int(seq), ctypes.byref(slot),
                                          ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def append_batch(self, seqs):
        """One token for each sequence; returns (slots [n], cow pairs [k, 2])."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = ids.size
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        n_cow, n_done = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_alloc_append_batch(self._h, ids.ctypes.data_as(_PI64), n, _i32p(slots),
                                           _i32p(pairs), ctypes.byref(n_cow), ctypes.byref(n_done)))
        return slots[:n], pairs[:n_cow.value]

    def free_seq(self, seq):
        _check(lib().pa_alloc_free_seq(self._h, int(seq)))

    def export(self, seqs, row_stride):
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = ids.size
        tables = np.empty((max(n, 1), int(row_stride)), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().pa_alloc_export(self._h, ids.ctypes.data_as(_PI64), n, int(row_stride),
                                     _i32p(tables), _i32p(lens)))
        return tables[:n], lens[:n]

    def stats(self):
        st = AllocStats()
        _check(lib().pa_alloc_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in AllocStats._fields_}

    def refcount(self, block):
        return int(lib().pa_alloc_refcount(self._h, int(block)))

    def num_free(self):
        return int(lib().pa_alloc_num_free(self._h))

    def free_list(self):
        out = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        n = lib().pa_alloc_free_list(self._h, _i32p(out), self.num_blocks)
        return out[:n]

    def seq_info(self, seq):
        n_tok, n_blk = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_alloc_seq_info(self._h, int(seq), ctypes.byref(n_tok), ctypes.byref(n_blk)))
        return n_tok.value, n_blk.value

    def seq_len(self, seq):
        return self.seq_info(seq)[0]

    def add_seq_tokens(self, seq, tokens):
        """Register a sequence by token ids, sharing cached full blocks;
        returns (slots, n_cached)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        n = toks.size
        slots = np.empty(max(n, 1), dtype=np.int32)
        n_cached = ctypes.c_int32()
        _check(lib().pa_alloc_add_seq_tokens(self._h, int(seq), _i32p(toks) if n else None, n,
                                             _i32p(slots), ctypes.byref(n_cached)))
        return slots[:n], n_cached.value

    def compact(self):
        """Renumber used blocks below the used count; returns the [k, 2]
        (src, dst) copies to apply to every cache."""
        cap = max(self.num_blocks // 2, 1)
        pairs = np.empty((cap, 2), dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_alloc_compact(self._h, _i32p(pairs), cap, ctypes.byref(n)))
        return pairs[:n.value]

    def prefix_stats(self):
        """(tokens queried, tokens found cached, blocks cached)."""
        q, h, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().pa_alloc_prefix_stats(self._h, ctypes.byref(q), ctypes.byref(h), ctypes.byref(c)))
        return q.value, h.value, c.value

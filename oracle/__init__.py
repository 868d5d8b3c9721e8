"""Plain CPU oracle for paged KV-cache decode.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything in this package. The
product path (the HIP library and its Python binding) never imports it and
shares no code with it.

Everything here is slow and written to be checked by eye against the pages it
follows.  Three pages describe the method; they are cited by title:

* [PA-mem]  "Deep dive into the nano-vLLM inference engine architecture:
  PagedAttention memory management" (blog.hotdry.top, 2026-02-02).
* [nano-KV] "Deep analysis of nano-vLLM's paged KV cache and memory
  optimisation architecture" (blog.hotdry.top, 2026-02-02).
* [vLLM-core] "vLLM core architecture: PagedAttention principle, KV Cache
  management, continuous batching" (an online book chapter).

Modules
-------
store          raw-bit scatter through ``slot_mapping`` and whole-block copies.
attention      gather through block tables + dense softmax attention (fp64).
prefill        causal attention of packed prompt chunks over the same cache.
splitk         the same attention computed over token chunks and recombined.
bruteforce     a second, scalar-loop coding of ``attention`` for tiny inputs.
allocator_model  free list, reference counts, fork and copy-on-write,
               content-hash prefix caching and compaction.

Pin status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle.py``, ``tests/test_oracle_prefill.py``,
``tests/test_allocator_model.py`` or ``tests/test_prefix_compact_model.py``.
"""

from .store import LAYOUTS, copy_blocks_ref, slot_view, store_ref
from .attention import gather_sequence, decode_ref
from .prefill import prefill_ref
from .splitk import decode_splitk_ref
from .bruteforce import decode_bruteforce, store_bruteforce
from .allocator_model import AllocatorModel, AllocError, block_hash, fnv1a64

__all__ = [
    "store_ref",
    "copy_blocks_ref",
    "gather_sequence",
    "decode_ref",
    "prefill_ref",
    "decode_splitk_ref",
    "decode_bruteforce",
    "store_bruteforce",
    "AllocatorModel",
    "AllocError",
    "block_hash",
    "fnv1a64",
]

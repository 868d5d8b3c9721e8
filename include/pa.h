/*
 * pa.h -- C ABI of a paged KV-cache decode library for AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * Three pages describe the method; they are cited by title:
 *   [PA-mem]    "Deep dive into the nano-vLLM inference engine architecture:
 *               PagedAttention memory management" (blog.hotdry.top, 2026-02-02)
 *   [nano-KV]   "Deep analysis of nano-vLLM's paged KV cache and memory
 *               optimisation architecture" (blog.hotdry.top, 2026-02-02)
 *   [vLLM-core] "vLLM core architecture: PagedAttention principle, KV Cache
 *               management, continuous batching"
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every call returns pa_status; PA_OK is 0.  On failure, pa_last_error()
 *    returns a message for the calling thread.  No C++ exception crosses the
 *    ABI.
 *  - Device calls take plain device pointers and a HIP stream (hipStream_t
 *    passed as void*; NULL means the default stream).  They only enqueue work
 *    and return; they never allocate device memory and never synchronise,
 *    except in validation mode (pa_set_validate), which copies the metadata
 *    to the host and checks it before launching.  All argument checks happen
 *    before any launch: a call that fails launches nothing.  Faults inside a
 *    kernel surface as a HIP error at the caller's next synchronisation.
 *  - The caller owns every device buffer, including the decode workspace.
 *  - Element type of q, k, v, caches and out is IEEE binary16 (fp16).  Device
 *    pointers to fp16 data must be 16-byte aligned.
 *
 * Cache layout (reading of [nano-KV] "Core mechanism of the paged KV cache",
 * which flattens the cache into token slots, and of [PA-mem] "PagedAttention:
 * the operating system's memory wisdom", which cuts it into fixed-size
 * blocks): one tensor for keys and one for values, each
 *     fp16 [num_blocks][block_size][num_kv_heads][head_dim], contiguous
 * (slot-major, the default; pa_cache_desc.layout may instead name the
 * head-major order [num_blocks][num_kv_heads][block_size][head_dim]).
 * Slot s is row (s % block_size) of physical block (s / block_size).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL = 1,           /* a required pointer is NULL                 */
    PA_ERR_SHAPE = 2,          /* inconsistent or non-positive sizes          */
    PA_ERR_ALIGN = 3,          /* a device pointer is not 16-byte aligned     */
    PA_ERR_UNSUPPORTED = 4,    /* head_dim / block_size / group not built     */
    PA_ERR_RANGE = 5,          /* a value outside its allowed range           */
    PA_ERR_WORKSPACE = 6,      /* decode workspace missing or too small       */
    PA_ERR_OUT_OF_BLOCKS = 7,  /* allocator: no free block left               */
    PA_ERR_SEQ_LIMIT = 8,      /* allocator: max_blocks_per_seq reached       */
    PA_ERR_UNKNOWN_SEQ = 9,    /* allocator: no such sequence                 */
    PA_ERR_SEQ_EXISTS = 10,    /* allocator: sequence id already in use       */
    PA_ERR_HIP = 11,           /* a HIP runtime call failed                   */
    PA_ERR_HOST = 12           /* host memory ran out (or another host-side
                                  failure); an allocator that returns it may
                                  be partly updated and must be destroyed    */
} pa_status;

/* Order of the rows inside a block.  Slot-major (the default) keeps each
 * token slot's KV heads together: [num_blocks][block_size][num_kv_heads]
 * [head_dim], so that the cache is a flat array of slots (each slot one row of
 * num_kv_heads * head_dim).  Head-major keeps each KV head's rows of a block
 * together: [num_blocks][num_kv_heads][block_size][head_dim], one contiguous
 * block_size * head_dim run per (block, KV head).  Slots, block numbers and
 * every result are the same in both; only addresses differ. */
typedef enum { PA_LAYOUT_SLOT_MAJOR = 0, PA_LAYOUT_HEAD_MAJOR = 1 } pa_layout;

typedef struct pa_cache_desc {
    int32_t num_blocks;        /* physical blocks in the pool                 */
    int32_t block_size;        /* token slots per block: 8, 16, 32 or 64      */
    int32_t num_kv_heads;      /* KV heads per token                          */
    int32_t head_dim;          /* 64 or 128                                   */
    int32_t layout;            /* pa_layout; other values: PA_ERR_UNSUPPORTED */
} pa_cache_desc;

/* Message describing the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

/* Turn validation mode on (nonzero) or off.  Its initial value comes from the
 * environment variable PA_VALIDATE ("1" = on).  In validation mode the device
 * calls copy their integer metadata to the host, synchronise the stream, and
 * reject out-of-range or duplicate entries with PA_ERR_RANGE before any
 * launch.  Returns the previous setting. */
int pa_set_validate(int on);

/* ----------------------------------------------------------------------- */
/* Store: write each new token's K and V rows into its cache slot.
 *
 * Source: [nano-KV] "Core mechanism of the paged KV cache" -- every new key
 * and value row goes to the cache slot that a per-token slot mapping names.
 *
 *   k, v          device fp16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  device int32 [num_tokens]; slot < 0 means "skip this token"
 *                 (padding).  Non-negative slots must be distinct and below
 *                 num_blocks * block_size; a slot at or beyond that bound is
 *                 skipped by the kernel (and rejected in validation mode).
 *   k_cache, v_cache  device fp16 caches described by *cache (written)
 *
 * The copy moves raw 16-bit patterns: every bit, NaN payloads included, lands
 * unchanged.  num_tokens == 0 is valid and launches nothing.  Works for any
 * head_dim that is a multiple of 8.
 */
pa_status pa_store_kvcache(const void* k, const void* v,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           void* k_cache, void* v_cache,
                           const pa_cache_desc* cache, void* hip_stream);

/* ----------------------------------------------------------------------- */
/* Copy whole physical blocks (copy-on-write of a shared block).
 *
 * Source: [vLLM-core] section 2 ("KV Cache management"), copy-on-write item:
 * a page shared by several requests is duplicated only when one of them is
 * about to modify it.
 *
 *   src_dst   device int32 [num_pairs][2]: copy block src_dst[i][0] into block
 *             src_dst[i][1], every slot, every head, in both caches.
 *
 * Pairs run concurrently: no destination may appear twice or also appear as a
 * source (the allocator's copy-on-write pairs always satisfy this).  Pairs
 * with an out-of-range block are skipped by the kernel (and rejected in
 * validation mode).  num_pairs == 0 is valid and launches nothing.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* cache,
                         const int32_t* src_dst, int32_t num_pairs, void* hip_stream);

/* ----------------------------------------------------------------------- */
/* Decode: single-query attention of every sequence over its paged context.
 *
 * Sources: [vLLM-core] section 1 ("PagedAttention: inspiration from virtual
 * memory") -- a logically contiguous cache stored in scattered physical pages
 * reached through a per-sequence page table; [PA-mem] "PagedAttention: the
 * operating system's memory wisdom" -- the per-sequence block table maps
 * logical positions to physical blocks; [nano-KV] "Engineering: configuration
 * and monitoring" -- decode attention reads the paged cache (standard
 * attention being the plain fallback).
 *
 * For every sequence s and query head h (KV head g = h / (num_q_heads /
 * num_kv_heads)), with L = context_lens[s]:
 *     z_p   = scale * dot(q[s][h], K[s, p, g])          p = 0 .. L-1
 *     out[s][h] = sum_p softmax(z)_p * V[s, p, g]
 * where K[s, p, g] is row (p % block_size), head g of physical block
 * block_tables[s][p / block_size].  Accumulation is fp32; the output is
 * rounded to fp16 (round to nearest even) once.  L == 0 gives a zero row.
 *
 *   q              device fp16 [num_seqs][num_q_heads][head_dim]
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]; only the first
 *                  ceil(L / block_size) entries of a row are read.  Entries
 *                  outside [0, num_blocks) are treated as holding no tokens
 *                  (and rejected in validation mode).
 *   context_lens   device int32 [num_seqs]; each must be at most
 *                  max_context_len and at most max_blocks_per_seq*block_size
 *                  (larger values are clamped; rejected in validation mode).
 *   max_context_len  host upper bound of context_lens (longer contexts are
 *                  clamped to it; rejected in validation mode).
 *   scale          softmax scale (commonly 1/sqrt(head_dim)).
 *   out            device fp16 [num_seqs][num_q_heads][head_dim] (written)
 *   num_splits     number of equal pieces N the work is cut into, one
 *                  workgroup each; 0 picks as many as the current device
 *                  holds at once, but no more than the chunk count can reach
 *                  (num_seqs * num_kv_heads * ceil(max_context_len / 16)).  The 16-token chunks of all (sequence, KV
 *                  head) pairs, in sequence-major order, are divided into N
 *                  contiguous ranges.  A pair that straddles ranges gets
 *                  fp32 partials (running max, sum, weighted values) from
 *                  each, which a second kernel combines, in range order, into
 *                  the output (online-softmax merge).  Must be in [-1, 2^20]:
 *                  -1 asks for one workgroup per (sequence, KV head) pair
 *                  whatever the lengths (at most 64 sequences, else
 *                  PA_ERR_RANGE) -- for a caller that knows its contexts are
 *                  of about equal length, where the split is that partition
 *                  anyway and no merge is needed.
 *                  With 0, at most 64 sequences and max_context_len <= 512,
 *                  each workgroup instead takes one whole (sequence, KV head)
 *                  pair and writes its rows directly: a single launch, no
 *                  merge (short contexts, where launches dominate).
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes (same cache, num_seqs, num_q_heads, num_splits, on
 *                  the same device), 256-byte aligned, for those partials.
 *                  Its contents on entry do not matter; calls sharing a
 *                  workspace must not overlap.  Where it applies (slot-major
 *                  layout, groups of 3 to 8 query heads, block_size >= 16, a
 *                  multiple of 4 KV heads), pa_decode_workspace_bytes reports
 *                  the size of the head-group order, in which the 4 waves of a
 *                  workgroup read the same tokens of 4 adjacent KV heads;
 *                  pa_decode takes that order whenever workspace_bytes holds
 *                  it, and the plain order (N + num_seqs * num_kv_heads slots)
 *                  otherwise.
 *
 * Supported: head_dim 64 or 128; block_size 8, 16, 32 or 64; num_q_heads any
 * multiple of num_kv_heads.  A group G = num_q_heads / num_kv_heads of up to 8
 * query heads shares each K/V read (groups of 3 to 8 on matrix cores); a
 * larger group runs as G / g groups of its largest
 * divisor g <= 8, each reading its KV head's rows again (the workspace and
 * the split count then cover num_kv_heads * G / g pairs per sequence).  Other
 * shapes return PA_ERR_UNSUPPORTED.  Results depend only on the context lengths,
 * N and the order (head groups or plain, fixed by the shapes and whether the
 * workspace holds the head-group order), never on which physical blocks hold
 * the tokens or on which workgroup handled which range: moving blocks (and
 * rewriting the tables to match) gives bitwise identical output.
 */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const pa_cache_desc* cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t max_context_len, float scale,
                    void* out, int32_t num_splits,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* pa_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The partial results live in a file-scope device
 * array of 8 MiB (8388608 bytes) that every GPU the library runs on holds
 * until the process ends; the call allocates
 * nothing (no hipMalloc, no host allocation) and does not apply validation
 * mode.  Arguments, layouts and results as pa_decode (same kernels, bitwise
 * the same output for the same num_splits as pa_decode with a workspace of
 * pa_decode_workspace_bytes, whenever the head-group order's partials fit the
 * array; larger calls that still fit in the plain order run that order).
 *
 * Errors: PA_ERR_WORKSPACE, before any launch, when the call's partial
 * results need more than the scratch holds (workspace formula as
 * pa_decode_workspace_bytes); the other errors of pa_decode.
 * Every call on one GPU shares that GPU's scratch and keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialised by the caller. */
pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const pa_cache_desc* cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            float scale, void* out, int32_t num_splits, void* hip_stream);

/* Bytes of workspace pa_decode needs for its faster order: (N + num_seqs *
 * num_kv_heads) slots of G x (head_dim + 2) floats, with G = num_q_heads /
 * num_kv_heads and N the resolved num_splits, each of the two arrays rounded
 * up to 256 bytes; (4N + num_seqs * num_kv_heads) slots where the head-group
 * order applies (slot-major layout, groups of 3 to 8 query heads, block_size
 * >= 16, a multiple of 4 KV heads; a larger group counts its virtual KV
 * heads).  Returns 0 for unsupported or invalid shapes. */
size_t pa_decode_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_splits);

/* The number of splits pa_decode uses at most (resolves 0 from the current
 * device's occupancy, assuming 1024 resident workgroups when no device can be
 * queried; pa_decode may use fewer for a small batch).  Returns 0 for invalid
 * shapes. */
int32_t pa_decode_num_splits(const pa_cache_desc* cache, int32_t num_q_heads,
                             int32_t num_splits);

/* ----------------------------------------------------------------------- */
/* Chunked prefill: causal attention of packed prompt chunks over the cache.
 *
 * Sources: [PA-mem] "Deployable configuration parameters" (prompts are
 * prefilled in chunks, 256 tokens); [vLLM-core] section 3 ("Continuous
 * batching": one batch carries the prefill of several requests); [nano-KV]
 * "Engineering: configuration and monitoring" (prefill attention is a
 * variable-length routine whose plain fallback is standard attention).
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1 (n_s rows):
 * the last n_s tokens of its context of L = context_lens[s] tokens, whose K
 * and V must already be in the caches (pa_store_kvcache).  Row j (KV head
 * g = h / (num_q_heads / num_kv_heads) for query head h) computes
 *     z_p = scale * dot(q[row][h], K[s, p, g])     p = 0 .. L - n_s + j
 *     out[row][h] = sum_p softmax(z)_p * V[s, p, g]
 * with K/V reached through the block table as in pa_decode.  Products and
 * sums are fp32 (matrix cores); the probabilities enter the second product
 * rounded to fp16; the output is rounded to fp16 (nearest even) once.
 *
 *   q, out         device fp16 [num_tokens][num_q_heads][head_dim]
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   device int32 [num_seqs], each in [n_s, max_context_len]
 *                  and at most max_blocks_per_seq * block_size
 *   query_start    device int32 [num_seqs + 1], from 0 to num_tokens, not
 *                  decreasing
 *   max_query_len  at least every n_s: it sizes the grid, and rows past it
 *                  are not written
 *   scale          positive and finite
 *
 * head_dim 64 or 128; block_size a power of two; any group size.  Lengths are clamped
 * on the device so that nothing outside the buffers is read; a key behind an
 * out-of-range table entry takes a zero V row and a zero K row (block_size
 * >= 16) or slot 0's K row (smaller blocks); the result of rows that see it
 * is then unspecified.  PA_VALIDATE
 * checks all of this on the host first.  No
 * workspace; enqueued on hip_stream.
 */
pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache,
                     const pa_cache_desc* cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                     float scale, void* out, void* hip_stream);

/* ----------------------------------------------------------------------- */
/* Host-side block allocator (the block manager).
 *
 * Sources: [PA-mem] "PagedAttention: the operating system's memory wisdom"
 * (a free-block list plus a per-sequence logical-to-physical table; initial
 * blocks on arrival, a new block whenever the current one fills); [PA-mem]
 * "Continuous batching and memory management working together" (a finished
 * request returns all its blocks at once); [vLLM-core] section 2 ("KV Cache
 * management": prefix pages shared between requests, copy-on-write, and
 * reference counts so that a shared page is not released while in use).
 *
 * Policy: the free list is FIFO (blocks taken from the front, returned to
 * the back in logical order); initial_free_order, if not NULL, is a
 * permutation of [0, num_blocks) giving its first order, else 0..n-1.
 * Every operation either succeeds completely or fails with the state
 * unchanged, except PA_ERR_HOST (host memory exhausted mid-operation): the
 * allocator must then be destroyed.  pa_alloc_append_batch is a sequence of
 * such appends: those before a failing one stay applied (*num_done counts
 * them).  Host memory only; one allocator must not be used by two threads at
 * once.  Sequence ids are arbitrary int64 values.
 */
typedef struct pa_allocator pa_allocator;

typedef struct pa_alloc_stats_t {
    int32_t num_blocks;
    int32_t free_blocks;
    int32_t used_blocks;            /* reference count > 0                    */
    int32_t shared_blocks;          /* reference count > 1                    */
    int64_t cow_copies;             /* copy-on-write pairs handed out so far  */
    int64_t live_seqs;
    int64_t logical_tokens;         /* sum of sequence lengths                */
    int64_t stored_tokens;          /* filled slots of used blocks            */
    double utilisation;             /* used_blocks / num_blocks               */
    double internal_fragmentation;  /* empty slots / slots of used blocks     */
} pa_alloc_stats_t;

/* Create an allocator.  block_size and max_blocks_per_seq must be positive. */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          int32_t max_blocks_per_seq,
                          const int32_t* initial_free_order, pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

/* Register sequence `seq` holding n_tokens tokens (n_tokens >= 0); takes
 * ceil(n_tokens / block_size) blocks.  slots_out (nullable, host int32
 * [n_tokens]) receives the slot of every token in order. */
pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq, int32_t n_tokens,
                           int32_t* slots_out);

/* `child` starts as a copy of `parent`, sharing (and counting) every block. */
pa_status pa_alloc_fork(pa_allocator* a, int64_t parent, int64_t child);

/* Reserve the slot of the sequence's next token.  A fresh block is taken when
 * the last block is full.  When the last block is partly filled and shared,
 * the sequence moves to a fresh block and (*cow_src, *cow_dst) name the copy
 * the caller must make (pa_copy_blocks) before storing; otherwise both are
 * -1. */
pa_status pa_alloc_append_slot(pa_allocator* a, int64_t seq, int32_t* slot,
                               int32_t* cow_src, int32_t* cow_dst);

/* One decode step for a batch: pa_alloc_append_slot on seqs[0..n) in order.
 * slots_out: host int32 [n]; cow_pairs_out: host int32 [n][2] receives the
 * copies in order, their count in *num_cow.  On failure *num_done tells how
 * many appends succeeded (those stay applied). */
pa_status pa_alloc_append_batch(pa_allocator* a, const int64_t* seqs, int32_t n,
                                int32_t* slots_out, int32_t* cow_pairs_out,
                                int32_t* num_cow, int32_t* num_done);

/* Drop a finished sequence; blocks whose count reaches 0 go back on the list. */
pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq);

/* Write block tables (host int32 [n][row_stride], padding -1) and context
 * lengths (host int32 [n], nullable) of seqs[0..n). */
pa_status pa_alloc_export(const pa_allocator* a, const int64_t* seqs, int32_t n,
                          int32_t row_stride, int32_t* block_tables_out,
                          int32_t* context_lens_out);

/* Counters of the allocator's state (copied into *out). */
pa_status pa_alloc_stats(const pa_allocator* a, pa_alloc_stats_t* out);

/* Reference count of a block, or -1 if out of range. */
int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block);

/* Number of free blocks. */
int32_t pa_alloc_num_free(const pa_allocator* a);

/* Copy up to `cap` entries of the free list, front first; returns the count
 * written (for inspection and tests). */
int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap);

/* Length (tokens) and block count of a sequence. */
pa_status pa_alloc_seq_info(const pa_allocator* a, int64_t seq,
                            int32_t* n_tokens, int32_t* n_blocks);

/* Register sequence `seq` by its token ids, sharing cached full blocks.
 *
 * Source: [PA-mem] "Architectural limits" and "Engineering: configuration
 * and monitoring" (prefix caching; its hit rate as a metric); [vLLM-core]
 * section 2 (pages of a common prefix are shared).
 *
 * tokens: host int32 [n_tokens].  Every full block is keyed by a chained
 * content hash: 64-bit FNV-1a over the previous block's key (8 bytes,
 * little-endian; 0 for the first block) and the block's token ids (4 bytes
 * each, little-endian).  The leading run of full blocks whose key, token ids
 * and previous block all match a live cached block is shared (reference
 * count + 1); the rest are taken from the free list, and each new full block
 * whose key is not yet cached is cached.  A partial last block is never
 * cached or shared; blocks filled later by appends are not cached.  A block
 * leaves the cache when its reference count reaches 0.
 *
 * slots_out (nullable, host int32 [n_tokens]) receives every token's slot;
 * *n_cached receives the number of leading tokens whose K/V already sit in
 * shared blocks (a multiple of block_size): the caller stores only tokens
 * from *n_cached on.  Errors as pa_alloc_add_seq, with the shared blocks not
 * counted against the free list. */
pa_status pa_alloc_add_seq_tokens(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                  int32_t n_tokens, int32_t* slots_out, int32_t* n_cached);

/* Renumber blocks so that every used block lies below the number of used
 * blocks u.
 *
 * Source: [PA-mem] "Continuous batching and memory management working
 * together" (compaction against fragmentation, weighed against the cost of
 * moving data).
 *
 * Each used block numbered u or above, in increasing order, takes the lowest
 * free block below u not yet taken; block tables, reference counts and the
 * prefix cache follow; the free list becomes u, u+1, ..., num_blocks-1.
 * pairs_out (host int32 [max_pairs][2]) receives the (src, dst) moves in
 * increasing src order; every src >= u > every dst, so no move overwrites
 * another's source and one pa_copy_blocks call on each layer's caches
 * applies them all.  The caller must make those copies before the next
 * store or decode that uses the new tables.
 * *n_pairs always receives the number of moves; if it exceeds max_pairs the
 * call fails with PA_ERR_RANGE and changes nothing (at most
 * min(u, num_blocks - u) moves are ever needed). */
pa_status pa_alloc_compact(pa_allocator* a, int32_t* pairs_out, int32_t max_pairs,
                           int32_t* n_pairs);

/* Prefix-cache counters: tokens asked for through pa_alloc_add_seq_tokens,
 * tokens found cached, and blocks currently cached. */
pa_status pa_alloc_prefix_stats(const pa_allocator* a, int64_t* queried_tokens,
                                int64_t* hit_tokens, int32_t* cached_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */

// Internal launch interface between the C ABI (capi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pa {

// Arguments of one paged decode call, already checked by the caller.
struct DecodeArgs {
    const uint16_t* q;             // fp16 [B][Hq][D]
    const uint16_t* k_cache;       // fp16 [NB][BS][Hkv][D]
    const uint16_t* v_cache;
    const int32_t* block_tables;   // [B][M]
    const int32_t* context_lens;   // [B]
    uint16_t* out;                 // fp16 [B][Hq][D]
    float* part_o;                 // fp32 [N + B*Hkv][G][D]  partial outputs per slot
    float* part_ml;                // fp32 [N + B*Hkv][G][2]  (running max, sum) per slot
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t num_q_heads;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;    // M, row stride of block_tables
    int32_t max_tokens;            // clamp of context lengths
    int32_t num_splits;            // N: equal pieces of the chunk list, one workgroup each
    float scale_log2;              // scale * log2(e)
    int32_t whole_pairs;           // 1: workgroup w takes (sequence, KV head) pair w whole
                                   // (N = num_seqs * num_kv_heads, at most 64 sequences, no merge)
    int32_t head_major;            // 1: cache [NB][Hkv][BS][D], else [NB][BS][Hkv][D]
    int32_t kv_split;              // virtual KV heads per KV head (>= 1): a query group of
                                   // G > 8 heads runs as kv_split groups of G / kv_split
    int32_t head_groups;           // 1: the matrix-core kernel may order each sequence's chunk
                                   // list by groups of 4 (virtual) KV heads (decode.hip); needs
                                   // num_kv_heads * kv_split % 4 == 0 and 4 * N + pairs slots;
                                   // the host sets it for the slot-major layout only
    int32_t num_splits_hg;         // 0, or a split count below num_splits (two workgroups a
                                   // compute unit) that the matrix-core and merge kernels use
                                   // instead when every sequence then takes the head-group order
};

// The query group a decode kernel takes (at most 8 heads) and how many such
// groups each KV head's group is cut into.
struct GroupSplit {
    int group;
    int kv_split;
};
GroupSplit decode_group_split(int group);

// group: heads per kernel group (1..8, after decode_group_split).
bool decode_supported(int head_dim, int block_size, int group);
// Whether the kernel for this block size and group (1..8) can order the chunk
// list by head groups: the matrix-core kernel, with a multiple of 4 (virtual)
// KV heads.
bool decode_head_groups_ok(int block_size, int group, int virtual_kv_heads);
// Workgroups of the decode kernel for these shapes that the current device
// holds at once; 0 when no device can be queried.
int decode_resident_workgroups(int head_dim, int block_size, int group);
// Compute units of the current device; 0 when it cannot be queried.
int decode_compute_units();
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Arguments of one chunked-prefill call, already checked by the caller.
struct PrefillArgs {
    const uint16_t* q;             // fp16 [T][Hq][D], chunk rows of all sequences, packed
    const uint16_t* k_cache;       // fp16 [NB][BS][Hkv][D]
    const uint16_t* v_cache;
    const int32_t* block_tables;   // [B][M]
    const int32_t* context_lens;   // [B], including the chunk
    const int32_t* query_start;    // [B + 1]
    uint16_t* out;                 // fp16 [T][Hq][D]
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t num_q_heads;
    int32_t num_seqs;
    int32_t num_tokens;            // T
    int32_t max_blocks_per_seq;    // M
    int32_t max_tokens;            // M * BS, clamp of context lengths
    int32_t max_query_len;         // bound on every chunk length (grid size)
    int32_t tiles_per_seq;         // set by the launcher
    int32_t block_shift;           // log2(block_size)
    float scale_log2;              // scale * log2(e), > 0
    int32_t head_major;            // 1: cache [NB][Hkv][BS][D], else [NB][BS][Hkv][D]
};

bool prefill_supported(int head_dim, int block_size);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// head_major: the cache is [NB][Hkv][BS][D] (else [NB][BS][Hkv][D]);
// head_vec16 = D / 8.
hipError_t launch_store_kvcache(const void* k, const void* v, const int32_t* slots,
                                int32_t num_tokens, void* k_cache, void* v_cache,
                                int32_t row_vec16, int64_t total_slots, bool head_major,
                                int32_t block_size, int32_t head_vec16, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, int64_t block_vec16, int32_t num_blocks,
                              hipStream_t stream);

}  // namespace pa

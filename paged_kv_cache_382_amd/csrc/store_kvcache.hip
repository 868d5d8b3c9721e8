// Store of the step's new K/V rows into the block-paged cache.
//
// Source: "Deep analysis of nano-vLLM's paged KV cache and memory
// optimisation architecture", section "Core mechanism of the paged KV cache":
// each new token's key and value rows are written to the cache slot named by
// a per-token slot mapping, with the cache seen as a flat array of slots.
//
// Design (store): one token row (num_kv_heads * head_dim fp16, contiguous in the
// input and in a slot-major cache; in a head-major cache each head's piece goes
// to that head's run of the block) is moved as 16-byte words.  grid.x walks
// tokens, grid.y splits a row over 256-lane workgroups so that a large row
// (8 KiB for 32 heads x 128) still spreads over several CUs.  The data never
// passes through a floating-point register: NaN payloads are preserved.

#include "kernels.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ slots, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int32_t row_vec16, int64_t total_slots, int32_t head_major,
    int32_t block_size, int32_t head_vec16) {
    const int32_t t = blockIdx.x;
    const int32_t i = blockIdx.y * 256 + threadIdx.x;
    const int32_t slot = slots[t];
    if (slot < 0 || slot >= total_slots || i >= row_vec16) return;
    const size_t src = static_cast<size_t>(t) * row_vec16 + i;
    // Word i of the token row is word (i % head_vec16) of KV head i / head_vec16.
    // Slot-major: the row is contiguous at slot * row.  Head-major: the head's
    // word sits in its run of block_size rows inside the slot's block.
    size_t dst = static_cast<size_t>(slot) * row_vec16 + i;
    if (head_major) {
        const int32_t blk = slot / block_size;
        const int32_t off = slot - blk * block_size;
        const int32_t h = i / head_vec16;
        const int32_t w = i - h * head_vec16;
        dst = (static_cast<size_t>(blk) * row_vec16 + static_cast<size_t>(h) * head_vec16) * block_size +
              static_cast<size_t>(off) * head_vec16 + w;
    }
    const uint4 kw = k[src];
    const uint4 vw = v[src];
    k_cache[dst] = kw;
    v_cache[dst] = vw;
}

// Block copy.  A workgroup moves one tile of kCopyUnroll * 256 16-byte words
// of one pair, in both caches: every lane issues all of its K and V loads
// before its first store, so 8 loads per lane are in flight.  The caches are
// far larger than L2 and the copied block is not read back soon, so loads and
// stores bypass it (non-temporal).
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyTile = 256 * kCopyUnroll;
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    u4* __restrict__ k_cache, u4* __restrict__ v_cache, const int32_t* __restrict__ pairs,
    int64_t block_vec16, int32_t num_blocks, int32_t tiles_per_block) {
    const int32_t pair = blockIdx.x / tiles_per_block;
    const int32_t tile = blockIdx.x - pair * tiles_per_block;
    const int32_t src = pairs[2 * pair];
    const int32_t dst = pairs[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const int64_t base = tile * kCopyTile + threadIdx.x;
    const u4* ks = k_cache + src * block_vec16;
    const u4* vs = v_cache + src * block_vec16;
    u4* kd = k_cache + dst * block_vec16;
    u4* vd = v_cache + dst * block_vec16;
    u4 kw[kCopyUnroll], vw[kCopyUnroll];
    if (base + (kCopyUnroll - 1) * 256 < block_vec16) {
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            kw[u] = __builtin_nontemporal_load(ks + base + u * 256);
            vw[u] = __builtin_nontemporal_load(vs + base + u * 256);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            __builtin_nontemporal_store(kw[u], kd + base + u * 256);
            __builtin_nontemporal_store(vw[u], vd + base + u * 256);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * 256;
            if (i < block_vec16) {
                kd[i] = ks[i];
                vd[i] = vs[i];
            }
        }
    }
}

}  // namespace

hipError_t launch_store_kvcache(const void* k, const void* v, const int32_t* slots,
                                int32_t num_tokens, void* k_cache, void* v_cache,
                                int32_t row_vec16, int64_t total_slots, bool head_major,
                                int32_t block_size, int32_t head_vec16, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>(num_tokens), static_cast<unsigned>((row_vec16 + 255) / 256));
    hipLaunchKernelGGL(store_kvcache_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), row_vec16,
                       total_slots, head_major ? 1 : 0, block_size, head_vec16);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, int64_t block_vec16, int32_t num_blocks,
                              hipStream_t stream) {
    if (num_pairs <= 0) return hipSuccess;
    const int64_t tiles = (block_vec16 + kCopyTile - 1) / kCopyTile;
    const int64_t grid = tiles * num_pairs;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       static_cast<u4*>(k_cache), static_cast<u4*>(v_cache), pairs, block_vec16,
                       num_blocks, static_cast<int32_t>(tiles));
    return hipGetLastError();
}

}  // namespace pa

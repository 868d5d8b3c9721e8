// Store of the step's new K/V rows into the block-paged cache.
//
// Source: "Deep analysis of nano-vLLM's paged KV cache and memory
// optimisation architecture", section "Core mechanism of the paged KV cache":
// each new token's key and value rows are written to the cache slot named by
// a per-token slot mapping, with the cache seen as a flat array of slots.
//
// Design: one token row (num_kv_heads * head_dim fp16, contiguous in both the
// input and the slot-major cache) is moved as 16-byte words.  grid.x walks
// tokens, grid.y splits a row over 256-lane workgroups so that a large row
// (8 KiB for 32 heads x 128) still spreads over several CUs.  The data never
// passes through a floating-point register: NaN payloads are preserved.

#include "kernels.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ slots, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int32_t row_vec16, int64_t total_slots) {
    const int32_t t = blockIdx.x;
    const int32_t i = blockIdx.y * 256 + threadIdx.x;
    const int32_t slot = slots[t];
    if (slot < 0 || slot >= total_slots || i >= row_vec16) return;
    const size_t src = static_cast<size_t>(t) * row_vec16 + i;
    const size_t dst = static_cast<size_t>(slot) * row_vec16 + i;
    const uint4 kw = k[src];
    const uint4 vw = v[src];
    k_cache[dst] = kw;
    v_cache[dst] = vw;
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ pairs, int64_t block_vec16, int32_t num_blocks) {
    const int32_t src = pairs[2 * blockIdx.x];
    const int32_t dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const size_t s0 = static_cast<size_t>(src) * block_vec16;
    const size_t d0 = static_cast<size_t>(dst) * block_vec16;
    for (int64_t i = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x; i < block_vec16;
         i += static_cast<int64_t>(gridDim.y) * 256) {
        const uint4 kw = k_cache[s0 + i];
        const uint4 vw = v_cache[s0 + i];
        k_cache[d0 + i] = kw;
        v_cache[d0 + i] = vw;
    }
}

}  // namespace

hipError_t launch_store_kvcache(const void* k, const void* v, const int32_t* slots,
                                int32_t num_tokens, void* k_cache, void* v_cache,
                                int32_t row_vec16, int64_t total_slots, hipStream_t stream) {
    if (num_tokens <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>(num_tokens), static_cast<unsigned>((row_vec16 + 255) / 256));
    hipLaunchKernelGGL(store_kvcache_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), row_vec16,
                       total_slots);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int32_t num_pairs, int64_t block_vec16, int32_t num_blocks,
                              hipStream_t stream) {
    if (num_pairs <= 0) return hipSuccess;
    int64_t ys = (block_vec16 + 255) / 256;
    if (ys > 64) ys = 64;
    dim3 grid(static_cast<unsigned>(num_pairs), static_cast<unsigned>(ys));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs,
                       block_vec16, num_blocks);
    return hipGetLastError();
}

}  // namespace pa

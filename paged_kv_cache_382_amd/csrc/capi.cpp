// C ABI of the device calls: argument checks, optional deep validation of the
// integer metadata, workspace sizing and kernel dispatch.  Every check runs
// before any launch, so a failing call enqueues nothing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace pa {

char* error_text() {
    static thread_local char text[kErrorChars] = {0};
    return text;
}

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Workgroups assumed resident when the device cannot be queried (no GPU).
constexpr int32_t kFallbackResident = 1024;
constexpr int32_t kMaxSplits = 1 << 20;

int validate_from_env() {
    const char* e = std::getenv("PA_VALIDATE");
    return (e && e[0] == '1') ? 1 : 0;
}

int& validate_flag() {
    static int flag = validate_from_env();
    return flag;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status check_cache(const pa_cache_desc* c, const char* fn) {
    if (!c) return fail(PA_ERR_NULL, "%s: cache descriptor is NULL", fn);
    if (c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
        return fail(PA_ERR_SHAPE, "%s: cache sizes must be positive", fn);
    if (static_cast<int64_t>(c->num_blocks) * c->block_size > INT32_MAX)
        return fail(PA_ERR_RANGE, "%s: num_blocks * block_size exceeds the int32 slot range", fn);
    if (c->layout != PA_LAYOUT_SLOT_MAJOR && c->layout != PA_LAYOUT_HEAD_MAJOR)
        return fail(PA_ERR_UNSUPPORTED, "%s: cache layout %d not supported", fn, c->layout);
    return PA_OK;
}

// Copy `n` int32 values from device memory to the host (validation mode only).
pa_status fetch(const int32_t* dev, size_t n, std::vector<int32_t>& host, hipStream_t stream,
                const char* fn) {
    host.resize(n);
    if (n == 0) return PA_OK;
    hipError_t err = hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: validation copy failed: %s", fn, hipGetErrorString(err));
    return PA_OK;
}

// Query heads per kernel group and virtual KV heads per KV head.
GroupSplit group_split(const pa_cache_desc* c, int32_t num_q_heads) {
    return decode_group_split(num_q_heads / c->num_kv_heads);
}

int32_t resident_workgroups(const pa_cache_desc* c, int32_t num_q_heads) {
    const int r = decode_resident_workgroups(c->head_dim, c->block_size, group_split(c, num_q_heads).group);
    return r > 0 ? r : kFallbackResident;
}

// Default split count: one per workgroup the device holds at once, so the
// whole grid runs in a single round.
int32_t resolve_splits(const pa_cache_desc* c, int32_t num_q_heads, int32_t requested) {
    if (requested > 0) return requested;
    return std::min<int32_t>(resident_workgroups(c, num_q_heads), kMaxSplits);
}

// Contexts of at most this many tokens (and at most 64 sequences) are decoded
// one workgroup per (sequence, KV head) pair: every pair is short, so the
// grid stays balanced, and no merge launch is needed.
constexpr int64_t kWholePairMaxTokens = 512;
// num_splits value asking for one workgroup per pair whatever the lengths: for
// a caller that knows its contexts are (nearly) equal, where the balanced
// split is this partition anyway and the merge launch would find nothing.
constexpr int32_t kWholePairs = -1;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Whether decode orders each sequence's chunk list by groups of 4 (virtual)
// KV heads: the matrix-core kernel with a multiple of 4 virtual KV heads, on
// the slot-major layout, where the 4 waves of a workgroup then read 1 KiB of
// each token row together (head-major blocks already hold a head's rows
// contiguously, and there the plain order measured faster).
bool head_groups_ok(const pa_cache_desc* c, int32_t num_q_heads) {
    const GroupSplit gs = group_split(c, num_q_heads);
    return c->layout == PA_LAYOUT_SLOT_MAJOR &&
           decode_head_groups_ok(c->block_size, gs.group, c->num_kv_heads * gs.kv_split);
}

// Partial-result slots: one per split plus one per (sequence, KV head) pair
// (virtual KV heads for a large query group), each of `group` rows; in the
// head-group order four per split plus one per pair.
size_t partial_rows(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads, int32_t splits, bool hg) {
    const GroupSplit gs = group_split(c, num_q_heads);
    const size_t slots = static_cast<size_t>(splits) * (hg ? 4 : 1) +
                         static_cast<size_t>(num_seqs) * c->num_kv_heads * gs.kv_split;
    return slots * static_cast<size_t>(gs.group);
}

// Workspace layout: part_ml fp32 [slots][G][2], then part_o fp32
// [slots][G][D], each 256-byte aligned.
size_t workspace_for(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads, int32_t splits, bool hg) {
    const size_t rows = partial_rows(c, num_seqs, num_q_heads, splits, hg);
    return round_up(rows * 2 * sizeof(float)) + round_up(rows * c->head_dim * sizeof(float));
}

pa_status check_decode_shapes(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len, int32_t num_splits, const char* fn) {
    pa_status st = check_cache(c, fn);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
        return fail(PA_ERR_SHAPE, "%s: num_seqs, num_q_heads and max_context_len must be >= 0 / > 0", fn);
    if (num_q_heads % c->num_kv_heads != 0)
        return fail(PA_ERR_SHAPE, "%s: num_q_heads (%d) is not a multiple of num_kv_heads (%d)", fn,
                    num_q_heads, c->num_kv_heads);
    if (!decode_supported(c->head_dim, c->block_size, group_split(c, num_q_heads).group))
        return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d, block_size %d, group %d not supported", fn,
                    c->head_dim, c->block_size, num_q_heads / c->num_kv_heads);
    if (num_splits < kWholePairs || num_splits > kMaxSplits)
        return fail(PA_ERR_RANGE, "%s: num_splits must be in [-1, %d]", fn, kMaxSplits);
    return PA_OK;
}

}  // namespace
}  // namespace pa

namespace pa {
namespace {

// Device memory of pa_decode_noalloc's partial results: a file-scope array of
// kScratchBytes on every GPU the library runs on, held until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress and kept here.
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex& scratch_mutex() {
    static std::mutex m;
    return m;
}
void* scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (looked up on its first use).
pa_status scratch_for_current_device(void** out, const char* fn) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(PA_ERR_RANGE, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(scratch_mutex());
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(err));
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return PA_OK;
}

// The whole of a decode call after the workspace is known.  `workspace` is
// the caller's buffer, or (scratch_ws) the library's own device array, in
// which case validation mode is not applied (it would allocate host memory
// and synchronise).
pa_status decode_call(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                      const pa_cache_desc* cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t max_context_len, float scale, void* out,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* hip_stream, bool scratch_ws) {
    {
        pa_status st = check_decode_shapes(cache, num_seqs, num_q_heads, max_context_len,
                                               num_splits, fn);
        if (st != PA_OK) return st;
        if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq must be positive", fn);
        if (num_seqs == 0) return ok();
        if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
            return fail(PA_ERR_NULL, "%s: NULL pointer", fn);
        if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
            return fail(PA_ERR_ALIGN, "%s: fp16 pointers must be 16-byte aligned", fn);
        const int64_t max_tokens64 = std::min<int64_t>(static_cast<int64_t>(max_blocks_per_seq) * cache->block_size,
                                                       max_context_len);
        int32_t splits = resolve_splits(cache, num_q_heads, num_splits);
        if (num_splits == 0) {
            // No more splits than chunks can exist: small batches launch a small grid.
            const int64_t chunk_bound = static_cast<int64_t>(num_seqs) * cache->num_kv_heads *
                                        group_split(cache, num_q_heads).kv_split *
                                        ((max_tokens64 + 15) / 16);
            splits = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(splits, chunk_bound)));
        }
        // The plain order needs `need`; the head-group order (faster, when the
        // kernel allows it) needs `need_hg` and is used whenever the
        // workspace holds it.
        const bool hg_ok = head_groups_ok(cache, num_q_heads);
        const size_t need = workspace_for(cache, num_seqs, num_q_heads, splits, false);
        const size_t need_hg = hg_ok ? workspace_for(cache, num_seqs, num_q_heads, splits, true) : need;
        if (scratch_ws) {
            // The library's own array: checked for size before the device
            // address is looked up (every argument check precedes it).
            if (need > kScratchBytes)
                return fail(PA_ERR_WORKSPACE,
                            "%s: this call needs %zu bytes of partial results; the built-in scratch "
                            "holds %zu (call pa_decode with a workspace instead)", fn, need, kScratchBytes);
            const pa_status sst = scratch_for_current_device(&workspace, fn);
            if (sst != PA_OK) return sst;
            workspace_bytes = kScratchBytes;
        }
        if (!workspace) return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes required", fn, need_hg);
        if (workspace_bytes < need)
            return fail(PA_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu required (%zu for the faster order)",
                        fn, workspace_bytes, need, need_hg);
        const bool hg = hg_ok && workspace_bytes >= need_hg;
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
            return fail(PA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
        const GroupSplit gsplit = group_split(cache, num_q_heads);
        const int64_t pairs = static_cast<int64_t>(num_seqs) * cache->num_kv_heads * gsplit.kv_split;
        if (pairs > INT32_MAX) return fail(PA_ERR_SHAPE, "%s: launch too large (%lld pairs)", fn, (long long)pairs);
        hipStream_t stream = static_cast<hipStream_t>(hip_stream);
        if (validate_flag() && !scratch_ws) {
            std::vector<int32_t> lens, tables;
            st = fetch(context_lens, static_cast<size_t>(num_seqs), lens, stream, fn);
            if (st != PA_OK) return st;
            st = fetch(block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, tables, stream, fn);
            if (st != PA_OK) return st;
            for (int32_t s = 0; s < num_seqs; ++s) {
                const int32_t L = lens[s];
                if (L < 0 || L > max_tokens64)
                    return fail(PA_ERR_RANGE, "%s: context_lens[%d] = %d outside [0, %lld]", fn, s, L,
                                (long long)max_tokens64);
                const int32_t used = (L + cache->block_size - 1) / cache->block_size;
                for (int32_t j = 0; j < used; ++j) {
                    const int32_t b = tables[static_cast<size_t>(s) * max_blocks_per_seq + j];
                    if (b < 0 || b >= cache->num_blocks)
                        return fail(PA_ERR_RANGE, "%s: block_tables[%d][%d] = %d out of range", fn, s, j, b);
                }
            }
        }
        DecodeArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.k_cache = static_cast<const uint16_t*>(k_cache);
        a.v_cache = static_cast<const uint16_t*>(v_cache);
        a.block_tables = block_tables;
        a.context_lens = context_lens;
        a.out = static_cast<uint16_t*>(out);
        {
            const size_t rows = partial_rows(cache, num_seqs, num_q_heads, splits, hg);
            char* ws = static_cast<char*>(workspace);
            a.part_ml = reinterpret_cast<float*>(ws);
            a.part_o = reinterpret_cast<float*>(ws + round_up(rows * 2 * sizeof(float)));
        }
        a.num_blocks = cache->num_blocks;
        a.block_size = cache->block_size;
        a.num_kv_heads = cache->num_kv_heads;
        a.head_dim = cache->head_dim;
        a.num_q_heads = num_q_heads;
        a.num_seqs = num_seqs;
        a.max_blocks_per_seq = max_blocks_per_seq;
        a.max_tokens = static_cast<int32_t>(max_tokens64);
        a.num_splits = splits;
        a.scale_log2 = scale * kLog2e;
        a.head_major = cache->layout == PA_LAYOUT_HEAD_MAJOR;
        a.kv_split = gsplit.kv_split;
        a.head_groups = hg ? 1 : 0;
        // With the split count left to the library, a batch whose sequences all
        // take the head-group order runs on two workgroups a compute unit (the
        // kernels decide, from the lengths they read): it streams faster so
        // (mixed lengths 101.6 vs 104.3 us a call, prefix sharing 66.5 vs 77.6),
        // while the plain order keeps three (4 x 131072 tokens 341 vs 355 us).
        a.num_splits_hg = 0;
        if (hg && num_splits == 0) {
            const int cus = decode_compute_units();
            if (cus > 0 && splits > 2 * cus) a.num_splits_hg = 2 * cus;
        }
        a.whole_pairs = 0;
        if (num_splits == kWholePairs && num_seqs > 64)
            return fail(PA_ERR_RANGE, "%s: num_splits -1 (whole pairs) takes at most 64 sequences", fn);
        if (num_splits == kWholePairs ||
            (num_splits == 0 && num_seqs <= 64 && max_tokens64 <= kWholePairMaxTokens)) {
            a.whole_pairs = 1;
            a.num_splits = static_cast<int32_t>(pairs);
        }
        hipError_t err = launch_decode(a, stream);
        if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
        return ok();
    }
}

}  // namespace
}  // namespace pa

using pa::fail;
using pa::ok;

extern "C" {

const char* pa_last_error(void) { return pa::error_text(); }

const char* pa_version(void) { return "0.2.0"; }

int pa_set_validate(int on) {
    int prev = pa::validate_flag();
    pa::validate_flag() = on ? 1 : 0;
    return prev;
}

pa_status pa_store_kvcache(const void* k, const void* v, const int32_t* slot_mapping,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           const pa_cache_desc* cache, void* hip_stream) {
    return pa::guard("pa_store_kvcache", [&]() -> pa_status {
        static const char* fn = "pa_store_kvcache";
        pa_status st = pa::check_cache(cache, fn);
        if (st != PA_OK) return st;
        if (num_tokens < 0) return fail(PA_ERR_SHAPE, "%s: negative num_tokens", fn);
        if (cache->head_dim % 8 != 0) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 8", fn);
        if (num_tokens == 0) return ok();
        if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_NULL, "%s: NULL pointer", fn);
        if (!pa::aligned16(k) || !pa::aligned16(v) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache))
            return fail(PA_ERR_ALIGN, "%s: fp16 pointers must be 16-byte aligned", fn);
        const int64_t total_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
        const int64_t row_vec16 = static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim / 8;
        if (row_vec16 > INT32_MAX / 2) return fail(PA_ERR_SHAPE, "%s: row too large", fn);
        hipStream_t stream = static_cast<hipStream_t>(hip_stream);
        if (pa::validate_flag()) {
            std::vector<int32_t> slots;
            st = pa::fetch(slot_mapping, static_cast<size_t>(num_tokens), slots, stream, fn);
            if (st != PA_OK) return st;
            std::unordered_set<int32_t> seen;
            for (int32_t t = 0; t < num_tokens; ++t) {
                int32_t s = slots[t];
                if (s < 0) continue;
                if (s >= total_slots) return fail(PA_ERR_RANGE, "%s: slot %d of token %d out of range", fn, s, t);
                if (!seen.insert(s).second) return fail(PA_ERR_RANGE, "%s: slot %d written twice", fn, s);
            }
        }
        hipError_t err = pa::launch_store_kvcache(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                                  static_cast<int32_t>(row_vec16), total_slots,
                                                  cache->layout == PA_LAYOUT_HEAD_MAJOR, cache->block_size,
                                                  cache->head_dim / 8, stream);
        if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
        return ok();
    });
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* cache,
                         const int32_t* src_dst, int32_t num_pairs, void* hip_stream) {
    return pa::guard("pa_copy_blocks", [&]() -> pa_status {
        static const char* fn = "pa_copy_blocks";
        pa_status st = pa::check_cache(cache, fn);
        if (st != PA_OK) return st;
        if (num_pairs < 0) return fail(PA_ERR_SHAPE, "%s: negative num_pairs", fn);
        if (cache->head_dim % 8 != 0) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 8", fn);
        if (num_pairs == 0) return ok();
        if (!k_cache || !v_cache || !src_dst) return fail(PA_ERR_NULL, "%s: NULL pointer", fn);
        if (!pa::aligned16(k_cache) || !pa::aligned16(v_cache))
            return fail(PA_ERR_ALIGN, "%s: caches must be 16-byte aligned", fn);
        hipStream_t stream = static_cast<hipStream_t>(hip_stream);
        if (pa::validate_flag()) {
            std::vector<int32_t> pairs;
            st = pa::fetch(src_dst, static_cast<size_t>(num_pairs) * 2, pairs, stream, fn);
            if (st != PA_OK) return st;
            std::unordered_set<int32_t> dsts, srcs;
            for (int32_t i = 0; i < num_pairs; ++i) {
                int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
                if (s < 0 || s >= cache->num_blocks || d < 0 || d >= cache->num_blocks)
                    return fail(PA_ERR_RANGE, "%s: pair %d (%d, %d) out of range", fn, i, s, d);
                if (!dsts.insert(d).second) return fail(PA_ERR_RANGE, "%s: destination %d repeated", fn, d);
                srcs.insert(s);
            }
            for (int32_t d : dsts)
                if (srcs.count(d)) return fail(PA_ERR_RANGE, "%s: block %d is both source and destination", fn, d);
        }
        const int64_t block_vec16 = static_cast<int64_t>(cache->block_size) * cache->num_kv_heads * cache->head_dim / 8;
        hipError_t err = pa::launch_copy_blocks(k_cache, v_cache, src_dst, num_pairs, block_vec16,
                                                cache->num_blocks, stream);
        if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
        return ok();
    });
}

size_t pa_decode_workspace_bytes(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_splits) {
    if (pa::check_decode_shapes(cache, num_seqs, num_q_heads, 0, num_splits,
                                "pa_decode_workspace_bytes") != PA_OK)
        return 0;
    return pa::workspace_for(cache, num_seqs, num_q_heads,
                             pa::resolve_splits(cache, num_q_heads, num_splits),
                             pa::head_groups_ok(cache, num_q_heads));
}

int32_t pa_decode_num_splits(const pa_cache_desc* cache, int32_t num_q_heads, int32_t num_splits) {
    if (pa::check_decode_shapes(cache, 1, num_q_heads, 0, num_splits, "pa_decode_num_splits") != PA_OK)
        return 0;
    return pa::resolve_splits(cache, num_q_heads, num_splits);
}

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const pa_cache_desc* cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t max_context_len, float scale, void* out,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    void* hip_stream) {
    return pa::guard("pa_decode", [&]() -> pa_status {
        return pa::decode_call("pa_decode", q, k_cache, v_cache, cache, block_tables,
                               max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                               max_context_len, scale, out, num_splits, workspace, workspace_bytes,
                               hip_stream, false);
    });
}

pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const pa_cache_desc* cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            float scale, void* out, int32_t num_splits, void* hip_stream) {
    return pa::guard("pa_decode_noalloc", [&]() -> pa_status {
        return pa::decode_call("pa_decode_noalloc", q, k_cache, v_cache, cache, block_tables,
                               max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                               max_context_len, scale, out, num_splits, nullptr, 0, hip_stream, true);
    });
}

pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache,
                     const pa_cache_desc* cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                     float scale, void* out, void* hip_stream) {
    return pa::guard("pa_prefill", [&]() -> pa_status {
        static const char* fn = "pa_prefill";
        pa_status st = pa::check_cache(cache, fn);
        if (st != PA_OK) return st;
        if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || max_query_len < 0 || max_context_len < 0)
            return fail(PA_ERR_SHAPE, "%s: negative size or num_q_heads <= 0", fn);
        if (num_q_heads % cache->num_kv_heads != 0)
            return fail(PA_ERR_SHAPE, "%s: num_q_heads (%d) is not a multiple of num_kv_heads (%d)", fn,
                        num_q_heads, cache->num_kv_heads);
        if (!pa::prefill_supported(cache->head_dim, cache->block_size))
            return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d / block_size %d not supported (64 or 128; a power of two)",
                        fn, cache->head_dim, cache->block_size);
        if (max_blocks_per_seq <= 0) return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq must be positive", fn);
        if (!(scale > 0.0f) || scale > 1e30f) return fail(PA_ERR_RANGE, "%s: scale must be positive and finite", fn);
        if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return ok();
        if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
            return fail(PA_ERR_NULL, "%s: NULL pointer", fn);
        if (!pa::aligned16(q) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache) || !pa::aligned16(out))
            return fail(PA_ERR_ALIGN, "%s: fp16 pointers must be 16-byte aligned", fn);
        const int64_t max_tokens64 = std::min<int64_t>(static_cast<int64_t>(max_blocks_per_seq) * cache->block_size,
                                                       max_context_len);
        const int64_t rows = static_cast<int64_t>(max_query_len) * (num_q_heads / cache->num_kv_heads);
        if (static_cast<int64_t>(num_seqs) * cache->num_kv_heads * ((rows + 127) / 128) > INT32_MAX / 2)
            return fail(PA_ERR_SHAPE, "%s: launch too large", fn);
        hipStream_t stream = static_cast<hipStream_t>(hip_stream);
        if (pa::validate_flag()) {
            std::vector<int32_t> lens, starts, tables;
            st = pa::fetch(context_lens, static_cast<size_t>(num_seqs), lens, stream, fn);
            if (st == PA_OK) st = pa::fetch(query_start, static_cast<size_t>(num_seqs) + 1, starts, stream, fn);
            if (st == PA_OK)
                st = pa::fetch(block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, tables, stream, fn);
            if (st != PA_OK) return st;
            if (starts[0] != 0 || starts[num_seqs] != num_tokens)
                return fail(PA_ERR_RANGE, "%s: query_start must run from 0 to num_tokens (%d)", fn, num_tokens);
            for (int32_t s = 0; s < num_seqs; ++s) {
                const int32_t n = starts[s + 1] - starts[s], L = lens[s];
                if (n < 0) return fail(PA_ERR_RANGE, "%s: query_start decreases at %d", fn, s);
                if (n > max_query_len)
                    return fail(PA_ERR_RANGE, "%s: chunk %d has %d rows > max_query_len %d", fn, s, n, max_query_len);
                if (L < n || L > max_tokens64)
                    return fail(PA_ERR_RANGE, "%s: context_lens[%d] = %d outside [%d, %lld]", fn, s, L, n,
                                (long long)max_tokens64);
                const int32_t used = (L + cache->block_size - 1) / cache->block_size;
                for (int32_t j = 0; j < used; ++j) {
                    const int32_t b = tables[static_cast<size_t>(s) * max_blocks_per_seq + j];
                    if (b < 0 || b >= cache->num_blocks)
                        return fail(PA_ERR_RANGE, "%s: block_tables[%d][%d] = %d out of range", fn, s, j, b);
                }
            }
        }
        pa::PrefillArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.k_cache = static_cast<const uint16_t*>(k_cache);
        a.v_cache = static_cast<const uint16_t*>(v_cache);
        a.block_tables = block_tables;
        a.context_lens = context_lens;
        a.query_start = query_start;
        a.out = static_cast<uint16_t*>(out);
        a.num_blocks = cache->num_blocks;
        a.block_size = cache->block_size;
        a.num_kv_heads = cache->num_kv_heads;
        a.head_major = cache->layout == PA_LAYOUT_HEAD_MAJOR;
        a.head_dim = cache->head_dim;
        a.num_q_heads = num_q_heads;
        a.num_seqs = num_seqs;
        a.num_tokens = num_tokens;
        a.max_blocks_per_seq = max_blocks_per_seq;
        a.max_tokens = static_cast<int32_t>(max_tokens64);
        a.max_query_len = max_query_len;
        a.block_shift = 0;
        while ((1 << a.block_shift) < cache->block_size) ++a.block_shift;
        a.scale_log2 = scale * pa::kLog2e;
        hipError_t err = pa::launch_prefill(a, stream);
        if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
        return ok();
    });
}

}  // extern "C"

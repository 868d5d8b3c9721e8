// Host-side block manager: FIFO free list, per-sequence block tables,
// reference counts, fork and copy-on-write.
//
// Sources (cited by page title):
//  * "Deep dive into the nano-vLLM inference engine architecture:
//    PagedAttention memory management", section "PagedAttention: the
//    operating system's memory wisdom": a free-block list and a per-sequence
//    logical-to-physical table; a request receives its first blocks on
//    arrival and a fresh block whenever its current block fills.
//  * same page, section "Continuous batching and memory management working
//    together": a finished request returns all its blocks to the free list.
//  * "vLLM core architecture: PagedAttention principle, KV Cache management,
//    continuous batching", section 2 ("KV Cache management"): pages of a
//    common prefix are shared; a shared page is copied only when a sharer
//    modifies it; reference counts keep a shared page alive until its last
//    user is done.
//  * same pages (nano-vLLM, sections "Architectural limits" and
//    "Engineering: configuration and monitoring"; vLLM core, section 2):
//    prefix caching -- full blocks of an already cached prompt prefix are
//    shared rather than recomputed -- and its hit rate as a metric.  Blocks are
//    keyed by a chained FNV-1a content hash; a hit also compares the tokens
//    and the parent block, so a hash collision can only cost a miss.
//  * nano-vLLM page, section "Continuous batching and memory management
//    working together": memory compaction against fragmentation, at the cost
//    of moving data.  Compaction here renumbers blocks only; the caller moves
//    the bytes with the returned copy list.
//
// Every operation checks everything it needs before mutating anything, so a
// failed call leaves the state unchanged.

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace {

struct Seq {
    std::vector<int32_t> blocks;
    int32_t n_tokens = 0;
};

// What a block was registered with in the prefix cache.
struct CachedKey {
    uint64_t hash;
    int32_t parent;                 // previous block of the chain, -1 for the first
    std::vector<int32_t> tokens;
};

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_bytes(uint64_t h, uint64_t v, int nbytes) {
    for (int i = 0; i < nbytes; ++i) {
        h ^= (v >> (8 * i)) & 0xFF;
        h *= kFnvPrime;
    }
    return h;
}

// FNV-1a over the parent hash (8 bytes, little-endian) and the token ids
// (4 bytes each, little-endian).
uint64_t chain_hash(uint64_t parent_hash, const int32_t* tokens, int32_t n) {
    uint64_t h = fnv_bytes(kFnvOffset, parent_hash, 8);
    for (int32_t i = 0; i < n; ++i) h = fnv_bytes(h, static_cast<uint32_t>(tokens[i]), 4);
    return h;
}

// Fixed-capacity ring buffer holding the free list.
class FreeList {
public:
    explicit FreeList(int32_t cap) : buf_(static_cast<size_t>(cap)) {}
    int32_t size() const { return count_; }
    bool empty() const { return count_ == 0; }
    int32_t pop_front() {
        int32_t b = buf_[head_];
        head_ = (head_ + 1) % cap();
        --count_;
        return b;
    }
    void push_back(int32_t b) {
        buf_[(head_ + count_) % cap()] = b;
        ++count_;
    }
    int32_t at(int32_t i) const { return buf_[(head_ + i) % cap()]; }

private:
    int32_t cap() const { return static_cast<int32_t>(buf_.size()); }
    std::vector<int32_t> buf_;
    int32_t head_ = 0;
    int32_t count_ = 0;
};

}  // namespace

struct pa_allocator {
    int32_t num_blocks;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    FreeList free_list;
    std::vector<int32_t> refcount;
    std::unordered_map<int64_t, Seq> seqs;
    int64_t cow_copies = 0;
    std::unordered_map<uint64_t, int32_t> prefix_index;    // hash -> live block
    std::unordered_map<int32_t, CachedKey> cached;          // block -> its key
    int64_t prefix_queried = 0;
    int64_t prefix_hits = 0;

    pa_allocator(int32_t nb, int32_t bs, int32_t mb)
        : num_blocks(nb), block_size(bs), max_blocks_per_seq(mb), free_list(nb),
          refcount(static_cast<size_t>(nb), 0) {}

    int32_t slot_of(const Seq& s, int32_t pos) const {
        return s.blocks[pos / block_size] * block_size + pos % block_size;
    }
};


#ifdef PA_ALLOC_CHECK_INVARIANTS
#include <cstdio>
#include <cstdlib>

namespace {

[[noreturn]] void invariant_broken(const char* what, long long a, long long b) {
    std::fprintf(stderr, "pa_allocator invariant broken: %s (%lld, %lld)\n", what, a, b);
    std::abort();
}

// Debug builds check the whole state after every mutating call, failed calls
// included (those must leave it unchanged, so it must still be consistent):
//  * each block's reference count equals the number of table entries naming it;
//  * the free list holds no block twice, only blocks with count 0, and every
//    block with count 0 (free and used partition the pool);
//  * a sequence holds ceil(tokens / block_size) blocks, at most the cap, all
//    in range;
//  * a cached prefix block is in use and indexed under its own key.
void check_invariants(const pa_allocator* a) {
    if (!a) return;
    const int32_t nb = a->num_blocks;
    std::vector<int64_t> refs(static_cast<size_t>(nb), 0);
    for (const auto& kv : a->seqs) {
        const Seq& s = kv.second;
        const int64_t need = (static_cast<int64_t>(s.n_tokens) + a->block_size - 1) / a->block_size;
        if (static_cast<int64_t>(s.blocks.size()) != need)
            invariant_broken("sequence blocks != ceil(tokens / block_size)", s.blocks.size(), need);
        if (static_cast<int64_t>(s.blocks.size()) > a->max_blocks_per_seq)
            invariant_broken("sequence longer than max_blocks_per_seq", s.blocks.size(), a->max_blocks_per_seq);
        for (int32_t b : s.blocks) {
            if (b < 0 || b >= nb) invariant_broken("table entry out of range", b, nb);
            ++refs[static_cast<size_t>(b)];
        }
    }
    int64_t used = 0;
    for (int32_t b = 0; b < nb; ++b) {
        if (refs[static_cast<size_t>(b)] != a->refcount[static_cast<size_t>(b)])
            invariant_broken("reference count != table references", refs[static_cast<size_t>(b)],
                             a->refcount[static_cast<size_t>(b)]);
        if (a->refcount[static_cast<size_t>(b)] > 0) ++used;
    }
    std::vector<char> on_list(static_cast<size_t>(nb), 0);
    for (int32_t i = 0; i < a->free_list.size(); ++i) {
        const int32_t b = a->free_list.at(i);
        if (b < 0 || b >= nb) invariant_broken("free-list entry out of range", b, nb);
        if (on_list[static_cast<size_t>(b)]) invariant_broken("block twice on the free list", b, i);
        on_list[static_cast<size_t>(b)] = 1;
        if (a->refcount[static_cast<size_t>(b)] != 0)
            invariant_broken("free block with references", b, a->refcount[static_cast<size_t>(b)]);
    }
    if (used + a->free_list.size() != nb)
        invariant_broken("free and used blocks do not partition the pool", used + a->free_list.size(), nb);
    for (const auto& kv : a->cached) {
        if (kv.first < 0 || kv.first >= nb || a->refcount[static_cast<size_t>(kv.first)] <= 0)
            invariant_broken("cached prefix block not in use", kv.first, 0);
        const auto it = a->prefix_index.find(kv.second.hash);
        if (it == a->prefix_index.end() || it->second != kv.first)
            invariant_broken("cached block not indexed under its key", kv.first, 0);
    }
    for (const auto& kv : a->prefix_index)
        if (a->cached.find(kv.second) == a->cached.end())
            invariant_broken("prefix index names an uncached block", kv.second, 0);
}

}  // namespace
#define PA_ALLOC_CHECKED(a, call)              \
    do {                                       \
        const pa_status pa_st_ = (call);       \
        check_invariants(a);                   \
        return pa_st_;                         \
    } while (0)
#else
#define PA_ALLOC_CHECKED(a, call) return (call)
#endif

using pa::fail;
using pa::ok;

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          int32_t max_blocks_per_seq,
                          const int32_t* initial_free_order, pa_allocator** out) {
    PA_ALLOC_CHECKED(out ? *out : nullptr, pa::guard("pa_alloc_create", [&]() -> pa_status {
        if (!out) return fail(PA_ERR_NULL, "pa_alloc_create: out is NULL");
        *out = nullptr;
        if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
            return fail(PA_ERR_SHAPE, "pa_alloc_create: sizes must be positive");
        if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
            return fail(PA_ERR_RANGE, "pa_alloc_create: num_blocks*block_size overflows int32 slots");
        pa_allocator* a = new (std::nothrow) pa_allocator(num_blocks, block_size, max_blocks_per_seq);
        if (!a) return fail(PA_ERR_RANGE, "pa_alloc_create: out of host memory");
        if (initial_free_order) {
            std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
            for (int32_t i = 0; i < num_blocks; ++i) {
                int32_t b = initial_free_order[i];
                if (b < 0 || b >= num_blocks || seen[b]) {
                    delete a;
                    return fail(PA_ERR_RANGE, "pa_alloc_create: initial order is not a permutation (entry %d)", i);
                }
                seen[b] = 1;
            }
            for (int32_t i = 0; i < num_blocks; ++i) a->free_list.push_back(initial_free_order[i]);
        } else {
            for (int32_t i = 0; i < num_blocks; ++i) a->free_list.push_back(i);
        }
        *out = a;
        return ok();
    }));
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq, int32_t n_tokens, int32_t* slots_out) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_add_seq", [&]() -> pa_status {
        if (!a) return fail(PA_ERR_NULL, "pa_alloc_add_seq: allocator is NULL");
        if (a->seqs.count(seq)) return fail(PA_ERR_SEQ_EXISTS, "pa_alloc_add_seq: sequence %lld exists", (long long)seq);
        if (n_tokens < 0) return fail(PA_ERR_RANGE, "pa_alloc_add_seq: negative token count");
        int32_t need = (n_tokens + a->block_size - 1) / a->block_size;
        if (need > a->max_blocks_per_seq)
            return fail(PA_ERR_SEQ_LIMIT, "pa_alloc_add_seq: %d blocks exceed the per-sequence limit %d", need, a->max_blocks_per_seq);
        if (need > a->free_list.size())
            return fail(PA_ERR_OUT_OF_BLOCKS, "pa_alloc_add_seq: need %d blocks, %d free", need, a->free_list.size());
        Seq s;
        s.blocks.reserve(static_cast<size_t>(need));
        for (int32_t i = 0; i < need; ++i) {
            int32_t b = a->free_list.pop_front();
            a->refcount[b] = 1;
            s.blocks.push_back(b);
        }
        s.n_tokens = n_tokens;
        if (slots_out)
            for (int32_t p = 0; p < n_tokens; ++p) slots_out[p] = a->slot_of(s, p);
        a->seqs.emplace(seq, std::move(s));
        return ok();
    }));
}

pa_status pa_alloc_fork(pa_allocator* a, int64_t parent, int64_t child) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_fork", [&]() -> pa_status {
        if (!a) return fail(PA_ERR_NULL, "pa_alloc_fork: allocator is NULL");
        auto it = a->seqs.find(parent);
        if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_alloc_fork: unknown parent %lld", (long long)parent);
        if (a->seqs.count(child)) return fail(PA_ERR_SEQ_EXISTS, "pa_alloc_fork: child %lld exists", (long long)child);
        // Insert first (the only step that can throw), then count the shares.
        Seq copy = it->second;
        const auto ins = a->seqs.emplace(child, std::move(copy));
        for (int32_t b : ins.first->second.blocks) ++a->refcount[b];
        return ok();
    }));
}

static pa_status append_one(pa_allocator* a, int64_t seq, int32_t* slot, int32_t* src, int32_t* dst) {
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_alloc_append_slot: unknown sequence %lld", (long long)seq);
    Seq& s = it->second;
    const int32_t pos = s.n_tokens;
    int32_t cs = -1, cd = -1;
    if (pos % a->block_size == 0) {
        if (static_cast<int32_t>(s.blocks.size()) >= a->max_blocks_per_seq)
            return fail(PA_ERR_SEQ_LIMIT, "pa_alloc_append_slot: sequence %lld at its block limit", (long long)seq);
        if (a->free_list.empty()) return fail(PA_ERR_OUT_OF_BLOCKS, "pa_alloc_append_slot: no free block");
        int32_t b = a->free_list.pop_front();
        a->refcount[b] = 1;
        s.blocks.push_back(b);
    } else {
        int32_t last = s.blocks.back();
        if (a->refcount[last] > 1) {
            if (a->free_list.empty()) return fail(PA_ERR_OUT_OF_BLOCKS, "pa_alloc_append_slot: no free block for copy-on-write");
            int32_t fresh = a->free_list.pop_front();
            --a->refcount[last];
            a->refcount[fresh] = 1;
            s.blocks.back() = fresh;
            cs = last;
            cd = fresh;
            ++a->cow_copies;
        }
    }
    s.n_tokens = pos + 1;
    *slot = a->slot_of(s, pos);
    *src = cs;
    *dst = cd;
    return PA_OK;
}

pa_status pa_alloc_append_slot(pa_allocator* a, int64_t seq, int32_t* slot, int32_t* cow_src, int32_t* cow_dst) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_append_slot", [&]() -> pa_status {
        if (!a || !slot || !cow_src || !cow_dst) return fail(PA_ERR_NULL, "pa_alloc_append_slot: NULL argument");
        pa_status st = append_one(a, seq, slot, cow_src, cow_dst);
        return st == PA_OK ? ok() : st;
    }));
}

pa_status pa_alloc_append_batch(pa_allocator* a, const int64_t* seqs, int32_t n, int32_t* slots_out,
                                int32_t* cow_pairs_out, int32_t* num_cow, int32_t* num_done) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_append_batch", [&]() -> pa_status {
        if (!a || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)) || !num_cow || !num_done)
            return fail(PA_ERR_NULL, "pa_alloc_append_batch: NULL argument");
        if (n < 0) return fail(PA_ERR_SHAPE, "pa_alloc_append_batch: negative count");
        *num_cow = 0;
        *num_done = 0;
        for (int32_t i = 0; i < n; ++i) {
            int32_t src, dst;
            pa_status st = append_one(a, seqs[i], &slots_out[i], &src, &dst);
            if (st != PA_OK) return st;
            if (src >= 0) {
                cow_pairs_out[2 * *num_cow] = src;
                cow_pairs_out[2 * *num_cow + 1] = dst;
                ++*num_cow;
            }
            *num_done = i + 1;
        }
        return ok();
    }));
}

pa_status pa_alloc_free_seq(pa_allocator* a, int64_t seq) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_free_seq", [&]() -> pa_status {
        if (!a) return fail(PA_ERR_NULL, "pa_alloc_free_seq: allocator is NULL");
        auto it = a->seqs.find(seq);
        if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_alloc_free_seq: unknown sequence %lld", (long long)seq);
        for (int32_t b : it->second.blocks)
            if (--a->refcount[b] == 0) {
                a->free_list.push_back(b);
                auto c = a->cached.find(b);
                if (c != a->cached.end()) {
                    auto ix = a->prefix_index.find(c->second.hash);
                    if (ix != a->prefix_index.end() && ix->second == b) a->prefix_index.erase(ix);
                    a->cached.erase(c);
                }
            }
        a->seqs.erase(it);
        return ok();
    }));
}

pa_status pa_alloc_add_seq_tokens(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                  int32_t n_tokens, int32_t* slots_out, int32_t* n_cached) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_add_seq_tokens", [&]() -> pa_status {
        if (!a || !n_cached || (n_tokens > 0 && !tokens))
            return fail(PA_ERR_NULL, "pa_alloc_add_seq_tokens: NULL argument");
        if (a->seqs.count(seq)) return fail(PA_ERR_SEQ_EXISTS, "pa_alloc_add_seq_tokens: sequence %lld exists", (long long)seq);
        if (n_tokens < 0) return fail(PA_ERR_RANGE, "pa_alloc_add_seq_tokens: negative token count");
        const int32_t bs = a->block_size;
        const int32_t need = (n_tokens + bs - 1) / bs, full = n_tokens / bs;
        if (need > a->max_blocks_per_seq)
            return fail(PA_ERR_SEQ_LIMIT, "pa_alloc_add_seq_tokens: %d blocks exceed the per-sequence limit %d", need, a->max_blocks_per_seq);
        // Hash every full block; the leading run of matching live blocks is shared.
        std::vector<uint64_t> hashes(static_cast<size_t>(full));
        std::vector<int32_t> hits;
        uint64_t h = 0;
        int32_t parent = -1;
        for (int32_t j = 0; j < full; ++j) {
            const int32_t* tk = tokens + static_cast<size_t>(j) * bs;
            h = chain_hash(h, tk, bs);
            hashes[j] = h;
            if (static_cast<int32_t>(hits.size()) != j) continue;
            auto ix = a->prefix_index.find(h);
            if (ix == a->prefix_index.end()) continue;
            const CachedKey& key = a->cached.at(ix->second);
            if (key.parent != parent || !std::equal(key.tokens.begin(), key.tokens.end(), tk)) continue;
            hits.push_back(ix->second);
            parent = ix->second;
        }
        const int32_t n_hit = static_cast<int32_t>(hits.size());
        if (need - n_hit > a->free_list.size())
            return fail(PA_ERR_OUT_OF_BLOCKS, "pa_alloc_add_seq_tokens: need %d blocks, %d free", need - n_hit, a->free_list.size());
        Seq s;
        s.blocks = hits;
        for (int32_t b : hits) ++a->refcount[b];
        parent = n_hit ? hits.back() : -1;
        for (int32_t j = n_hit; j < need; ++j) {
            int32_t b = a->free_list.pop_front();
            a->refcount[b] = 1;
            s.blocks.push_back(b);
            if (j < full) {
                if (!a->prefix_index.count(hashes[j])) {
                    const int32_t* tk = tokens + static_cast<size_t>(j) * bs;
                    a->prefix_index.emplace(hashes[j], b);
                    a->cached[b] = CachedKey{hashes[j], parent, std::vector<int32_t>(tk, tk + bs)};
                }
                parent = b;
            }
        }
        s.n_tokens = n_tokens;
        if (slots_out)
            for (int32_t p = 0; p < n_tokens; ++p) slots_out[p] = a->slot_of(s, p);
        a->seqs.emplace(seq, std::move(s));
        a->prefix_queried += n_tokens;
        a->prefix_hits += static_cast<int64_t>(n_hit) * bs;
        *n_cached = n_hit * bs;
        return ok();
    }));
}

pa_status pa_alloc_compact(pa_allocator* a, int32_t* pairs_out, int32_t max_pairs, int32_t* n_pairs) {
    PA_ALLOC_CHECKED(a, pa::guard("pa_alloc_compact", [&]() -> pa_status {
        if (!a || !n_pairs) return fail(PA_ERR_NULL, "pa_alloc_compact: NULL argument");
        const int32_t nb = a->num_blocks;
        int32_t used = 0;
        for (int32_t b = 0; b < nb; ++b) used += a->refcount[b] > 0;
        // Used blocks at or above `used` pair, in increasing order, with the free
        // blocks below it; the two lists have equal length.
        std::vector<int32_t> remap(static_cast<size_t>(nb));
        for (int32_t b = 0; b < nb; ++b) remap[b] = b;
        int32_t moves = 0, hole = 0;
        for (int32_t b = used; b < nb; ++b) {
            if (a->refcount[b] == 0) continue;
            while (a->refcount[hole] != 0) ++hole;
            remap[b] = hole++;
            ++moves;
        }
        *n_pairs = moves;
        if (moves > max_pairs)
            return fail(PA_ERR_RANGE, "pa_alloc_compact: %d moves, room for %d", moves, max_pairs);
        if (moves > 0 && !pairs_out) return fail(PA_ERR_NULL, "pa_alloc_compact: pairs_out is NULL");
        int32_t k = 0;
        for (int32_t b = used; b < nb; ++b) {
            if (remap[b] == b) continue;
            pairs_out[2 * k] = b;
            pairs_out[2 * k + 1] = remap[b];
            ++k;
            a->refcount[remap[b]] = a->refcount[b];
            a->refcount[b] = 0;
        }
        if (moves > 0) {
            for (auto& kv : a->seqs)
                for (int32_t& b : kv.second.blocks) b = remap[b];
            std::unordered_map<int32_t, CachedKey> cached;
            cached.reserve(a->cached.size());
            for (auto& kv : a->cached) {
                CachedKey key = std::move(kv.second);
                if (key.parent >= 0) key.parent = remap[key.parent];
                cached.emplace(remap[kv.first], std::move(key));
            }
            a->cached = std::move(cached);
            for (auto& kv : a->prefix_index) kv.second = remap[kv.second];
        }
        a->free_list = FreeList(nb);       // rebuilt in increasing order even with no moves
        for (int32_t b = used; b < nb; ++b) a->free_list.push_back(b);
        return ok();
    }));
}

pa_status pa_alloc_prefix_stats(const pa_allocator* a, int64_t* queried_tokens, int64_t* hit_tokens,
                                int32_t* cached_blocks) {
    return pa::guard("pa_alloc_prefix_stats", [&]() -> pa_status {
        if (!a || !queried_tokens || !hit_tokens || !cached_blocks)
            return fail(PA_ERR_NULL, "pa_alloc_prefix_stats: NULL argument");
        *queried_tokens = a->prefix_queried;
        *hit_tokens = a->prefix_hits;
        *cached_blocks = static_cast<int32_t>(a->prefix_index.size());
        return ok();
    });
}

pa_status pa_alloc_export(const pa_allocator* a, const int64_t* seqs, int32_t n, int32_t row_stride,
                          int32_t* block_tables_out, int32_t* context_lens_out) {
    return pa::guard("pa_alloc_export", [&]() -> pa_status {
        if (!a || (n > 0 && (!seqs || !block_tables_out))) return fail(PA_ERR_NULL, "pa_alloc_export: NULL argument");
        if (n < 0 || row_stride <= 0) return fail(PA_ERR_SHAPE, "pa_alloc_export: bad sizes");
        for (int32_t i = 0; i < n; ++i) {          // check everything first
            auto it = a->seqs.find(seqs[i]);
            if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_alloc_export: unknown sequence %lld", (long long)seqs[i]);
            if (static_cast<int32_t>(it->second.blocks.size()) > row_stride)
                return fail(PA_ERR_SHAPE, "pa_alloc_export: sequence %lld has %zu blocks > row stride %d",
                            (long long)seqs[i], it->second.blocks.size(), row_stride);
        }
        for (int32_t i = 0; i < n; ++i) {
            const Seq& s = a->seqs.find(seqs[i])->second;
            int32_t* row = block_tables_out + static_cast<size_t>(i) * row_stride;
            std::copy(s.blocks.begin(), s.blocks.end(), row);
            std::fill(row + s.blocks.size(), row + row_stride, -1);
            if (context_lens_out) context_lens_out[i] = s.n_tokens;
        }
        return ok();
    });
}

pa_status pa_alloc_stats(const pa_allocator* a, pa_alloc_stats_t* out) {
    return pa::guard("pa_alloc_stats", [&]() -> pa_status {
        if (!a || !out) return fail(PA_ERR_NULL, "pa_alloc_stats: NULL argument");
        std::vector<int32_t> fill(static_cast<size_t>(a->num_blocks), 0);
        int64_t logical = 0;
        for (const auto& kv : a->seqs) {
            const Seq& s = kv.second;
            logical += s.n_tokens;
            for (size_t j = 0; j < s.blocks.size(); ++j) {
                int64_t in_block = static_cast<int64_t>(s.n_tokens) - static_cast<int64_t>(j) * a->block_size;
                int32_t f = static_cast<int32_t>(std::min<int64_t>(a->block_size, in_block));
                fill[s.blocks[j]] = std::max(fill[s.blocks[j]], f);
            }
        }
        int32_t used = 0, shared = 0;
        int64_t filled = 0;
        for (int32_t b = 0; b < a->num_blocks; ++b) {
            if (a->refcount[b] > 0) ++used;
            if (a->refcount[b] > 1) ++shared;
            filled += fill[b];
        }
        out->num_blocks = a->num_blocks;
        out->free_blocks = a->free_list.size();
        out->used_blocks = used;
        out->shared_blocks = shared;
        out->cow_copies = a->cow_copies;
        out->live_seqs = static_cast<int64_t>(a->seqs.size());
        out->logical_tokens = logical;
        out->stored_tokens = filled;
        out->utilisation = static_cast<double>(used) / a->num_blocks;
        const double slots = static_cast<double>(used) * a->block_size;
        out->internal_fragmentation = used ? (slots - static_cast<double>(filled)) / slots : 0.0;
        return ok();
    });
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->refcount[block];
}

int32_t pa_alloc_num_free(const pa_allocator* a) { return a ? a->free_list.size() : 0; }

int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap) {
    if (!a || !out || cap <= 0) return 0;
    int32_t n = std::min(cap, a->free_list.size());
    for (int32_t i = 0; i < n; ++i) out[i] = a->free_list.at(i);
    return n;
}

pa_status pa_alloc_seq_info(const pa_allocator* a, int64_t seq, int32_t* n_tokens, int32_t* n_blocks) {
    return pa::guard("pa_alloc_seq_info", [&]() -> pa_status {
        if (!a || !n_tokens || !n_blocks) return fail(PA_ERR_NULL, "pa_alloc_seq_info: NULL argument");
        auto it = a->seqs.find(seq);
        if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_alloc_seq_info: unknown sequence %lld", (long long)seq);
        *n_tokens = it->second.n_tokens;
        *n_blocks = static_cast<int32_t>(it->second.blocks.size());
        return ok();
    });
}

}  // extern "C"

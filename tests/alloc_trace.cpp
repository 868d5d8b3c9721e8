// Seeded random traces over the block manager's whole C ABI, for a build with
// AddressSanitizer, UndefinedBehaviorSanitizer and the allocator's own
// invariant checker (PA_ALLOC_CHECK_INVARIANTS).  Built and run by
// tests/test_allocator_sanitized.py; a sanitizer report, a broken invariant
// or a failed content check ends the process with a nonzero status.
//
// Besides the allocator's internal invariants, the driver keeps a shadow
// cache: every slot handed out receives the id of the token it stores,
// copy-on-write and compaction copies move whole blocks, and after every
// operation each live sequence's tokens, gathered through its exported block
// table, must be that sequence's token list.  This is the reference-count
// bug class of shared prefixes: a block released while another sequence
// still reads it would be handed out again and overwritten.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <map>
#include <random>
#include <vector>

#include "pa.h"

namespace pa {
char* error_text() {
    static thread_local char text[512] = {0};
    return text;
}
}  // namespace pa

namespace {

[[noreturn]] void die(const char* what, long long a = 0, long long b = 0) {
    std::fprintf(stderr, "alloc_trace: %s (%lld, %lld): %s\n", what, a, b, pa::error_text());
    std::exit(2);
}

struct Trace {
    int32_t nb, bs, mb;
    std::mt19937_64 rng;
    pa_allocator* a = nullptr;
    std::vector<int32_t> shadow;                   // slot -> token id stored there
    std::map<int64_t, std::vector<int32_t>> live;  // sequence -> its token ids
    std::vector<std::vector<int32_t>> prefixes;    // shared prompt prefixes
    int64_t next_id = 1;
    int32_t next_token = 1;
    long ops = 0, failures = 0, cows = 0, hits = 0, moves = 0;

    Trace(int32_t nb_, int32_t bs_, int32_t mb_, uint64_t seed) : nb(nb_), bs(bs_), mb(mb_), rng(seed) {
        std::vector<int32_t> order(static_cast<size_t>(nb));
        for (int32_t i = 0; i < nb; ++i) order[static_cast<size_t>(i)] = i;
        std::shuffle(order.begin(), order.end(), rng);
        if (pa_alloc_create(nb, bs, mb, order.data(), &a) != PA_OK) die("create");
        shadow.assign(static_cast<size_t>(nb) * bs, -1);
        for (int k = 0; k < 4; ++k) {
            std::vector<int32_t> p(static_cast<size_t>(bs) * (1 + rng() % 4) + rng() % bs);
            for (auto& t : p) t = next_token++;
            prefixes.push_back(p);
        }
    }
    ~Trace() { pa_alloc_destroy(a); }

    int pick(int n) { return static_cast<int>(rng() % static_cast<uint64_t>(n)); }
    int64_t any_live() {
        auto it = live.begin();
        std::advance(it, pick(static_cast<int>(live.size())));
        return it->first;
    }

    void store(const int32_t* slots, const int32_t* toks, int32_t n) {
        for (int32_t i = 0; i < n; ++i) {
            if (slots[i] < 0 || slots[i] >= nb * bs) die("slot out of range", slots[i]);
            shadow[static_cast<size_t>(slots[i])] = toks[i];
        }
    }
    void copy_block(int32_t src, int32_t dst) {
        if (src < 0 || src >= nb || dst < 0 || dst >= nb) die("copy pair out of range", src, dst);
        std::memcpy(&shadow[static_cast<size_t>(dst) * bs], &shadow[static_cast<size_t>(src) * bs],
                    sizeof(int32_t) * static_cast<size_t>(bs));
    }

    // Every live sequence's tokens, read back through its exported table.
    void verify() {
        if (live.empty()) return;
        std::vector<int64_t> ids;
        for (auto& kv : live) ids.push_back(kv.first);
        const int32_t n = static_cast<int32_t>(ids.size());
        std::vector<int32_t> tables(static_cast<size_t>(n) * mb), lens(static_cast<size_t>(n));
        if (pa_alloc_export(a, ids.data(), n, mb, tables.data(), lens.data()) != PA_OK) die("export");
        for (int32_t i = 0; i < n; ++i) {
            const auto& toks = live[ids[static_cast<size_t>(i)]];
            if (lens[static_cast<size_t>(i)] != static_cast<int32_t>(toks.size()))
                die("length differs", lens[static_cast<size_t>(i)], static_cast<long long>(toks.size()));
            for (int32_t p = 0; p < lens[static_cast<size_t>(i)]; ++p) {
                const int32_t blk = tables[static_cast<size_t>(i) * mb + p / bs];
                if (blk < 0 || blk >= nb) die("table entry out of range", blk);
                if (shadow[static_cast<size_t>(blk) * bs + p % bs] != toks[static_cast<size_t>(p)])
                    die("a sequence reads another token", ids[static_cast<size_t>(i)], p);
            }
        }
        pa_alloc_stats_t st;
        if (pa_alloc_stats(a, &st) != PA_OK) die("stats");
        if (st.live_seqs != static_cast<int64_t>(live.size())) die("live count", st.live_seqs, live.size());
        if (st.free_blocks + st.used_blocks != nb) die("free + used", st.free_blocks, st.used_blocks);
        if (pa_alloc_num_free(a) != st.free_blocks) die("num_free");
        int64_t q = 0, h = 0;
        int32_t c = 0;
        if (pa_alloc_prefix_stats(a, &q, &h, &c) != PA_OK || h > q) die("prefix stats", q, h);
    }

    void step() {
        ++ops;
        int op = pick(100);
        if (live.size() > 48 && op < 44) op = 80;                  // keep the batch bounded: free
        if (op < 18 || live.empty()) {                               // add by length
            const int32_t n = pick(3 * bs * mb / 2 + 1);
            std::vector<int32_t> slots(static_cast<size_t>(n) + 1), toks(static_cast<size_t>(n));
            for (auto& t : toks) t = next_token++;
            const int64_t id = next_id++;
            const pa_status st = pa_alloc_add_seq(a, id, n, slots.data());
            if (st == PA_OK) {
                store(slots.data(), toks.data(), n);
                live[id] = toks;
            } else if (st == PA_ERR_OUT_OF_BLOCKS || st == PA_ERR_SEQ_LIMIT) {
                ++failures;
            } else {
                die("add_seq status", st);
            }
        } else if (op < 34) {                                         // add by tokens (prefix cache)
            std::vector<int32_t> toks = prefixes[static_cast<size_t>(pick(4))];
            const int32_t extra = pick(2 * bs + 1);
            for (int32_t i = 0; i < extra; ++i) toks.push_back(next_token++);
            if (pick(4) == 0 && toks.size() > 1) toks.resize(static_cast<size_t>(pick(static_cast<int>(toks.size()))));
            const int32_t n = static_cast<int32_t>(toks.size());
            std::vector<int32_t> slots(static_cast<size_t>(n) + 1);
            int32_t n_cached = -1;
            const int64_t id = next_id++;
            const pa_status st = pa_alloc_add_seq_tokens(a, id, n ? toks.data() : nullptr, n, slots.data(),
                                                         &n_cached);
            if (st == PA_OK) {
                if (n_cached < 0 || n_cached > n || n_cached % bs) die("n_cached", n_cached, n);
                for (int32_t i = 0; i < n_cached; ++i)
                    if (shadow[static_cast<size_t>(slots[static_cast<size_t>(i)])] != toks[static_cast<size_t>(i)])
                        die("cached slot does not hold the token", i);
                store(slots.data() + n_cached, toks.data() + n_cached, n - n_cached);
                hits += n_cached;
                live[id] = toks;
            } else if (st == PA_ERR_OUT_OF_BLOCKS || st == PA_ERR_SEQ_LIMIT) {
                ++failures;
            } else {
                die("add_seq_tokens status", st);
            }
        } else if (op < 44) {                                         // fork
            const int64_t parent = any_live(), child = next_id++;
            const pa_status st = pa_alloc_fork(a, parent, child);
            if (st != PA_OK) die("fork", st);
            live[child] = live[parent];
        } else if (op < 62) {                                         // append one token
            const int64_t id = any_live();
            int32_t slot = -1, src = -1, dst = -1;
            const pa_status st = pa_alloc_append_slot(a, id, &slot, &src, &dst);
            if (st == PA_OK) {
                if (src >= 0) {
                    copy_block(src, dst);
                    ++cows;
                }
                const int32_t t = next_token++;
                store(&slot, &t, 1);
                live[id].push_back(t);
            } else if (st == PA_ERR_OUT_OF_BLOCKS || st == PA_ERR_SEQ_LIMIT) {
                ++failures;
            } else {
                die("append_slot status", st);
            }
        } else if (op < 70) {                                         // append a batch
            std::vector<int64_t> ids;
            for (auto& kv : live)
                if (pick(2)) ids.push_back(kv.first);
            const int32_t n = static_cast<int32_t>(ids.size());
            std::vector<int32_t> slots(static_cast<size_t>(n) + 1), pairs(2 * static_cast<size_t>(n) + 2);
            int32_t n_cow = -1, done = -1;
            const pa_status st = pa_alloc_append_batch(a, n ? ids.data() : nullptr, n, slots.data(),
                                                       pairs.data(), &n_cow, &done);
            if (st != PA_OK && st != PA_ERR_OUT_OF_BLOCKS && st != PA_ERR_SEQ_LIMIT)
                die("append_batch status", st);
            if (st != PA_OK) ++failures;
            if (done < 0 || done > n || n_cow < 0) die("append_batch counts", done, n_cow);
            for (int32_t i = 0; i < n_cow; ++i) {
                copy_block(pairs[2 * static_cast<size_t>(i)], pairs[2 * static_cast<size_t>(i) + 1]);
                ++cows;
            }
            for (int32_t i = 0; i < done; ++i) {
                const int32_t t = next_token++;
                store(&slots[static_cast<size_t>(i)], &t, 1);
                live[ids[static_cast<size_t>(i)]].push_back(t);
            }
        } else if (op < 90) {                                         // free
            const int64_t id = any_live();
            if (pa_alloc_free_seq(a, id) != PA_OK) die("free");
            live.erase(id);
        } else if (op < 94) {                                         // compact
            std::vector<int32_t> pairs(2 * static_cast<size_t>(nb) + 2);
            int32_t n_pairs = -1;
            const int32_t cap = pick(3) == 0 ? pick(4) : nb;
            const pa_status st = pa_alloc_compact(a, pairs.data(), cap, &n_pairs);
            if (st == PA_OK) {
                for (int32_t i = 0; i < n_pairs; ++i)
                    copy_block(pairs[2 * static_cast<size_t>(i)], pairs[2 * static_cast<size_t>(i) + 1]);
                moves += n_pairs;
            } else if (st == PA_ERR_RANGE) {
                if (n_pairs <= cap) die("compact refused a plan that fits", n_pairs, cap);
                ++failures;
            } else {
                die("compact status", st);
            }
        } else {                                                      // error paths
            int32_t slot, src, dst;
            if (pa_alloc_append_slot(a, -5 - pick(100), &slot, &src, &dst) != PA_ERR_UNKNOWN_SEQ)
                die("append to an unknown sequence");
            if (pa_alloc_free_seq(a, -7) != PA_ERR_UNKNOWN_SEQ) die("free an unknown sequence");
            if (pa_alloc_fork(a, any_live(), any_live()) != PA_ERR_SEQ_EXISTS) die("fork onto a live id");
            if (pa_alloc_add_seq(a, any_live(), 1, nullptr) != PA_ERR_SEQ_EXISTS) die("add a live id");
            if (pa_alloc_add_seq(a, next_id++, (mb + 1) * bs, nullptr) != PA_ERR_SEQ_LIMIT &&
                pa_alloc_add_seq(a, next_id - 1, (mb + 1) * bs, nullptr) != PA_ERR_OUT_OF_BLOCKS)
                die("add past the table cap");
            if (pa_alloc_refcount(a, -1) != -1 || pa_alloc_refcount(a, nb) != -1) die("refcount range");
            failures += 5;
        }
        verify();
    }
};

}  // namespace

int main(int argc, char** argv) {
    const long steps = argc > 1 ? std::atol(argv[1]) : 4000;
    const int32_t shapes[][3] = {{64, 16, 8}, {96, 8, 16}, {40, 4, 32}, {256, 16, 32}, {33, 1, 64}};
    uint64_t seed = 12345;
    for (const auto& sh : shapes) {
        for (int rep = 0; rep < 3; ++rep) {
            Trace t(sh[0], sh[1], sh[2], seed++);
            for (long i = 0; i < steps; ++i) t.step();
            std::printf("pool %d block %d cap %d seed %llu: %ld ops, %ld refused, %ld copy-on-write, "
                        "%ld cached tokens, %ld compaction moves, %zu live\n",
                        sh[0], sh[1], sh[2], static_cast<unsigned long long>(seed - 1), t.ops, t.failures,
                        t.cows, t.hits, t.moves, t.live.size());
        }
    }
    std::printf("ok\n");
    return 0;
}

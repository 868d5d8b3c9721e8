// Paged single-query attention (decode) for CDNA4 / gfx950.
//
// Sources (cited by page title):
//  * "vLLM core architecture: PagedAttention principle, KV Cache management,
//    continuous batching", section 1 ("PagedAttention: inspiration from
//    virtual memory"): a sequence's cache is logically contiguous but stored
//    in scattered fixed-size pages, reached through a per-sequence page table.
//  * "Deep dive into the nano-vLLM inference engine architecture:
//    PagedAttention memory management", section "PagedAttention: the
//    operating system's memory wisdom": blocks of 16 tokens and the
//    logical-to-physical block table.
//  * "Deep analysis of nano-vLLM's paged KV cache and memory optimisation
//    architecture", section "Engineering: configuration and monitoring":
//    decode attention reads the paged cache directly (plain attention being
//    the fallback); section 3 of the vLLM page ties decode speed to memory
//    bandwidth.
//
// What is computed, per sequence s and query head h (KV head g = h / G):
//   out[s][h] = sum_p softmax_p(scale * q[s][h] . K[s,p,g]) V[s,p,g]
// with K/V row p found in physical block table[s][p / BS], row p % BS.
//
// Design (HBM-bound streaming).  This vector kernel (decode_split_kernel)
// serves 1 or 2 query heads per KV head; 3 to 8 query heads per KV head run
// the same partition on the matrix cores (decode_mfma_kernel, below), and
// larger groups are cut into virtual KV heads of at most 8:
//  * Short contexts (a bound of at most 512 tokens, at most 64 sequences):
//    workgroup w takes (sequence, KV head) pair w whole and writes its fp16
//    rows; no merge kernel runs.  One launch instead of two where launch
//    latency, not bandwidth, sets the time.
//  * Balanced split.  The work is the list of 16-token chunks of every
//    (sequence, KV head) pair, in sequence-major order; the grid is W
//    workgroups (by default as many as the device holds at once) and
//    workgroup w takes the contiguous range [w*U/W, (w+1)*U/W) of the U
//    chunks.  Every workgroup streams the same number of bytes, whatever the
//    mix of context lengths, and the whole grid starts in one round.  A
//    range crosses pair boundaries: each piece of it (a "segment") is one
//    pair's chunks [c0, c1).
//  * A segment that covers a whole pair is normalised and written to fp16
//    directly.  Otherwise the workgroup writes fp32 (m, l, o) partials to
//    slot w + pair of the workspace (distinct for every segment: along the
//    chunk order, either w or pair grows at each segment start; in the
//    matrix-core kernel's head-group order, slot 4 * (w + group) + head in
//    group), and the merge kernel combines the slots of workgroups
//    first(pair) .. last(pair).
//  * Within a segment, chunks are dealt round-robin to the 4 wave64s of the
//    workgroup.  A K (or V) row of D fp16 is D/8 lanes x 16 bytes, so one
//    buffer_load_dwordx4 per lane covers 64/(D/8) whole rows (1 KiB per wave
//    instruction, fully coalesced).  The G query heads sharing the KV head
//    live in registers, so every K/V byte is fetched from HBM once.
//  * Block numbers: a wave loads the table entries of up to 64 of its chunks
//    into one VGPR (lane k <- chunk k) and reads them back with v_readlane
//    into SGPRs, so each load is a scalar buffer base (the physical block)
//    plus a per-lane constant offset.  No LDS round trip, no barrier.
//  * Software pipelining: the next chunk's K and V loads are issued before
//    the current chunk is consumed (two register buffers).  The loads carry
//    the non-temporal hint: every byte is read once per call.  A pair's
//    ragged last chunk rides the same pipeline where it has one block (blocks
//    of 16 tokens or more): that block's buffer range ends at the context's
//    last token, so the rows past it read as zeros and are never fetched.
//  * Both cache layouts (slot-major [block][token][head][dim] and head-major
//    [block][head][token][dim]) run the same code: only the stride between a
//    head's consecutive token rows and the head's offset in a block differ.
//  * Each 16-lane row group keeps its own online-softmax stream (running max
//    m, sum l, fp32 accumulator of its 8 columns), so the per-chunk work
//    needs only an in-row DPP butterfly for the q.k dot product; the row
//    groups, then the 4 waves (through LDS), are merged once per segment.
//  * Exponentials are exp2 with scale*log2(e) folded into the scores.
//  * The split depends only on the context lengths and W, and every
//    reduction has a fixed order, so results are bitwise reproducible and
//    independent of which physical blocks hold the tokens.

#include <atomic>
#include <type_traits>

#include "kernels.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;          // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kChunk = 16;         // tokens per chunk
// Occupancy (waves per SIMD) of the vector kernel, which serves 1-2 query
// heads per KV head: 4 waves (128 VGPRs) with two chunks of K and V in
// registers.
constexpr int kVectorWavesPerSimd = 4;
constexpr float kNegBig = -1.0e30f;  // start value of a running max
// Word 3 of a gfx9-family buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of a buffer load: the "nt" (non-temporal) bit.  Every
// K/V byte is read once per call, so the loads are marked as streaming; on
// gfx950 this raises sustained read bandwidth by about a tenth.
constexpr int kNonTemporal = 2;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (LPR = 8 or 16).  Every lane of a group
// ends with the same, bitwise identical value (each step adds a commutative
// pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp_mov<0xB1>(x);                       // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);                       // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);                      // row_half_mirror
    if constexpr (LPR == 16) x += dpp_mov<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ uint4 as_uint4(__attribute__((ext_vector_type(4))) unsigned int v) {
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int64_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    return x;
}

// Wave-uniform value of lane `src` (src itself uniform), in scalar registers.
__device__ __forceinline__ int64_t readlane64(int64_t x, int src) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), src);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32), src);
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int64_t uniform64(int64_t x) { return readlane64(x, 0); }

// Context length of sequence s, clamped to [0, max_tokens].
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int s) {
    const int L = a.context_lens[s];
    return L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
}

__device__ __forceinline__ int chunks_of(int L) { return (L + kChunk - 1) / kChunk; }

// Chunks of one KV head over the whole batch (wave-uniform result).
__device__ int64_t chunks_per_head(const DecodeArgs& a, int lane) {
    int64_t tot = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += kWave) {
        const int s = b0 + lane;
        tot += wave_sum64(s < a.num_seqs ? chunks_of(clamped_len(a, s)) : 0);
    }
    return uniform64(tot);
}

// The split whose range holds chunk x: the largest w with floor(w*U/W) <= x,
// i.e. floor(((x+1)*W - 1) / U).
__device__ __forceinline__ int owner_of(int64_t x, int64_t U, int W) {
    return static_cast<int>(((x + 1) * W - 1) / U);
}

// Most chunks of any one sequence (wave-uniform result).
__device__ int max_chunks(const DecodeArgs& a, int lane) {
    int m = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += kWave) {
        const int s = b0 + lane;
        int x = s < a.num_seqs ? chunks_of(clamped_len(a, s)) : 0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) x = max(x, __shfl_xor(x, o, kWave));
        m = max(m, x);
    }
    return uniform(m);
}

// The split count the matrix-core and merge kernels work with: num_splits,
// or the smaller num_splits_hg (two workgroups a compute unit, which the
// head-group order streams faster with) when every sequence would take the
// head-group order with it.  Workgroups past it have no work.  U: chunks of
// the list.
__device__ int splits_in_use(const DecodeArgs& a, int64_t U, int lane) {
    const int N = a.num_splits, Nh = a.num_splits_hg;
    if (!a.head_groups || a.whole_pairs || Nh <= 0 || Nh >= N || U < 4 * static_cast<int64_t>(Nh)) return N;
    return 4 * static_cast<int64_t>(max_chunks(a, lane)) * Nh <= 30 * U ? Nh : N;
}

template <int D>
struct Geometry {
    static constexpr int LPR = D / 8;            // lanes per token row
    static constexpr int RPL = kWave / LPR;      // token rows per wave load
    static constexpr int LPC = kChunk / RPL;     // loads per chunk (K or V)
};

template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kVectorWavesPerSimd)))
void decode_split_kernel(const DecodeArgs a) {
    static_assert(G >= 1 && G <= 2, "3 to 8 query heads per KV head run on decode_mfma_kernel");
    using Geo = Geometry<D>;
    constexpr int LPR = Geo::LPR;
    constexpr int RPL = Geo::RPL;
    constexpr int LPC = Geo::LPC;
    constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;   // blocks per chunk
    constexpr int kPerBlock = LPC / BPC;                  // granules of a chunk per block
    static_assert(BS % RPL == 0, "a load must not straddle two blocks");
    // The pair's ragged last chunk goes through the load pipeline (its rows
    // past the context read as zeros through a shortened buffer range) when
    // it lies in one block.  Otherwise it is loaded after the pipeline and
    // its rows are dropped in registers.
    constexpr bool kFold = BS >= kChunk;

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int row = lane / LPR;
    const int col = lane % LPR;
    // (sequence, KV head) pairs per sequence: virtual heads when a large
    // query group is cut into several (each re-reads its KV head's rows).
    const int Hkv = a.num_kv_heads * a.kv_split;
    const int N = a.num_splits;

    // Bytes from one token's row of a KV head to the next token's: a whole slot
    // (slot-major) or one head row (head-major).
    const uint32_t row_bytes = a.head_major ? D * 2 : static_cast<uint32_t>(a.num_kv_heads) * D * 2;
    const uint32_t block_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2 * BS;
    // Per-lane byte offset inside a load: row `row` of the load, 16-byte column `col`.
    const uint32_t lane_off = row * row_bytes + col * 16;

    // With at most 64 sequences, one load of the context lengths (lane i holds
    // sequence i) serves the total, the search for the first pair and the walk
    // from pair to pair; larger batches read them again as needed.
    const bool lens_in_regs = a.num_seqs <= kWave;
    const int len_reg = (lens_in_regs && lane < a.num_seqs) ? clamped_len(a, lane) : 0;
    const int64_t incl_reg = wave_incl_scan64(chunks_of(len_reg), lane);
    const int64_t U = (lens_in_regs ? readlane64(incl_reg, kWave - 1) : chunks_per_head(a, lane)) * Hkv;
    auto len_of = [&](int sq) {
        return lens_in_regs ? __builtin_amdgcn_readlane(len_reg, sq) : clamped_len(a, sq);
    };

    // Process the chunks [start, end) of split `unit`: walk the pairs they
    // cover; each piece of a pair (a segment) is reduced by the workgroup and
    // written as fp16 output (whole pair) or as partials (slot unit + pair).
    auto process_split = [&](int unit, int64_t start, int64_t end) {
        // Locate the pair holding chunk `start`: the first sequence whose running
        // chunk total (times Hkv) passes it.
        int s = 0, L = 0, nch = 0;
        int64_t seq_base = 0;        // Hkv * chunks of all earlier sequences
        if (lens_in_regs) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.num_seqs && incl_reg * Hkv > start);
            if (hit) {
                const int f = __builtin_ctzll(hit);
                s = f;
                L = __builtin_amdgcn_readlane(len_reg, f);
                nch = chunks_of(L);
                seq_base = (readlane64(incl_reg, f) - nch) * Hkv;
            }
        } else {
            int64_t base = 0;
            for (int b0 = 0; b0 < a.num_seqs; b0 += kWave) {
                const int sl = b0 + lane;
                const int Ll = sl < a.num_seqs ? clamped_len(a, sl) : 0;
                const int64_t n = chunks_of(Ll);
                const int64_t incl = wave_incl_scan64(n, lane);
                const uint64_t hit = __builtin_amdgcn_ballot_w64(sl < a.num_seqs && (base + incl) * Hkv > start);
                if (hit) {
                    const int f = __builtin_ctzll(hit);
                    s = b0 + f;
                    L = __builtin_amdgcn_readlane(Ll, f);
                    nch = chunks_of(L);
                    seq_base = (base + readlane64(incl, f) - nch) * Hkv;
                    break;
                }
                base += readlane64(incl, kWave - 1);
            }
        }
        if (nch == 0) return;        // not reached: chunk `start` < U lies in some pair
        int g = static_cast<int>((start - seq_base) / nch);
        int c0 = static_cast<int>((start - seq_base) % nch);
        int64_t pos = start;

        for (;;) {
            const int c1 = static_cast<int>(nch - c0 < end - pos ? nch : c0 + (end - pos));
            const int n_seg = c1 - c0;
            // This wave's chunks of the segment: c0 + wave + 4k, k < n_local;
            // the first n_full of them hold 16 tokens each.
            const int n_local = n_seg > wave ? (n_seg - wave + kWaves - 1) / kWaves : 0;
            const int full_seg = (c1 * kChunk <= L ? c1 : c1 - 1) - c0;
            const int n_full = full_seg > wave ? (full_seg - wave + kWaves - 1) / kWaves : 0;
            // The pair's ragged last chunk (none when L is a multiple of 16) and
            // the bytes of its block that hold tokens.
            const int c_rag = (L % kChunk) ? nch - 1 : -1;
            const uint32_t rag_bytes = static_cast<uint32_t>(L - ((nch - 1) * kChunk / BS) * BS) * row_bytes;
            const int h0 = g * G;
            const size_t out_row0 = (static_cast<size_t>(s) * a.num_q_heads + h0) * D;
            const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
            // KV head g's first row in a block.
            const size_t head_off = static_cast<size_t>(g / a.kv_split) * D * 2 * (a.head_major ? BS : 1);
            const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
            const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;

            // This lane's 8 columns of the G query rows.
            half2_t qv[G][4];
    #pragma unroll
            for (int h = 0; h < G; ++h) {
                const uint4 qw = *reinterpret_cast<const uint4*>(a.q + out_row0 + h * D + col * 8);
                qv[h][0] = __builtin_bit_cast(half2_t, qw.x);
                qv[h][1] = __builtin_bit_cast(half2_t, qw.y);
                qv[h][2] = __builtin_bit_cast(half2_t, qw.z);
                qv[h][3] = __builtin_bit_cast(half2_t, qw.w);
            }

            float m[G], l[G], acc[G][8];
    #pragma unroll
            for (int h = 0; h < G; ++h) {
                m[h] = kNegBig;
                l[h] = 0.f;
    #pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
            }

            for (int kw = 0; kw < n_local; kw += kWave) {
                // Table entries of this window of the wave's chunks: lane k holds
                // local chunk kw + k.
                int ids[BPC];
                bool bad = false;
                {
                    const int c = c0 + wave + (kw + lane) * kWaves;
                    const int j0 = c * kChunk / BS;
    #pragma unroll
                    for (int e = 0; e < BPC; ++e) {
                        int id = -1;
                        const int j = j0 + e;
                        if (kw + lane < n_local && j * BS < L) {
                            id = trow[j];
                            if (id < 0 || id >= a.num_blocks) {
                                id = -1;
                                bad = true;
                            }
                        }
                        ids[e] = id;
                    }
                }
                const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
                const int nw = n_local - kw < kWave ? n_local - kw : kWave;          // chunks in window
                const int nfw = n_full - kw < 0 ? 0 : (n_full - kw < nw ? n_full - kw : nw);

                // Block and in-block row offset of granule i (static, 0 <= i <
                // LPC: RPL token rows, one per row group) of window chunk k.
                // A load through a descriptor with an empty range returns zeros
                // without touching memory: used past the end of the work (so a
                // pipeline issues the same loads every step and its wait counts
                // are compile-time constants) and for bad table entries.
                struct Src {
                    __amdgpu_buffer_rsrc_t kr, vr;
                    int soff;
                    bool ok;          // this lane's row holds a token of the context
                };
                auto source = [&](int k, int i, bool live) -> Src {
                    const int e = i / kPerBlock;
                    const int c = c0 + wave + (kw + k) * kWaves;
                    int blk = __builtin_amdgcn_readlane(ids[e], k & (kWave - 1));
                    const bool blk_ok = blk >= 0;
                    blk = blk_ok ? blk : 0;
                    uint32_t full = block_bytes;
                    if constexpr (kFold) {
                        if (c == c_rag) full = rag_bytes;    // ends at the context's last token
                    }
                    const uint32_t range = (live && blk_ok) ? full : 0u;
                    const size_t boff = static_cast<size_t>(blk) * block_bytes;
                    Src r;
                    r.kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + boff), 0, range, kRsrcWord3);
                    r.vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + boff), 0, range, kRsrcWord3);
                    r.soff = static_cast<int>((static_cast<uint32_t>(c * kChunk + i * RPL) % BS) * row_bytes);
                    r.ok = blk_ok && (i * RPL + row < L - c * kChunk);
                    return r;
                };
                // Loads are issued in program order (a scheduling barrier after
                // each): the wait counts of the pipeline depend on the order of
                // the loads in flight being the same on every path into a step.
                auto load = [&](const __amdgpu_buffer_rsrc_t& rs, int soff) {
                    const uint4 r = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, soff, kNonTemporal));
                    __builtin_amdgcn_sched_barrier(0);
                    return r;
                };
                // Issue a chunk's loads: its K rows first, then its V rows.
                auto issue_chunk = [&](uint4 (&kd)[LPC], uint4 (&vd)[LPC], int k, bool live) {
    #pragma unroll
                    for (int i = 0; i < LPC; ++i) {
                        const Src r = source(k, i, live);
                        kd[i] = load(r.kr, r.soff);
                    }
    #pragma unroll
                    for (int i = 0; i < LPC; ++i) {
                        const Src r = source(k, i, live);
                        vd[i] = load(r.vr, r.soff);
                    }
                };

                // Consume chunk k held in (kd, vd) and refill the registers with
                // chunk k2 as they free up: the K rows right after the scores,
                // each V row right after its P.V update.  While a chunk is
                // consumed, the next chunk and part of the one after are in
                // flight.  One max update (and rescale) per chunk and row group.
                auto consume = [&](uint4 (&kd)[LPC], uint4 (&vd)[LPC], int k, int k2, bool live2,
                                   auto masked_tag) {
                    constexpr bool kMasked = decltype(masked_tag)::value;
                    // Rows of the chunk that hold a token.  On the pipelined path
                    // of a folded kernel only rows past the context (the ragged
                    // chunk) fail; their K and V read as zeros, and the score is
                    // masked here.
                    bool ok[LPC];
                    if (kMasked) {
    #pragma unroll
                        for (int i = 0; i < LPC; ++i) ok[i] = source(k, i, true).ok;
                    } else if (kFold) {
                        const int rem = L - (c0 + wave + (kw + k) * kWaves) * kChunk;
    #pragma unroll
                        for (int i = 0; i < LPC; ++i) ok[i] = i * RPL + row < rem;
                    }
                    float sc[LPC][G];
    #pragma unroll
                    for (int i = 0; i < LPC; ++i) {
                        const half2_t k0 = __builtin_bit_cast(half2_t, kd[i].x);
                        const half2_t k1 = __builtin_bit_cast(half2_t, kd[i].y);
                        const half2_t k2h = __builtin_bit_cast(half2_t, kd[i].z);
                        const half2_t k3 = __builtin_bit_cast(half2_t, kd[i].w);
    #pragma unroll
                        for (int h = 0; h < G; ++h) {
                            float d = __builtin_amdgcn_fdot2(qv[h][0], k0, 0.f, false);
                            d = __builtin_amdgcn_fdot2(qv[h][1], k1, d, false);
                            d = __builtin_amdgcn_fdot2(qv[h][2], k2h, d, false);
                            d = __builtin_amdgcn_fdot2(qv[h][3], k3, d, false);
                            d = row_sum<LPR>(d) * a.scale_log2;
                            if ((kMasked || kFold) && !ok[i]) d = -__builtin_inff();
                            sc[i][h] = d;
                        }
                    }
                    if (!kMasked) {
    #pragma unroll
                        for (int i = 0; i < LPC; ++i) {
                            const Src r = source(k2, i, live2);
                            kd[i] = load(r.kr, r.soff);
                        }
                    }
    #pragma unroll
                    for (int h = 0; h < G; ++h) {
                        float mx = sc[0][h];
    #pragma unroll
                        for (int i = 1; i < LPC; ++i) mx = __builtin_fmaxf(mx, sc[i][h]);
                        const float m_new = __builtin_fmaxf(m[h], mx);
                        const float alpha = fast_exp2(m[h] - m_new);
                        m[h] = m_new;
                        l[h] *= alpha;
    #pragma unroll
                        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
                    }
    #pragma unroll
                    for (int i = 0; i < LPC; ++i) {
                        uint32_t vw[4] = {vd[i].x, vd[i].y, vd[i].z, vd[i].w};
                        if (kMasked && !ok[i]) {
                            // p is 0 here, but 0 * (NaN or Inf) is not: drop the row.
                            vw[0] = vw[1] = vw[2] = vw[3] = 0;
                        }
    #pragma unroll
                        for (int h = 0; h < G; ++h) {
                            const float pr = fast_exp2(sc[i][h] - m[h]);
                            l[h] += pr;
    #pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const half2_t v2 = __builtin_bit_cast(half2_t, vw[j]);
                                acc[h][2 * j] = __builtin_fmaf(pr, static_cast<float>(v2.x), acc[h][2 * j]);
                                acc[h][2 * j + 1] = __builtin_fmaf(pr, static_cast<float>(v2.y), acc[h][2 * j + 1]);
                            }
                        }
                        if (!kMasked) {
                            const Src r = source(k2, i, live2);
                            vd[i] = load(r.vr, r.soff);
                        }
                    }
                };

                using Full = std::integral_constant<bool, false>;
                using Masked = std::integral_constant<bool, true>;
                // Chunks the pipeline takes: every chunk of the window when the
                // ragged one is folded in, else the full ones.
                const int npw = kFold ? nw : nfw;
                if (!any_bad && npw > 0) {
                    // Chunks alternate between two register sets X and Y.  Both
                    // loop bodies are unconditional, so every wait is static.
                    uint4 xk[LPC], xv[LPC], yk[LPC], yv[LPC];
                    issue_chunk(xk, xv, 0, true);
                    issue_chunk(yk, yv, 1, 1 < npw);
                    int k = 0;
                    for (; k + 1 < npw; k += 2) {
                        consume(xk, xv, k, k + 2, k + 2 < npw, Full{});
                        consume(yk, yv, k + 1, k + 3, k + 3 < npw, Full{});
                    }
                    if (k < npw) consume(xk, xv, k, k + 2, false, Full{});
                }
                // The pair's ragged last chunk (when not folded), or every chunk
                // of a window with a bad table entry: rows holding no token are
                // dropped.
                for (int k = any_bad ? 0 : npw; k < nw; ++k) {
                    uint4 tk[LPC], tv[LPC];
                    issue_chunk(tk, tv, k, true);
                    consume(tk, tv, k, 0, false, Masked{});
                }
            }

            // Merge the row groups of this wave (each kept its own stream).
    #pragma unroll
            for (int h = 0; h < G; ++h) {
                float mw = m[h];
    #pragma unroll
                for (int o = LPR; o < kWave; o <<= 1) mw = __builtin_fmaxf(mw, shfl_xor(mw, o));
                const float f = fast_exp2(m[h] - mw);
                float lw = l[h] * f;
    #pragma unroll
                for (int o = LPR; o < kWave; o <<= 1) lw += shfl_xor(lw, o);
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = acc[h][e] * f;
    #pragma unroll
                    for (int o = LPR; o < kWave; o <<= 1) x += shfl_xor(x, o);
                    acc[h][e] = x;
                }
                m[h] = mw;
                l[h] = lw;
            }
            if (row == 0) {
    #pragma unroll
                for (int h = 0; h < G; ++h)
    #pragma unroll
                    for (int e = 0; e < 8; ++e) s_acc[wave][h][col * 8 + e] = acc[h][e];
            }
            if (lane == 0) {
    #pragma unroll
                for (int h = 0; h < G; ++h) {
                    s_m[wave][h] = m[h];
                    s_l[wave][h] = l[h];
                }
            }
            __syncthreads();

            // Merge the 4 waves; write the fp16 rows when the segment is the whole
            // pair, else this segment's partials.
            const bool whole = c0 == 0 && c1 == nch;
            const size_t slot = static_cast<size_t>(unit) + static_cast<size_t>(s) * Hkv + g;
            for (int o = threadIdx.x; o < G * D; o += kThreads) {
                const int h = o / D;
                const int d = o % D;
                float mm = s_m[0][h];
    #pragma unroll
                for (int v = 1; v < kWaves; ++v) mm = __builtin_fmaxf(mm, s_m[v][h]);
                float num = 0.f, den = 0.f;
    #pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    const float f = fast_exp2(s_m[v][h] - mm);
                    num = __builtin_fmaf(f, s_acc[v][h][d], num);
                    den = __builtin_fmaf(f, s_l[v][h], den);
                }
                if (whole) {
                    // den is 0 only when no token was read (every table entry of
                    // the pair out of range); NaN inputs still propagate.
                    const float r = den == 0.f ? 0.f : num / den;
                    a.out[out_row0 + o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
                } else {
                    a.part_o[(slot * G + h) * D + d] = num;
                    if (d == 0) {
                        a.part_ml[(slot * G + h) * 2] = mm;
                        a.part_ml[(slot * G + h) * 2 + 1] = den;
                    }
                }
            }

            pos += n_seg;
            if (pos >= end) break;
            __syncthreads();             // LDS is reused by the next segment
            // Next pair: the next KV head, or the next sequence holding tokens.
            c0 = 0;
            if (++g == Hkv) {
                g = 0;
                L = 0;
                while (L == 0 && s + 1 < a.num_seqs) L = len_of(++s);
                nch = chunks_of(L);
                if (nch == 0) break;     // not reached while pos < end
            }
        }
    };

    const int u = blockIdx.x;
    int64_t start, end;
    if (a.whole_pairs) {
        // Pair u = (s, g) whole: its chunks follow Hkv * (chunks of the earlier
        // sequences) + g * (its own chunk count).  An empty context has no
        // chunk; its zero rows are written here (no merge kernel runs).
        const int s = u / Hkv;
        const int g = u - s * Hkv;
        const int L = __builtin_amdgcn_readlane(len_reg, s);
        const int nch = chunks_of(L);
        if (nch == 0) {
            for (int o = threadIdx.x; o < G * D; o += kThreads)
                a.out[(static_cast<size_t>(s) * a.num_q_heads + g * G) * D + o] = 0;
            return;
        }
        start = (readlane64(incl_reg, s) - nch) * Hkv + static_cast<int64_t>(g) * nch;
        end = start + nch;
    } else {
        start = static_cast<int64_t>(u) * U / N;
        end = static_cast<int64_t>(u + 1) * U / N;
    }
    if (start < end) process_split(u, start, end);
}

// ---------------------------------------------------------------------------
// Matrix-core variant for 3 to 8 query heads per KV head (blocks of 8 tokens
// or more; at block 8 a 16-token chunk takes two table entries).
//
// Same partition, workspace and merge as decode_split_kernel, except that on
// the slot-major layout with a multiple of 4 KV heads (blocks of 16 or more) a
// sequence's part of the chunk list may run in the head-group order (groups of
// 4 heads, chunk-major inside a group, one head per wave; see hg_mode below),
// whose partial slots are 4 * (split + group) + head in group.  The work on a
// segment: the G query rows of a KV head are the rows of
// v_mfma_f32_4x4x4_16b_f16 tiles (one set of 4 rows for G <= 4, two for
// G <= 8; rows past G hold zero queries and are never written), so that the
// products run on the matrix cores and the vector ALUs only keep the
// softmax bookkeeping of one score per lane:
//  * scores.  The instruction holds 16 independent 4x4x4 blocks.  Block
//    b = 4*tg + p of lane l = 4*b + j pairs token 4*tg + j of the 16-token
//    chunk with a quarter p of the head dimension: the lane loads 16 bytes
//    of that token's K row at byte 64*m + 16*p (m = 0 .. D/32-1), which is
//    the B operand of two k-steps as loaded; the A operand is the matching
//    query columns, held in registers for the whole segment.  The four
//    quarters' partial scores are summed across lanes (bits 2 and 3 of the
//    lane id) so that lane l ends with the score of head p, token 4*tg + j.
//  * softmax: one running max per head, shared by every lane holding that
//    head, updated once per chunk (cross-lane max over the 16 tokens); exp2
//    of the scaled score; the probability is rounded to fp16 (the operand
//    type) and the row sum adds the rounded values, so numerator and
//    denominator use the same weights.
//  * values.  P.V contracts over tokens, so its B operand needs 4 tokens of
//    one column per lane.  The chunk's V rows are loaded in the natural
//    layout (16 lanes per 256-byte row), written to a wave-private LDS tile
//    (rows padded by 64 bytes: the transposing reads hit each bank at most
//    twice) and read back with ds_read_b64_tr_b16, whose 16-lane transpose
//    turns 4 rows x 4 columns into the operand of lane l: tokens
//    4*ks .. 4*ks+3 of column 64*grp + l.  The probabilities reach the A
//    operand through a 128-byte LDS tile per row set.
//  * the output accumulator of lane l is column 64*grp + l of all the set's
//    heads: nothing to reduce at the segment end but the row sums.
// K and V of the next two chunks stay in flight in registers (two sets) as in
// the vector kernel; loads past a context or behind a bad table entry go
// through a shortened or empty buffer range and return zeros.
// ---------------------------------------------------------------------------
typedef _Float16 mf_h4 __attribute__((ext_vector_type(4)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));
typedef short mf_s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mf_s4 lds_s4;

template <int G>
constexpr int mfma_row_sets() { return (G + 3) / 4; }

__device__ __forceinline__ float permswap16_a(float x, float& b) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
    return __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
}
__device__ __forceinline__ float permswap32_a(float x, float& b) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
    return __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
}
// Max / sum over the 16 tokens of a chunk held by lanes that differ in bits
// 0, 1 (token within a group of 4), 4 and 5 (group).  Every lane of the set
// gets the same bits: each step combines a commutative pair.
__device__ __forceinline__ float tok_max(float x) {
    x = __builtin_fmaxf(x, dpp_mov<0xB1>(x));
    x = __builtin_fmaxf(x, dpp_mov<0x4E>(x));
    float b;
    float a = permswap16_a(x, b);
    x = __builtin_fmaxf(a, b);
    a = permswap32_a(x, b);
    return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float tok_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    float b;
    float a = permswap16_a(x, b);
    x = a + b;
    a = permswap32_a(x, b);
    return a + b;
}

// Register budget: 3 waves a SIMD (168 VGPRs) for G = 3 and 4, whose 128-register
// forms spill (the split count puts 3 workgroups on a CU anyway), 2 for G = 5..8.
template <int G>
constexpr int mfma_waves_per_simd() { return G <= 4 ? 3 : 2; }

template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<G>())))
void decode_mfma_kernel(const DecodeArgs a) {
    static_assert(BS >= kChunk || 2 * BS == kChunk, "one or two blocks per chunk");
    constexpr int BPC = BS >= kChunk ? 1 : 2;     // blocks per chunk
    constexpr int RS = mfma_row_sets<G>();        // sets of 4 query rows
    constexpr int KM = D / 32;                    // K loads per chunk (4 or 8 whole rows each)
    constexpr int SL = D / 8;                     // 16-byte slices of a row
    constexpr int TPL = kChunk / KM;              // K rows per load
    constexpr int NG = D / 64;                    // 64-column groups of the output
    constexpr int LPR = D / 8;                    // lanes per V row (natural layout)
    constexpr int RPL = kWave / LPR;              // V rows per wave load
    constexpr int VL = kChunk / RPL;              // V loads per chunk
    constexpr int VROW = D * 2 + 64;              // padded LDS row of the V tile (bytes)

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];
    __shared__ __attribute__((aligned(16))) char s_v[kWaves][kChunk * VROW];
    __shared__ __attribute__((aligned(16))) _Float16 s_p[kWaves][RS][4][kChunk];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int lj = lane & 3;                      // token in group (B, D) / query row (A)
    const int lp = (lane >> 2) & 3;               // quarter of the head dimension / head after the sum
    const int ltg = lane >> 4;                    // token group
    // (sequence, KV head) pairs per sequence: virtual heads when a large
    // query group is cut into several (each re-reads its KV head's rows).
    const int Hkv = a.num_kv_heads * a.kv_split;

    const uint32_t row_bytes = a.head_major ? D * 2 : static_cast<uint32_t>(a.num_kv_heads) * D * 2;
    const uint32_t block_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2 * BS;
    // K loads: lane 4*b + j reads slice b % SL of row j + 4*(b / SL) of the
    // load's TPL rows -- whole rows per instruction, in the lane order of the
    // B operand (block b = slice, column j = row).
    const int k_slice = (lane >> 2) % SL;
    const uint32_t k_lane_off = static_cast<uint32_t>(lj + 4 * ((lane >> 2) / SL)) * row_bytes + 16 * k_slice;
    const uint32_t v_lane_off = static_cast<uint32_t>(lane / LPR) * row_bytes + 16 * (lane % LPR);
    // Token of this lane's score after the slice sum (see consume()).
    const int t_lane = D == 128 ? 4 * ltg + lj : 8 * ((lane >> 4) & 1) + 4 * (lane >> 5) + lj;
    char* vtile = &s_v[wave][0];
    const uint32_t v_wr_off = static_cast<uint32_t>(lane / LPR) * VROW + 16 * (lane % LPR);
    // Transposing read of lane l = 16*g' + 4*e + q: row e of a 4-row step,
    // columns 16*g' + 4*q .. +3 of a 64-column group.
    const uint32_t v_rd_off = static_cast<uint32_t>((lane >> 2) & 3) * VROW + (16 * (lane >> 4) + 4 * (lane & 3)) * 2;

    const bool lens_in_regs = a.num_seqs <= kWave;
    const int len_reg = (lens_in_regs && lane < a.num_seqs) ? clamped_len(a, lane) : 0;
    const int64_t incl_reg = wave_incl_scan64(chunks_of(len_reg), lane);
    const int64_t U = (lens_in_regs ? readlane64(incl_reg, kWave - 1) : chunks_per_head(a, lane)) * Hkv;
    const int N = splits_in_use(a, U, lane);
    // Head groups: a sequence's part of the list may run group by group of 4
    // (virtual) KV heads, chunk-major inside a group with the group's heads
    // interleaved (entry 4c + j: chunk c of head 4*hg + j).  Each wave then
    // keeps one head for a whole segment, and the 4 waves of a workgroup read
    // the same 16 tokens of 4 adjacent heads (1 KiB of each slot-major token
    // row instead of 256-byte pieces 2 KiB apart).  Allowed with at least 4
    // entries a split (every split that touches a head's entries then holds
    // one of them), never for whole pairs; taken by a sequence whose groups
    // span at most about 32 splits (seq_hg), so that the merge still reads
    // each pair's partials in one round.  With head groups allowed, every
    // partial slot is 4 * (split + group) + head in group, in either order.
    const bool hg_mode = a.head_groups && !a.whole_pairs && U >= 4 * static_cast<int64_t>(N);
    auto seq_hg = [&](int nch) {
        return hg_mode && 4 * static_cast<int64_t>(nch) * N <= 30 * U;
    };
    auto len_of = [&](int sq) {
        return lens_in_regs ? __builtin_amdgcn_readlane(len_reg, sq) : clamped_len(a, sq);
    };

    auto process_split = [&](int unit, int64_t start, int64_t end) {
        int s = 0, L = 0, nch = 0;
        int64_t seq_base = 0;
        if (lens_in_regs) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.num_seqs && incl_reg * Hkv > start);
            if (hit) {
                const int f = __builtin_ctzll(hit);
                s = f;
                L = __builtin_amdgcn_readlane(len_reg, f);
                nch = chunks_of(L);
                seq_base = (readlane64(incl_reg, f) - nch) * Hkv;
            }
        } else {
            int64_t base = 0;
            for (int b0 = 0; b0 < a.num_seqs; b0 += kWave) {
                const int sl = b0 + lane;
                const int Ll = sl < a.num_seqs ? clamped_len(a, sl) : 0;
                const int64_t n = chunks_of(Ll);
                const int64_t incl = wave_incl_scan64(n, lane);
                const uint64_t hit = __builtin_amdgcn_ballot_w64(sl < a.num_seqs && (base + incl) * Hkv > start);
                if (hit) {
                    const int f = __builtin_ctzll(hit);
                    s = b0 + f;
                    L = __builtin_amdgcn_readlane(Ll, f);
                    nch = chunks_of(L);
                    seq_base = (base + readlane64(incl, f) - nch) * Hkv;
                    break;
                }
                base += readlane64(incl, kWave - 1);
            }
        }
        if (nch == 0) return;
        // g: the pair (with head groups, the group) of the first segment;
        // c0, c1: the segment's first and end entries in that pair's (group's)
        // part of the list, which holds span entries.
        int HG = seq_hg(nch) ? 4 : 1;             // pairs one segment of this sequence covers
        int64_t span = static_cast<int64_t>(HG) * nch;
        int g = static_cast<int>((start - seq_base) / span);
        int c0 = static_cast<int>((start - seq_base) % span);
        int64_t pos = start;

        for (;;) {
            const int c1 = static_cast<int>(span - c0 < end - pos ? span : c0 + (end - pos));
            const int n_seg = c1 - c0;
            const int n_local = n_seg > wave ? (n_seg - wave + kWaves - 1) / kWaves : 0;
            // This wave's entries are c0 + wave + 4k (k < n_local): chunks
            // cb + cs*k of (virtual) KV head gw.
            const bool hgs = HG == 4;
            const int jw = hgs ? (c0 + wave) & 3 : 0;
            const int gw = hgs ? HG * g + jw : g;
            const int cb = hgs ? (c0 + wave) >> 2 : c0 + wave;
            const int cs = hgs ? 1 : kWaves;
            const int c_rag = (L % kChunk) ? nch - 1 : -1;
            const uint32_t rag_bytes = static_cast<uint32_t>(L - ((nch - 1) * kChunk / BS) * BS) * row_bytes;
            // Two blocks a chunk: the ragged chunk's rows in its first and
            // second block (rag_bytes counts them from the first).
            const int rag_rows = L - (nch - 1) * kChunk;
            const uint32_t rag_lo = static_cast<uint32_t>(rag_rows < BS ? rag_rows : BS) * row_bytes;
            const uint32_t rag_hi = static_cast<uint32_t>(rag_rows > BS ? rag_rows - BS : 0) * row_bytes;
            const int h0 = gw * G;
            const size_t out_row0 = (static_cast<size_t>(s) * a.num_q_heads + h0) * D;
            const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
            const size_t head_off = static_cast<size_t>(gw / a.kv_split) * D * 2 * (a.head_major ? BS : 1);
            const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
            const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;

            // A operands of the scores: query row 4*r + lj, the 8 columns of
            // slice k_slice (k-steps hh = 0, 1 of 4 columns each).
            mf_h4 qop[RS][2];
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                uint4 w = make_uint4(0u, 0u, 0u, 0u);
                if (4 * r + lj < G) w = *reinterpret_cast<const uint4*>(a.q + out_row0 + (4 * r + lj) * D + 8 * k_slice);
                qop[r][0] = __builtin_bit_cast(mf_h4, make_uint2(w.x, w.y));
                qop[r][1] = __builtin_bit_cast(mf_h4, make_uint2(w.z, w.w));
            }
            mf_f4 acc[RS][NG];
            float m_run[RS], l_run[RS];
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                m_run[r] = kNegBig;
                l_run[r] = 0.f;
#pragma unroll
                for (int n = 0; n < NG; ++n) acc[r][n] = mf_f4{0.f, 0.f, 0.f, 0.f};
            }

            for (int kw = 0; kw < n_local; kw += kWave) {
                int ids = -1, ids2 = -1;               // ids2: a chunk's second block
                {
                    const int c = cb + (kw + lane) * cs;
                    if (kw + lane < n_local) {
                        const int id = trow[c * kChunk / BS];
                        ids = (id < 0 || id >= a.num_blocks) ? -1 : id;
                        // The second block's entry exists only if it holds tokens.
                        if (BPC == 2 && c * kChunk + BS < L) {
                            const int id2 = trow[c * kChunk / BS + 1];
                            ids2 = (id2 < 0 || id2 >= a.num_blocks) ? -1 : id2;
                        }
                    }
                }
                const int nw = n_local - kw < kWave ? n_local - kw : kWave;

                struct Src {
                    __amdgpu_buffer_rsrc_t kr, vr;   // the chunk's (first) block
                    __amdgpu_buffer_rsrc_t kr2, vr2; // two blocks a chunk: tokens BS .. 2BS-1
                    int soff;               // byte offset of the chunk's first row in its block
                    bool ok_lo, ok_hi;      // table entries of tokens 0 .. BS-1 and BS .. in range
                    int rem;                // tokens of the context from the chunk's first on
                };
                auto source = [&](int k, bool live) -> Src {
                    const int c = cb + (kw + k) * cs;
                    int blk = __builtin_amdgcn_readlane(ids, k & (kWave - 1));
                    const bool blk_ok = blk >= 0;
                    blk = blk_ok ? blk : 0;
                    const bool rag = c == c_rag;
                    const uint32_t full = rag ? (BPC == 2 ? rag_lo : rag_bytes) : block_bytes;
                    const uint32_t range = (live && blk_ok) ? full : 0u;
                    const size_t boff = static_cast<size_t>(blk) * block_bytes;
                    Src r;
                    r.kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + boff), 0, range, kRsrcWord3);
                    r.vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + boff), 0, range, kRsrcWord3);
                    r.kr2 = r.kr;
                    r.vr2 = r.vr;
                    r.ok_lo = r.ok_hi = blk_ok;
                    if constexpr (BPC == 2) {
                        // A block id of -1 here is an entry out of range or a
                        // block holding no token of the context; either way its
                        // rows read as zeros and their scores are masked.
                        int blk2 = __builtin_amdgcn_readlane(ids2, k & (kWave - 1));
                        const bool ok2 = blk2 >= 0;
                        blk2 = ok2 ? blk2 : 0;
                        const uint32_t range2 = (live && ok2) ? (rag ? rag_hi : block_bytes) : 0u;
                        const size_t boff2 = static_cast<size_t>(blk2) * block_bytes;
                        r.kr2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + boff2), 0, range2, kRsrcWord3);
                        r.vr2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + boff2), 0, range2, kRsrcWord3);
                        r.ok_hi = ok2;
                    }
                    r.soff = static_cast<int>((static_cast<uint32_t>(c * kChunk) % BS) * row_bytes);
                    r.rem = L - c * kChunk;
                    return r;
                };
                auto load = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t voff, int soff) {
                    const uint4 r = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNonTemporal));
                    __builtin_amdgcn_sched_barrier(0);
                    return r;
                };
                // Load m (v) holds rows TPL*m (RPL*v) on: with two blocks a
                // chunk, the first half of the loads reads the first block and
                // the second half the second, each from its block's row 0.
                auto issue_k = [&](uint4 (&kd)[KM], const Src& r) {
#pragma unroll
                    for (int m = 0; m < KM; ++m) {
                        const bool hi = BPC == 2 && m >= KM / 2;
                        kd[m] = load(hi ? r.kr2 : r.kr, k_lane_off,
                                     r.soff + static_cast<int>(TPL * (hi ? m - KM / 2 : m) * row_bytes));
                    }
                };
                auto issue_v = [&](uint4 (&vd)[VL], const Src& r) {
#pragma unroll
                    for (int v = 0; v < VL; ++v) {
                        const bool hi = BPC == 2 && v >= VL / 2;
                        vd[v] = load(hi ? r.vr2 : r.vr, v_lane_off,
                                     r.soff + static_cast<int>(RPL * (hi ? v - VL / 2 : v) * row_bytes));
                    }
                };

                auto consume = [&](uint4 (&kd)[KM], uint4 (&vd)[VL], int k, int k2, bool live2) {
                    const Src cur = source(k, true);
                    // Scores: partial dot products over slice k_slice, for the
                    // rows of each load (value 4*m + i: load m, head 4r + i).
                    mf_f4 sc[RS][KM];
#pragma unroll
                    for (int m = 0; m < KM; ++m) {
                        const mf_h4 b0 = __builtin_bit_cast(mf_h4, make_uint2(kd[m].x, kd[m].y));
                        const mf_h4 b1 = __builtin_bit_cast(mf_h4, make_uint2(kd[m].z, kd[m].w));
#pragma unroll
                        for (int r = 0; r < RS; ++r) {
                            sc[r][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(qop[r][0], b0, mf_f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                            sc[r][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(qop[r][1], b1, sc[r][m], 0, 0, 0);
                        }
                    }
                    const Src nxt = source(k2, live2);
                    issue_k(kd, nxt);
                    const bool need_mask = !(cur.ok_lo && cur.ok_hi) || (cb + (kw + k) * cs) == c_rag;
                    const bool tok_ok = (t_lane < BS ? cur.ok_lo : cur.ok_hi) && t_lane < cur.rem;
                    const bool b3 = lp & 2, b2 = lp & 1;
                    float pr[RS];
#pragma unroll
                    for (int r = 0; r < RS; ++r) {
                        // Sum the slices across lanes, halving the values held
                        // at each step: lane bit 5 (D = 128 only) keeps loads
                        // {0,1} or {2,3}, bit 4 one load, bit 3 heads {0,1} or
                        // {2,3}, bit 2 one head.  Each lane ends with one score:
                        // head lp of token t_lane.
                        float y[2][4];
                        if constexpr (KM == 4) {
#pragma unroll
                            for (int m = 0; m < 2; ++m)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    // Copy the elements out first: this compiler's bit_cast
                                    // of a vector element reads element 0 whatever the index.
                                    const float e0 = sc[r][m][i], e1 = sc[r][m + 2][i];
                                    const unsigned u0 = __builtin_bit_cast(unsigned, e0);
                                    const unsigned u1 = __builtin_bit_cast(unsigned, e1);
                                    const auto x = __builtin_amdgcn_permlane32_swap(u0, u1, false, false);
                                    y[m][i] = __builtin_bit_cast(float, static_cast<unsigned>(x[0])) +
                                              __builtin_bit_cast(float, static_cast<unsigned>(x[1]));
                                }
                        } else {
#pragma unroll
                            for (int m = 0; m < 2; ++m)
#pragma unroll
                                for (int i = 0; i < 4; ++i) y[m][i] = sc[r][m][i];
                        }
                        float z[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const unsigned u0 = __builtin_bit_cast(unsigned, y[0][i]);
                            const unsigned u1 = __builtin_bit_cast(unsigned, y[1][i]);
                            const auto x = __builtin_amdgcn_permlane16_swap(u0, u1, false, false);
                            z[i] = __builtin_bit_cast(float, static_cast<unsigned>(x[0])) +
                                   __builtin_bit_cast(float, static_cast<unsigned>(x[1]));
                        }
                        const float n0 = (b3 ? z[2] : z[0]) + dpp_mov<0x128>(b3 ? z[0] : z[2]);   // row_ror:8 = lane ^ 8
                        const float n1 = (b3 ? z[3] : z[1]) + dpp_mov<0x128>(b3 ? z[1] : z[3]);
                        const float send = b2 ? n0 : n1;
                        const float own = b2 ? n1 : n0;
                        // row_ror:n moves a value n lanes up its row: lane i reads lane i - n.
                        const float from_up = dpp_mov<0x12C>(send);     // lane + 4
                        const float from_dn = dpp_mov<0x124>(send);     // lane - 4
                        float t = (own + (b2 ? from_dn : from_up)) * a.scale_log2;
                        if (need_mask && !tok_ok) t = -__builtin_inff();
                        const float mx = tok_max(t);
                        const float m_new = __builtin_fmaxf(m_run[r], mx);
                        const float alpha = fast_exp2(m_run[r] - m_new);
                        m_run[r] = m_new;
                        const _Float16 ph = static_cast<_Float16>(fast_exp2(t - m_new));
                        l_run[r] = __builtin_fmaf(l_run[r], alpha, static_cast<float>(ph));
                        s_p[wave][r][lp][t_lane] = ph;
                        pr[r] = alpha;
                    }
                    __builtin_amdgcn_wave_barrier();
                    // Rescale the accumulators by each head's factor (one
                    // value per quarter, read from lanes 0, 4, 8, 12).
#pragma unroll
                    for (int r = 0; r < RS; ++r) {
                        const float f0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[r]), 0));
                        const float f1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[r]), 4));
                        const float f2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[r]), 8));
                        const float f3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[r]), 12));
                        if (f0 != 1.f || f1 != 1.f || f2 != 1.f || f3 != 1.f) {
#pragma unroll
                            for (int n = 0; n < NG; ++n) {
                                acc[r][n][0] *= f0;
                                acc[r][n][1] *= f1;
                                acc[r][n][2] *= f2;
                                acc[r][n][3] *= f3;
                            }
                        }
                    }
                    // V rows to the wave's LDS tile, then refill.
#pragma unroll
                    for (int v = 0; v < VL; ++v)
                        *reinterpret_cast<uint4*>(vtile + v_wr_off + RPL * v * VROW) = vd[v];
                    __builtin_amdgcn_wave_barrier();
                    issue_v(vd, nxt);
                    // P.V: k-step ks takes tokens 4ks .. 4ks+3.
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        mf_h4 pa[RS];
#pragma unroll
                        for (int r = 0; r < RS; ++r)
                            pa[r] = *reinterpret_cast<const mf_h4*>(&s_p[wave][r][lj][4 * ks]);
#pragma unroll
                        for (int n = 0; n < NG; ++n) {
                            const mf_s4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (lds_s4*)(vtile + v_rd_off + 4 * ks * VROW + 128 * n));
                            const mf_h4 vb = __builtin_bit_cast(mf_h4, raw);
#pragma unroll
                            for (int r = 0; r < RS; ++r)
                                acc[r][n] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa[r], vb, acc[r][n], 0, 0, 0);
                        }
                    }
                };

                if (nw > 0) {
                    uint4 xk[KM], xv[VL], yk[KM], yv[VL];
                    {
                        const Src r0 = source(0, true);
                        issue_k(xk, r0);
                        issue_v(xv, r0);
                        const Src r1 = source(1, 1 < nw);
                        issue_k(yk, r1);
                        issue_v(yv, r1);
                    }
                    int k = 0;
                    for (; k + 1 < nw; k += 2) {
                        consume(xk, xv, k, k + 2, k + 2 < nw);
                        consume(yk, yv, k + 1, k + 3, k + 3 < nw);
                    }
                    if (k < nw) consume(xk, xv, k, k + 2, false);
                }
            }

            if (hgs) {
                // Each wave finishes its own pair (sequence s, head gw): the
                // running max and the row sum of head 4r + i sit in lane 4i.
                if (n_local > 0) {
                    const bool whole = c0 <= jw && c1 > 4 * (nch - 1) + jw;
                    const size_t slot = 4 * (static_cast<size_t>(unit) + static_cast<size_t>(s) * (Hkv / 4) + g) + jw;
#pragma unroll
                    for (int r = 0; r < RS; ++r) {
                        const float lw = tok_sum(l_run[r]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int h = 4 * r + i;
                            if (h >= G) continue;
                            const float mh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_run[r]), 4 * i));
                            const float lh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lw), 4 * i));
#pragma unroll
                            for (int n = 0; n < NG; ++n) {
                                const int d = 64 * n + lane;
                                const float num = acc[r][n][i];
                                if (whole) {
                                    const float o = lh == 0.f ? 0.f : num / lh;
                                    a.out[out_row0 + h * D + d] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(o));
                                } else {
                                    a.part_o[(slot * G + h) * D + d] = num;
                                }
                            }
                            if (!whole && lane == 0) {
                                a.part_ml[(slot * G + h) * 2] = mh;
                                a.part_ml[(slot * G + h) * 2 + 1] = lh;
                            }
                        }
                    }
                }
            } else {
                // Row sums over the chunk tokens of this wave; then to LDS.
#pragma unroll
                for (int r = 0; r < RS; ++r) {
                    const float lw = tok_sum(l_run[r]);
                    const int h = 4 * r + lp;
                    if (ltg == 0 && lj == 0 && h < G) {
                        s_m[wave][h] = m_run[r];
                        s_l[wave][h] = lw;
                    }
#pragma unroll
                    for (int n = 0; n < NG; ++n)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (4 * r + i < G) s_acc[wave][4 * r + i][64 * n + lane] = acc[r][n][i];
                }
                __syncthreads();

                const bool whole = c0 == 0 && c1 == nch;
                const size_t slot = hg_mode ? 4 * (static_cast<size_t>(unit) + static_cast<size_t>(s) * (Hkv / 4) + (g >> 2)) + (g & 3)
                                            : static_cast<size_t>(unit) + static_cast<size_t>(s) * Hkv + g;
                for (int o = threadIdx.x; o < G * D; o += kThreads) {
                    const int h = o / D;
                    const int d = o % D;
                    float mm = s_m[0][h];
#pragma unroll
                    for (int v = 1; v < kWaves; ++v) mm = __builtin_fmaxf(mm, s_m[v][h]);
                    float num = 0.f, den = 0.f;
#pragma unroll
                    for (int v = 0; v < kWaves; ++v) {
                        const float f = fast_exp2(s_m[v][h] - mm);
                        num = __builtin_fmaf(f, s_acc[v][h][d], num);
                        den = __builtin_fmaf(f, s_l[v][h], den);
                    }
                    if (whole) {
                        const float r = den == 0.f ? 0.f : num / den;
                        a.out[out_row0 + o] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
                    } else {
                        a.part_o[(slot * G + h) * D + d] = num;
                        if (d == 0) {
                            a.part_ml[(slot * G + h) * 2] = mm;
                            a.part_ml[(slot * G + h) * 2 + 1] = den;
                        }
                    }
                }
            }

            pos += n_seg;
            if (pos >= end) break;
            if (!hgs) __syncthreads();               // LDS is reused by the next segment
            c0 = 0;
            if (++g == Hkv / HG) {
                g = 0;
                L = 0;
                while (L == 0 && s + 1 < a.num_seqs) L = len_of(++s);
                nch = chunks_of(L);
                if (nch == 0) break;
                HG = seq_hg(nch) ? 4 : 1;
                span = static_cast<int64_t>(HG) * nch;
            }
        }
    };

    const int u = blockIdx.x;
    int64_t start, end;
    if (a.whole_pairs) {
        const int s = u / Hkv;
        const int g = u - s * Hkv;
        const int L = __builtin_amdgcn_readlane(len_reg, s);
        const int nch = chunks_of(L);
        if (nch == 0) {
            for (int o = threadIdx.x; o < G * D; o += kThreads)
                a.out[(static_cast<size_t>(s) * a.num_q_heads + g * G) * D + o] = 0;
            return;
        }
        start = (readlane64(incl_reg, s) - nch) * Hkv + static_cast<int64_t>(g) * nch;
        end = start + nch;
    } else {
        if (u >= N) return;                       // beyond the split count in use
        start = static_cast<int64_t>(u) * U / N;
        end = static_cast<int64_t>(u + 1) * U / N;
    }
    if (start < end) process_split(u, start, end);
}

// Merge the partials of pairs that span several splits, and write the zero
// rows of empty contexts.  One workgroup of 4 waves per (sequence, KV head)
// pair; pairs the split kernel wrote whole return at once.
//
// A pair's partial output of split v is G*D contiguous floats (slot v + pair,
// or 4 * (v + group) + head in group when the split kernel ran head groups).
// The threads form kS groups of kT = G*D/4 threads: thread (grp, t) takes the
// 16-byte piece t of splits w0 + grp, w0 + grp + kS, ..., with each split's
// (max, sum) for the piece's head, and folds them in split order into its own
// online-softmax state; all of a round's loads (kRound splits of the pair) are
// issued before the first is used, so a pair of up to kRound splits costs one
// round trip after the split range is known.  The kS states are then combined
// in group order through LDS.  Every order is fixed: results are bitwise
// reproducible.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeArgs a) {
    constexpr int kO = G * D;                     // outputs of a pair
    constexpr int kT = kO / 4;                    // threads covering one split's partial
    constexpr int kS = kThreads / kT > 0 ? kThreads / kT : 1;   // split groups
    constexpr int kIter = 32 / kS > 16 ? 16 : (32 / kS > 0 ? 32 / kS : 1);   // splits per thread a round
    constexpr int kRound = kS * kIter;            // splits of the pair a round
    constexpr int kPasses = (kT + kThreads - 1) / kThreads;     // pieces per thread (G*D > 1024)
    static_assert(kO % 4 == 0, "pieces of 4 outputs");

    const int lane = threadIdx.x & (kWave - 1);
    // (sequence, KV head) pairs per sequence: virtual heads when a large
    // query group is cut into several (each re-reads its KV head's rows).
    const int Hkv = a.num_kv_heads * a.kv_split;
    const int s = blockIdx.x / Hkv;
    const int g = blockIdx.x % Hkv;
    const int L = uniform(clamped_len(a, s));
    const size_t out_row0 = (static_cast<size_t>(s) * a.num_q_heads + g * G) * D;
    if (L == 0) {
        for (int o = threadIdx.x; o < kO; o += kThreads) a.out[out_row0 + o] = 0;
        return;
    }
    const int nch = chunks_of(L);
    // Chunks before this pair, and in total.
    int64_t before = 0, total = 0;
    for (int b0 = 0; b0 < a.num_seqs; b0 += kWave) {
        const int sl = b0 + lane;
        const int64_t n = sl < a.num_seqs ? chunks_of(clamped_len(a, sl)) : 0;
        total += wave_sum64(n);
        before += wave_sum64(sl < s ? n : 0);
    }
    const int64_t U = uniform64(total) * Hkv;
    const int N = splits_in_use(a, U, lane);
    // The pair's entries in the list: first, first + step, ... (nch of them);
    // in the head-group order (decided as in the split kernel, per sequence)
    // a group's 4 heads interleave chunk by chunk.
    const bool hg_mode = a.head_groups && U >= 4 * static_cast<int64_t>(N);
    const bool hgs = hg_mode && 4 * static_cast<int64_t>(nch) * N <= 30 * U;
    const int64_t step = hgs ? 4 : 1;
    const int64_t first = uniform64(before) * Hkv +
                          (hgs ? static_cast<int64_t>(g & ~3) * nch + (g & 3) : static_cast<int64_t>(g) * nch);
    const int w0 = owner_of(first, U, N);
    const int w1 = owner_of(first + step * (nch - 1), U, N);
    if (w0 == w1) return;                         // written whole by the split kernel
    const int P = w1 - w0 + 1;
    const bool may_be_empty = U < N;              // some splits then hold no chunk
    auto empty_split = [&](int64_t v) { return v * U / N == (v + 1) * U / N; };
    const size_t pair = static_cast<size_t>(s) * Hkv + g;
    // Partial slot of split v: v + pair, or, with head groups allowed (in
    // either order), 4 * (v + group) + head in group.
    auto slot_of = [&](int64_t v) -> size_t {
        return hg_mode ? 4 * (static_cast<size_t>(v) + static_cast<size_t>(s) * (Hkv / 4) + (g >> 2)) + (g & 3)
                       : static_cast<size_t>(v) + pair;
    };

    __shared__ float s_m[kS][kT], s_l[kS][kT];
    __shared__ float4 s_o[kS][kT];
    for (int pass = 0; pass < kPasses; ++pass) {
        const int idx = threadIdx.x + pass * kThreads;
        const int grp = kS > 1 ? idx / kT : 0;
        const int t = idx % kT;                   // piece: outputs 4t .. 4t+3
        const bool on = idx < kS * kT;
        const int h = (4 * t) / D;
        float m = kNegBig, l = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r0 = 0; r0 < P; r0 += kRound) {
            float4 po[kIter];
            float2 pml[kIter];
    #pragma unroll
            for (int k = 0; k < kIter; ++k) {
                const int i = r0 + grp + k * kS;  // split w0 + i
                const int64_t v = w0 + i;
                const bool live = on && i < P && (!may_be_empty || !empty_split(v));
                po[k] = make_float4(0.f, 0.f, 0.f, 0.f);
                pml[k] = make_float2(-__builtin_inff(), 0.f);
                if (live) {
                    const size_t slot = slot_of(v);
                    po[k] = *reinterpret_cast<const float4*>(a.part_o + slot * kO + 4 * t);
                    pml[k] = *reinterpret_cast<const float2*>(a.part_ml + (slot * G + h) * 2);
                }
            }
            float mr = m;
    #pragma unroll
            for (int k = 0; k < kIter; ++k) mr = __builtin_fmaxf(mr, pml[k].x);
            const float sc = fast_exp2(m - mr);
            l *= sc;
            o.x *= sc;
            o.y *= sc;
            o.z *= sc;
            o.w *= sc;
    #pragma unroll
            for (int k = 0; k < kIter; ++k) {
                // An absent split has max -inf: weight 0 and zero partials.
                const float f = pml[k].x == -__builtin_inff() ? 0.f : fast_exp2(pml[k].x - mr);
                l = __builtin_fmaf(f, pml[k].y, l);
                o.x = __builtin_fmaf(f, po[k].x, o.x);
                o.y = __builtin_fmaf(f, po[k].y, o.y);
                o.z = __builtin_fmaf(f, po[k].z, o.z);
                o.w = __builtin_fmaf(f, po[k].w, o.w);
            }
            m = mr;
        }
        if (on) {
            s_m[grp][t] = m;
            s_l[grp][t] = l;
            s_o[grp][t] = o;
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < kT; t += kThreads) {
        float mm = s_m[0][t];
    #pragma unroll
        for (int grp = 1; grp < kS; ++grp) mm = __builtin_fmaxf(mm, s_m[grp][t]);
        float den = 0.f;
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    #pragma unroll
        for (int grp = 0; grp < kS; ++grp) {
            const float f = s_m[grp][t] == kNegBig && s_l[grp][t] == 0.f ? 0.f : fast_exp2(s_m[grp][t] - mm);
            den = __builtin_fmaf(f, s_l[grp][t], den);
            num.x = __builtin_fmaf(f, s_o[grp][t].x, num.x);
            num.y = __builtin_fmaf(f, s_o[grp][t].y, num.y);
            num.z = __builtin_fmaf(f, s_o[grp][t].z, num.z);
            num.w = __builtin_fmaf(f, s_o[grp][t].w, num.w);
        }
        const float r[4] = {num.x, num.y, num.z, num.w};
        uint16_t hv[4];
    #pragma unroll
        for (int e = 0; e < 4; ++e)
            hv[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(den == 0.f ? 0.f : r[e] / den));
        *reinterpret_cast<uint2*>(a.out + out_row0 + 4 * t) =
            make_uint2(hv[0] | (static_cast<uint32_t>(hv[1]) << 16), hv[2] | (static_cast<uint32_t>(hv[3]) << 16));
    }
}

// Matrix cores take groups of 3 to 8 query heads (blocks of 8 tokens or
// more); the vector kernel takes groups of 1 and 2.
template <int BS, int G>
constexpr bool use_mfma() { return (BS >= kChunk || 2 * BS == kChunk) && G >= 3 && G <= 8; }

template <int D, int BS, int G>
constexpr auto split_kernel() {
    if constexpr (use_mfma<BS, G>()) return decode_mfma_kernel<D, BS, G>;
    else return decode_split_kernel<D, BS, G>;
}

template <int D, int BS, int G>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((split_kernel<D, BS, G>()), dim3(a.num_splits), dim3(kThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.whole_pairs) return err;
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(a.num_seqs * a.num_kv_heads * a.kv_split), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

// Workgroups of decode_split_kernel<D, BS, G> the current device holds at
// once (occupancy x compute units), cached per device; 0 if unknown.
template <int D, int BS, int G>
int resident_one() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_kernel<D, BS, G>(),
                                                     kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    // The matrix-core kernel runs 3 workgroups a CU (its register budget;
    // 4 had streamed slower: 4 x 131072-token contexts 342 vs 370 us a call).
    // The vector kernel for 1 or 2 query heads a KV head fits 4 but streams
    // faster on 2 (32 x 2048 tokens, 32/32 heads: 171 vs 178.5 us a call;
    // mixed lengths 362 vs 366); for 4 or more (blocks of 8) it keeps what fits
    // (4 x 131072 tokens at block 8: 3 a CU, 362 vs 380 us on 2).
    if (use_mfma<BS, G>() && per_cu > 3) per_cu = 3;
    if (!use_mfma<BS, G>() && G <= 2 && per_cu > 2) per_cu = 2;
    v = per_cu * cus;
    if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int D, int BS>
int resident_group(int group) {
    switch (group) {
        case 1: return resident_one<D, BS, 1>();
        case 2: return resident_one<D, BS, 2>();
        case 3: return resident_one<D, BS, 3>();
        case 4: return resident_one<D, BS, 4>();
        case 5: return resident_one<D, BS, 5>();
        case 6: return resident_one<D, BS, 6>();
        case 7: return resident_one<D, BS, 7>();
        case 8: return resident_one<D, BS, 8>();
        default: return 0;
    }
}

template <int D>
int resident_block(int block_size, int group) {
    switch (block_size) {
        case 8: return resident_group<D, 8>(group);
        case 16: return resident_group<D, 16>(group);
        case 32: return resident_group<D, 32>(group);
        case 64: return resident_group<D, 64>(group);
        default: return 0;
    }
}

template <int D, int BS>
hipError_t dispatch_group(const DecodeArgs& a, hipStream_t stream) {
    switch (a.num_q_heads / (a.num_kv_heads * a.kv_split)) {
        case 1: return launch_one<D, BS, 1>(a, stream);
        case 2: return launch_one<D, BS, 2>(a, stream);
        case 3: return launch_one<D, BS, 3>(a, stream);
        case 4: return launch_one<D, BS, 4>(a, stream);
        case 5: return launch_one<D, BS, 5>(a, stream);
        case 6: return launch_one<D, BS, 6>(a, stream);
        case 7: return launch_one<D, BS, 7>(a, stream);
        case 8: return launch_one<D, BS, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t dispatch_block(const DecodeArgs& a, hipStream_t stream) {
    switch (a.block_size) {
        case 8: return dispatch_group<D, 8>(a, stream);
        case 16: return dispatch_group<D, 16>(a, stream);
        case 32: return dispatch_group<D, 32>(a, stream);
        case 64: return dispatch_group<D, 64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

GroupSplit decode_group_split(int group) {
    // Groups of up to 8 query heads run as they are; a larger group is cut
    // into kv_split equal groups of its largest divisor not above 8.
    if (group <= 8) return {group, 1};
    int g = 8;
    while (group % g != 0) --g;
    return {g, group / g};
}

bool decode_head_groups_ok(int block_size, int group, int virtual_kv_heads) {
    return block_size >= kChunk && group >= 3 && group <= 8 && virtual_kv_heads % 4 == 0;
}

bool decode_supported(int head_dim, int block_size, int group) {
    const bool d_ok = head_dim == 64 || head_dim == 128;
    const bool b_ok = block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
    const bool g_ok = group >= 1 && group <= 8;      // larger groups are cut into these
    return d_ok && b_ok && g_ok;
}

int decode_compute_units() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

int decode_resident_workgroups(int head_dim, int block_size, int group) {
    if (head_dim == 128) return resident_block<128>(block_size, group);
    if (head_dim == 64) return resident_block<64>(block_size, group);
    return 0;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.head_dim == 128) return dispatch_block<128>(a, stream);
    if (a.head_dim == 64) return dispatch_block<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa

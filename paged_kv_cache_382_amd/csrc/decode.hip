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
// Design (HBM-bound streaming; no matrix cores: G <= 8 query rows never fill
// an MFMA tile):
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
//    chunk order, either w or pair grows at each segment start), and the merge
//    kernel combines the slots of workgroups first(pair) .. last(pair).
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
//    ragged last chunk rides the same pipeline where that costs no registers
//    (one block per chunk, G <= 4): its block's buffer range ends at the
//    context's last token, so the rows past it read as zeros and are never
//    fetched.
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
// Occupancy (waves per SIMD) the register allocator may trade down to while
// keeping two chunks of K and V in registers: 4 waves (128 VGPRs) for 1-2
// query heads per KV head, 3 (168) for 4, 2 (256) for 8.
template <int G>
constexpr int waves_per_simd() { return G <= 2 ? 4 : (G == 4 ? 3 : 2); }
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

template <int D>
struct Geometry {
    static constexpr int LPR = D / 8;            // lanes per token row
    static constexpr int RPL = kWave / LPR;      // token rows per wave load
    static constexpr int LPC = kChunk / RPL;     // loads per chunk (K or V)
};

template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_simd<G>())))
void decode_split_kernel(const DecodeArgs a) {
    using Geo = Geometry<D>;
    constexpr int LPR = Geo::LPR;
    constexpr int RPL = Geo::RPL;
    constexpr int LPC = Geo::LPC;
    constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;   // blocks per chunk
    constexpr int kPerBlock = LPC / BPC;                  // granules of a chunk per block
    static_assert(BS % RPL == 0, "a load must not straddle two blocks");
    // The pair's ragged last chunk goes through the load pipeline (its rows
    // past the context read as zeros through a shortened buffer range) where
    // that costs no registers: one block per chunk and G <= 4.  Otherwise it
    // is loaded after the pipeline and its rows are dropped in registers.
    constexpr bool kFold = BS >= kChunk && G <= 4;

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = uniform(threadIdx.x / kWave);
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int Hkv = a.num_kv_heads;
    const int N = a.num_splits;

    // Bytes from one token's row of a KV head to the next token's: a whole slot
    // (slot-major) or one head row (head-major).
    const uint32_t row_bytes = a.head_major ? D * 2 : static_cast<uint32_t>(Hkv) * D * 2;
    const uint32_t block_bytes = static_cast<uint32_t>(Hkv) * D * 2 * BS;
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
            const size_t head_off = static_cast<size_t>(g) * D * 2 * (a.head_major ? BS : 1);
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

// Merge the partials of pairs that span several splits, and write the zero
// rows of empty contexts.  One workgroup of 4 waves per (sequence, KV head)
// pair; pairs the split kernel wrote whole return at once.
//
// A pair's partial output of split v is G*D contiguous floats (slot v + pair).
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
    const int Hkv = a.num_kv_heads;
    const int N = a.num_splits;
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
    const int64_t first = uniform64(before) * Hkv + static_cast<int64_t>(g) * nch;
    const int w0 = owner_of(first, U, N);
    const int w1 = owner_of(first + nch - 1, U, N);
    if (w0 == w1) return;                         // written whole by the split kernel
    const int P = w1 - w0 + 1;
    const bool may_be_empty = U < N;              // some splits then hold no chunk
    auto empty_split = [&](int64_t v) { return v * U / N == (v + 1) * U / N; };
    const size_t pair = static_cast<size_t>(s) * Hkv + g;

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
                    const size_t slot = static_cast<size_t>(v) + pair;
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

template <int D, int BS, int G>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<D, BS, G>), dim3(a.num_splits), dim3(kThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.whole_pairs) return err;
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), dim3(a.num_seqs * a.num_kv_heads), dim3(kThreads), 0,
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, BS, G>,
                                                     kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    v = per_cu * cus;
    if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <int D, int BS>
int resident_group(int group) {
    switch (group) {
        case 1: return resident_one<D, BS, 1>();
        case 2: return resident_one<D, BS, 2>();
        case 4: return resident_one<D, BS, 4>();
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
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_one<D, BS, 1>(a, stream);
        case 2: return launch_one<D, BS, 2>(a, stream);
        case 4: return launch_one<D, BS, 4>(a, stream);
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

bool decode_supported(int head_dim, int block_size, int group) {
    const bool d_ok = head_dim == 64 || head_dim == 128;
    const bool b_ok = block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
    const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
    return d_ok && b_ok && g_ok;
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

// Chunked-prefill attention over the block-paged KV cache, on MFMA.
//
// Sources (cited by page title):
//  * "Deep dive into the nano-vLLM inference engine architecture:
//    PagedAttention memory management", section "Deployable configuration
//    parameters": prompts are prefilled in chunks (256 tokens).
//  * "vLLM core architecture ...", section 3 ("Continuous batching"): one
//    batch carries the prefill of several requests of different lengths.
//  * "Deep analysis of nano-vLLM's paged KV cache ...", section
//    "Engineering: configuration and monitoring": prefill attention is a
//    variable-length routine whose plain fallback is standard attention.
//
// What is computed: query row j of sequence s's chunk (n_s rows, the last
// n_s tokens of its L_s-token context, already in the cache) attends to
// logical positions 0 .. L_s - n_s + j through the block table.
//
// Design.  The packed query rows of one (sequence, KV head) are r = j*G + h'
// (token-major, then the G query heads that share the KV head), so grouped
// heads become extra rows of one contraction and every K/V row read from HBM
// serves all G heads.  A workgroup of kWaves waves owns 32*kNT*kWaves rows,
// 32*kNT a wave.  For each tile of KT keys:
//   * the workgroup brings the tile's K and V rows into LDS: with blocks of
//     16 tokens or more straight from HBM (prefill_lds_kernel, below: loads
//     that write LDS, three stages, V in row order); with smaller blocks
//     through registers (prefill_kernel: K rows padded to D*2+16 bytes, V
//     transposed, [d][slot], slot = key with bits 2 and 3 swapped, two LDS
//     buffers, tile t+2's loads in flight and tile t+3's block ids being
//     fetched); one barrier per tile either way;
//   * each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_f16 (A = K from
//     LDS, B = Q held in registers), so that a lane owns one query row
//     (column l % 32) and 16 keys of each 32-key sub-tile;
//   * online softmax in the exp2 domain per lane; the running reference
//     max only moves when a row's max exceeds it by more than kSlack (any
//     reference gives the same normalised result, so the 64-register output
//     rescale is rare);
//   * O^T += V^T P^T with the probabilities taken straight from the S^T
//     accumulators as the B operand: accumulator register r of a 32-key
//     sub-tile holds key (r/4)*8 + 4*(l/32) + r%4, which is MFMA k-slot
//     8*(l/32) + r%8 of k-step r/8 once V's keys are read in that order
//     (stored so in the register-staged kernel, picked so by the transposing
//     reads in the other).
// Keys past the context or behind an out-of-range table entry contribute no
// value: their V rows are zero (the register-staged kernel reads slot 0 of the
// cache for them, a safe address, and zeroes the V rows when staging; the
// other loads them through a buffer range that ends before them); keys past
// the context are also behind every row's causal limit, so their scores are
// masked.
// The output is normalised once and rounded to fp16 (round to nearest even).

#include <type_traits>

#include "kernels.h"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ constexpr h2 kOnes2 = {1.0f16, 1.0f16};

constexpr float kNegBig = -1e30f;
// Word 3 of a gfx9-family buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
constexpr float kSlack = 8.0f;        // log2 units: probabilities stay below 2^8

// Key position inside a 32-key group -> its column in the transposed V tile.
__device__ __forceinline__ int v_slot(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// The two halves of a wave hold different keys of the same query rows (lane l
// and lane l ^ 32 share row l % 32): every lane receives both halves' values
// of its row, swapped across the halves by v_permlane32_swap.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __builtin_bit_cast(float, static_cast<unsigned>(r[0]));
    b = __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}

// XCD-aware order: consecutive work items (the row tiles of one sequence and
// KV head) go to workgroups that the dispatcher places on the same XCD, so
// they share that XCD's L2 copy of the K/V rows.
__device__ __forceinline__ int work_item(int b, int grid) {
    const int per_xcd = grid >> 3;                   // grid is a multiple of 8
    return (b & 7) * per_xcd + (b >> 3);
}

template <int D, int KT, int kWaves, int kNT, bool kOff32>
__global__ __launch_bounds__(kWaves * 64) void prefill_kernel(PrefillArgs a) {
    constexpr int kThreads = kWaves * 64;
    constexpr int kRowsWave = 32 * kNT;               // query rows of one wave
    constexpr int kRowsWG = kRowsWave * kWaves;
    constexpr int kKRow = D * 2 + 16;                 // bytes per K row in LDS
    constexpr int kVRow = KT * 2 + 16;                // bytes per V^T row in LDS
    constexpr int kChunks = D / 8;                    // 16-byte pieces of a row
    constexpr int kKPieces = KT * kChunks;
    constexpr int kVPieces = KT / 2 * kChunks;        // (key pair, piece) units
    constexpr int kKLoads = (kKPieces + kThreads - 1) / kThreads;
    constexpr int kVLoads = (kVPieces + kThreads - 1) / kThreads;
    constexpr int kSub = KT / 32;                     // 32-key sub-tiles per tile
    constexpr int kDT = D / 32;                       // 32-wide output column tiles
    constexpr int kQS = D / 16;                       // k-steps of the QK contraction
    constexpr int kKBytes = KT * kKRow;
    constexpr int kBuf = kKBytes + D * kVRow;         // one K + V^T stage
    static_assert(kKPieces % 64 == 0 && kVPieces % 64 == 0, "whole waves per load slot");
    __shared__ __align__(16) unsigned char lds[2 * kBuf];

    const int G = a.num_q_heads / a.num_kv_heads;
    const int items = a.num_seqs * a.num_kv_heads * a.tiles_per_seq;
    const int item = work_item(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const int tile = item % a.tiles_per_seq;
    const int sg = item / a.tiles_per_seq;
    const int g = sg % a.num_kv_heads;
    const int s = sg / a.num_kv_heads;

    const int qs = a.query_start[s];
    if (qs < 0 || qs > a.num_tokens) return;
    int L = a.context_lens[s];
    L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
    int n = a.query_start[s + 1] - qs;
    n = n < 0 ? 0 : (n > L ? L : n);
    n = n > a.num_tokens - qs ? a.num_tokens - qs : n;
    const int rows = n * G;
    const int row0 = tile * kRowsWG;
    if (row0 >= rows) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m = lane & 31;
    const int hi = lane >> 5;
    const int first = L - n;                          // position of chunk row 0

    const int w_row_lo = row0 + wave * kRowsWave;
    const bool wave_on = w_row_lo < rows;
    const int w_row_hi = min(w_row_lo + kRowsWave - 1, rows - 1);
    const int w_pos_lo = first + w_row_lo / G;
    const int w_pos_hi = first + w_row_hi / G;
    const int n_keys = first + (min(row0 + kRowsWG, rows) - 1) / G + 1;
    const int n_tiles = (n_keys + KT - 1) / KT;

    // Rows of this lane (one per 32-row group) and their Q^T operands.
    int row_tok[kNT], row_head[kNT], row_pos[kNT];
    bool row_ok[kNT];
    h8 qv[kNT][kQS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int r = w_row_lo + 32 * nt + m;
        row_ok[nt] = r < rows;
        const int re = row_ok[nt] ? r : rows - 1;
        const int jj = re / G;
        row_tok[nt] = qs + jj;
        row_head[nt] = g * G + (re - jj * G);
        row_pos[nt] = first + jj;
        const _Float16* qp = reinterpret_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(row_tok[nt]) * a.num_q_heads + row_head[nt]) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < kQS; ++ks) qv[nt][ks] = *reinterpret_cast<const h8*>(qp + 16 * ks);
    }

    const int bshift = a.block_shift;
    const int bmask = (1 << bshift) - 1;
    const int* table = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
    const uint32_t row_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;   // bytes per slot
    // Bytes from one token's row of a KV head to the next token's inside a
    // block (a whole slot, or one head row when head-major), and head g's first
    // row in a block.
    const uint32_t tok_bytes = a.head_major ? D * 2 : row_bytes;
    const size_t head_off = static_cast<size_t>(g) * D * (a.head_major ? a.block_size : 1);
    const uint16_t* kbase = a.k_cache + head_off;
    const uint16_t* vbase = a.v_cache + head_off;

    // This thread's fixed key offsets inside a tile: K piece slots and V pairs.
    int koff[kKLoads], kpiece[kKLoads], voff[kVLoads], vpiece[kVLoads];
#pragma unroll
    for (int u = 0; u < kKLoads; ++u) {
        const int idx = min(tid + u * kThreads, kKPieces - 1);
        koff[u] = idx / kChunks;
        kpiece[u] = idx % kChunks;
    }
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) {
        const int idx = min(tid + u * kThreads, kVPieces - 1);
        voff[u] = 2 * (idx % (KT / 2));
        vpiece[u] = idx / (KT / 2);
    }

    // Block ids of the tile after the one being loaded (one tile ahead).
    int kblk[kKLoads], vblk[kVLoads][2];
    auto fetch_ids = [&](int k0) {
#pragma unroll
        for (int u = 0; u < kKLoads; ++u) {
            const int key = k0 + koff[u];
            kblk[u] = key < L ? table[key >> bshift] : -1;
        }
#pragma unroll
        for (int u = 0; u < kVLoads; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = k0 + voff[u] + e;
                vblk[u][e] = key < L ? table[key >> bshift] : -1;
            }
    };
    // Address of 16-byte piece `piece` of (key, this KV head); a key that holds
    // no token reads piece `piece` of slot 0 instead.  When every offset of the
    // cache fits in 32 bits the address is a uniform base plus a 32-bit offset
    // (scalar-base loads, no 64-bit vector arithmetic).
    auto piece_ptr = [&](const uint16_t* base, bool ok, int b, int key, int piece) -> const u4* {
        if constexpr (kOff32) {
            const uint32_t off = (ok ? (static_cast<uint32_t>(b) << bshift) * row_bytes +
                                           static_cast<uint32_t>(key & bmask) * tok_bytes : 0u) +
                                 16u * piece;
            return reinterpret_cast<const u4*>(reinterpret_cast<const unsigned char*>(base) + off);
        } else {
            const size_t off = ok ? (static_cast<size_t>(b) << bshift) * row_bytes +
                                        static_cast<size_t>(key & bmask) * tok_bytes : 0;
            return reinterpret_cast<const u4*>(reinterpret_cast<const unsigned char*>(base) + off + 16u * piece);
        }
    };
    // Global loads of one tile into registers; the V pieces of keys that hold
    // no token are zeroed when staged.
    u4 kreg[kKLoads], vreg[kVLoads][2];
    unsigned vvalid = 0;
    auto issue_tile = [&](int k0) {
#pragma unroll
        for (int u = 0; u < kKLoads; ++u) {
            const int key = k0 + koff[u];
            const int b = kblk[u];
            const bool ok = b >= 0 && b < a.num_blocks;
            kreg[u] = *piece_ptr(kbase, ok, b, key, kpiece[u]);
        }
        vvalid = 0;
#pragma unroll
        for (int u = 0; u < kVLoads; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = k0 + voff[u] + e;
                const int b = vblk[u][e];
                const bool ok = b >= 0 && b < a.num_blocks;
                vreg[u][e] = *piece_ptr(vbase, ok, b, key, vpiece[u]);
                vvalid |= (ok ? 1u : 0u) << (2 * u + e);
            }
    };
    auto stage_tile = [&](unsigned char* buf) {
#pragma unroll
        for (int u = 0; u < kKLoads; ++u)
            if (tid + u * kThreads < kKPieces)
                *reinterpret_cast<u4*>(buf + koff[u] * kKRow + kpiece[u] * 16) = kreg[u];
        unsigned char* vt = buf + kKBytes;
#pragma unroll
        for (int u = 0; u < kVLoads; ++u) {
            if (tid + u * kThreads >= kVPieces) continue;
            const int col = (voff[u] & ~31) + v_slot(voff[u] & 31);
            unsigned char* base = vt + (8 * vpiece[u]) * kVRow + col * 2;
            const bool ok0 = (vvalid >> (2 * u)) & 1u, ok1 = (vvalid >> (2 * u + 1)) & 1u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned w0 = ok0 ? vreg[u][0][i] : 0u;
                const unsigned w1 = ok1 ? vreg[u][1][i] : 0u;
                // dims 8c + 2i and 8c + 2i + 1, keys (key, key + 1)
                *reinterpret_cast<unsigned*>(base + (2 * i) * kVRow) = (w0 & 0xFFFFu) | (w1 << 16);
                *reinterpret_cast<unsigned*>(base + (2 * i + 1) * kVRow) = (w0 >> 16) | (w1 & 0xFFFF0000u);
            }
        }
    };

    f16x acc_o[kNT][kDT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc_o[nt][dt][r] = 0.0f;
    float m_ref[kNT], l_sum[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        m_ref[nt] = kNegBig;                          // reference max (log2 units)
        l_sum[nt] = 0.0f;                             // this half-wave's keys only
    }
    const float c_log2 = a.scale_log2;

    // Prologue: stage tile 0, put tile 1 in flight, fetch the ids of tile 2.
    fetch_ids(0);
    issue_tile(0);
    fetch_ids(KT);
    stage_tile(lds);
    if (n_tiles > 1) issue_tile(KT);
    fetch_ids(2 * KT);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int k0 = t * KT;
        const unsigned char* kt = lds + (t & 1) * kBuf;
        const unsigned char* vt = kt + kKBytes;
        if (wave_on && k0 <= w_pos_hi) {
            // S^T = K Q^T: each K operand feeds kNT products.
            f16x sacc[kNT][kSub];
            // All K operands of the tile are read from LDS before the first
            // product, and all V operands right after the last one, so the LDS
            // latency is paid once a tile and the V reads overlap the softmax.
            h8 kop[kSub][kQS];
#pragma unroll
            for (int st = 0; st < kSub; ++st)
#pragma unroll
                for (int ks = 0; ks < kQS; ++ks)
                    kop[st][ks] = *reinterpret_cast<const h8*>(kt + (32 * st + m) * kKRow + 16 * hi + 32 * ks);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < kSub; ++st)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[nt][st][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < kQS; ++ks)
#pragma unroll
                for (int st = 0; st < kSub; ++st)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt)
                        sacc[nt][st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[st][ks], qv[nt][ks], sacc[nt][st], 0, 0, 0);
            h8 vop[kDT][2 * kSub];
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int ks = 0; ks < 2 * kSub; ++ks)
                    vop[dt][ks] = *reinterpret_cast<const h8*>(vt + (32 * dt + m) * kVRow + 16 * hi + 32 * ks);
            __builtin_amdgcn_sched_barrier(0);
            const bool need_mask = k0 + KT - 1 > w_pos_lo;
            h8 pb[kNT][2 * kSub];
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                if (need_mask) {
#pragma unroll
                    for (int st = 0; st < kSub; ++st)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + 32 * st + (r >> 2) * 8 + 4 * hi + (r & 3);
                            if (key > row_pos[nt]) sacc[nt][st][r] = kNegBig;
                        }
                }
                float mv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) mv[i] = kNegBig;
#pragma unroll
                for (int st = 0; st < kSub; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mv[r & 7] = fmaxf(mv[r & 7], sacc[nt][st][r]);
                float mx = fmaxf(fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])),
                                 fmaxf(fmaxf(mv[4], mv[5]), fmaxf(mv[6], mv[7])));
                {
                    float ma, mb;
                    halves(mx, ma, mb);
                    mx = fmaxf(ma, mb) * c_log2;
                }
                const bool grow = mx > m_ref[nt] + kSlack;
                if (__ballot(grow)) {
                    const float m_new = grow ? mx : m_ref[nt];
                    const float alpha = __builtin_amdgcn_exp2f(m_ref[nt] - m_new);
                    m_ref[nt] = m_new;
                    l_sum[nt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc_o[nt][dt][r] *= alpha;
                }
                // probabilities -> fp16 B operands, k-step = (sub-tile, half)
#pragma unroll
                for (int st = 0; st < kSub; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nt][st][r], c_log2, -m_ref[nt]));
                        pb[nt][2 * st + (r >> 3)][r & 7] = static_cast<_Float16>(p);
                    }
            }
            // row sums of the fp16 probabilities the products use
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int ks = 0; ks < 2 * kSub; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const h2 pp = {pb[nt][ks][2 * e], pb[nt][ks][2 * e + 1]};
                        l_sum[nt] = __builtin_amdgcn_fdot2(pp, kOnes2, l_sum[nt], false);
                    }
            // O^T += V^T P^T: each V operand feeds kNT products.
#pragma unroll
            for (int ks = 0; ks < 2 * kSub; ++ks)
#pragma unroll
                for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                    for (int nt = 0; nt < kNT; ++nt)
                        acc_o[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[dt][ks], pb[nt][ks], acc_o[nt][dt], 0, 0, 0);
        }
        // Stage tile t+1 into the other buffer (last read before the previous
        // barrier), put tile t+2 in flight, fetch the ids of tile t+3.
        if (t + 1 < n_tiles) {
            stage_tile(lds + ((t + 1) & 1) * kBuf);
            if (t + 2 < n_tiles) {
                issue_tile(k0 + 2 * KT);
                fetch_ids(k0 + 3 * KT);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        float la, lb;
        halves(l_sum[nt], la, lb);
        const float l_tot = la + lb;
        if (!row_ok[nt]) continue;
        const float inv = 1.0f / l_tot;
        _Float16* op = reinterpret_cast<_Float16*>(a.out) +
                       (static_cast<size_t>(row_tok[nt]) * a.num_q_heads + row_head[nt]) * D + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                h4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = static_cast<_Float16>(acc_o[nt][dt][4 * rq + i] * inv);
                *reinterpret_cast<h4*>(op + 32 * dt + 8 * rq) = o;
            }
    }
}

// Variant for blocks of 16 tokens or more: K and V travel from HBM straight
// into LDS with gfx950's buffer_load ... lds (no register staging, no LDS
// store instructions), and V stays in its natural row order.
//  * A wave's load instruction fills 1 KiB of LDS, lane-contiguous; which
//    global bytes each lane fetches decides the layout:
//      K: instruction (row group rg, piece group pg) holds rows 16 rg .. +15,
//         16-byte pieces 4 pg .. +3, lane L taking row L % 16, piece
//         4 pg + L / 16.  A K operand read (16 rows of one piece) is then 256
//         contiguous bytes, and successive k-steps are 512 bytes apart.
//      V: instruction i holds whole rows (4 at D = 128, 8 at D = 64) in
//         order; slot c of row r holds piece c ^ swz_v(r), which keeps the
//         transposing reads below free of bank conflicts.
//    A wave's instructions cover one 16-token group of a stage, which lies
//    in one cache block: one block id and one buffer resource per matrix,
//    starting at the group's first row and covering only the rows that hold
//    tokens (rows past the keys this workgroup sees, or behind an
//    out-of-range table entry, arrive as zeros); the instructions differ in
//    the scalar offset (which the range check covers) and the LDS address.
//  * The V^T operand of O^T += V^T P^T comes from ds_read_b64_tr_b16, whose
//    16-lane transpose turns 4 rows x 4 columns into each lane's 4 keys of one
//    column, in the key order the P operand needs (key bits 2 and 3 swapped,
//    as in the register-staged kernel's slot order).
//  * Tile t (KT = 64 keys) sits in stage t % 3; the stages are separate LDS
//    arrays so that the compiler's own wait before reading one covers only
//    that stage's loads (the loop is unrolled by three).  Iteration t fetches
//    the block ids of tile t + 3, puts tile t + 2 in flight (into the stage
//    that iteration t - 1 finished reading), computes tile t, and ends at the
//    workgroup barrier once each wave's own loads of tile t + 1 have landed.
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// A buffer resource over `range` bytes at `p`, built from wave-uniform values
// (read from the first lane) so that it lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, uint32_t range) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    void* pu = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(pu, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(range)), kRsrcWord3);
}

typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;
typedef __attribute__((address_space(3))) void lds_void;

template <int S>
struct Stage {};

template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void prefill_lds_kernel(PrefillArgs a) {
    constexpr int KT = 64;                            // keys of a tile
    constexpr int kRowB = D * 2;                      // bytes of a row
    constexpr int kP = D / 8;                         // 16-byte pieces of a row
    constexpr int kPG = kP / 4;                       // K piece groups of a row
    constexpr int kVRows = 64 / kP;                   // rows of one V instruction
    constexpr int kInstTile = KT * kP / 64;           // instructions per matrix and tile
    constexpr int kInst = kInstTile / kWaves;         // of them, per wave
    static_assert(kInst * kWaves == kInstTile && kPG % kInst == 0, "a wave's K instructions in one row group");
    static_assert(kInst * 64 / kP <= 16 && 16 % (kInst * 64 / kP) == 0, "a wave's rows in one 16-token group");
    constexpr int kSub = KT / 32;                     // 32-key sub-tiles of a tile
    constexpr int kDT = D / 32;                       // 32-wide output column tiles
    constexpr int kQS = D / 16;                       // k-steps of the QK contraction
    constexpr int kTileB = KT * kRowB;                // one matrix of one tile
    __shared__ __align__(16) unsigned char st0[2 * kTileB];
    __shared__ __align__(16) unsigned char st1[2 * kTileB];
    __shared__ __align__(16) unsigned char st2[2 * kTileB];

    const int G = a.num_q_heads / a.num_kv_heads;
    const int items = a.num_seqs * a.num_kv_heads * a.tiles_per_seq;
    const int item = work_item(blockIdx.x, gridDim.x);
    if (item >= items) return;
    const int tile = item % a.tiles_per_seq;
    const int sg = item / a.tiles_per_seq;
    const int g = sg % a.num_kv_heads;
    const int s = sg / a.num_kv_heads;

    const int qs = a.query_start[s];
    if (qs < 0 || qs > a.num_tokens) return;
    int L = a.context_lens[s];
    L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
    int n = a.query_start[s + 1] - qs;
    n = n < 0 ? 0 : (n > L ? L : n);
    n = n > a.num_tokens - qs ? a.num_tokens - qs : n;
    const int rows = n * G;
    const int row0 = tile * 32 * kWaves;
    if (row0 >= rows) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 31;
    const int hi = lane >> 5;
    const int first = L - n;                          // position of chunk row 0

    const int w_row_lo = row0 + wave * 32;
    const bool wave_on = w_row_lo < rows;
    const int w_row_hi = min(w_row_lo + 31, rows - 1);
    const int w_pos_lo = first + w_row_lo / G;
    const int w_pos_hi = first + w_row_hi / G;
    // Keys this workgroup's rows see: the loads stop there.
    const int n_keys = __builtin_amdgcn_readfirstlane(first + (min(row0 + 32 * kWaves, rows) - 1) / G + 1);
    const int n_tiles = (n_keys + KT - 1) / KT;

    // This lane's query row and its Q^T operands.
    const int r_q = w_row_lo + m;
    const bool row_ok = r_q < rows;
    const int re = row_ok ? r_q : rows - 1;
    const int jj = re / G;
    const int row_tok = qs + jj;
    const int row_head = g * G + (re - jj * G);
    const int row_pos = first + jj;
    h8 qv[kQS];
    {
        const _Float16* qp = reinterpret_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(row_tok) * a.num_q_heads + row_head) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < kQS; ++ks) qv[ks] = *reinterpret_cast<const h8*>(qp + 16 * ks);
    }
    // Let the Q rows land before the loads of the tile loop are counted (so
    // that no wait inside the loop is for them).
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)

    const int bshift = a.block_shift;
    const int bmask = (1 << bshift) - 1;
    const int* table = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
    const uint32_t tok_bytes = a.head_major ? D * 2 : static_cast<uint32_t>(a.num_kv_heads) * D * 2;
    const size_t block_bytes = static_cast<size_t>(a.block_size) * a.num_kv_heads * D * 2;
    const size_t head_off = static_cast<size_t>(g) * D * 2 * (a.head_major ? a.block_size : 1);
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k_cache) + head_off;
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v_cache) + head_off;
    // Per-lane global offsets of the load instructions (relative to their
    // first row): K row L % 16, piece 4 pg + L / 16; V row L / P, the piece
    // that its slot L % P holds.
    const uint32_t k_lane = static_cast<uint32_t>(lane & 15) * tok_bytes + 16u * (lane >> 4);
    const int v_row = lane / kP;
    const uint32_t v_lane = static_cast<uint32_t>(v_row) * tok_bytes + 16u * ((lane % kP) ^ swz_v<D>(v_row));
    const int inst0 = wave * kInst;                   // this wave's first instruction of a stage

    // Block id of this wave's 16-token group of tile k0 (keys past the
    // workgroup's keys read entry 0, which every table has).
    auto fetch_ids = [&](int k0) __attribute__((always_inline)) -> int {
        const int key = k0 + 16 * (inst0 / kPG);
        return table[key < n_keys ? key >> bshift : 0];
    };
    auto issue_tile = [&](int k0, int ids, unsigned char* stage) __attribute__((always_inline)) {
        int b = __builtin_amdgcn_readfirstlane(ids);
        const bool b_ok = b >= 0 && b < a.num_blocks;
        b = b_ok ? b : 0;
        const size_t blk = static_cast<size_t>(b) * block_bytes;
        const int kkey = k0 + 16 * (inst0 / kPG);
        int kval = n_keys - kkey;
        kval = !b_ok || kval < 0 ? 0 : (kval > 16 ? 16 : kval);
        const int vkey = k0 + kVRows * inst0;
        int vval = n_keys - vkey;
        vval = !b_ok || vval < 0 ? 0 : (vval > kVRows * kInst ? kVRows * kInst : vval);
        const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(
            kbase + blk + static_cast<size_t>(kkey & bmask) * tok_bytes, static_cast<uint32_t>(kval) * tok_bytes);
        const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(
            vbase + blk + static_cast<size_t>(vkey & bmask) * tok_bytes, static_cast<uint32_t>(vval) * tok_bytes);
        const uint32_t k_off = k_lane + 64u * (inst0 % kPG);
#pragma unroll
        for (int u = 0; u < kInst; ++u) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + (inst0 + u) * 1024), 16, k_off, 64 * u, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(stage + kTileB + (inst0 + u) * 1024), 16, v_lane,
                                                     u * kVRows * static_cast<int>(tok_bytes), 0, 0);
        }
    };

    // Fixed per-lane parts of the LDS operand reads, relative to a tile's K
    // and V.
    //  K (A operand of S^T): row 32 st + m, piece 2 ks + hi.
    const uint32_t k_rd = static_cast<uint32_t>((m >> 4) * kPG * 1024 + hi * 256 + (m & 15) * 16);
    //  V (transposing read, as a source lane 16 gg + 4 e + q): row
    //  16 ks + 8 h + 4 (gg / 2) + e, columns 32 dt + 16 (gg % 2) + 4 q .. + 3.
    const int gg = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
    const int v_r = 4 * (gg >> 1) + ve;               // row, less 16 ks + 8 h
    uint32_t v_rd[kDT];
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
        const int piece = 4 * dt + 2 * (gg & 1) + (vq >> 1);
        v_rd[dt] = static_cast<uint32_t>(v_r * kRowB + 16 * (piece ^ swz_v<D>(v_r)) + 8 * (vq & 1));
    }

    f16x acc_o[kDT];
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.0f;
    float m_ref = kNegBig;                            // reference max (log2 units)
    float l_sum = 0.0f;                               // this half-wave's keys only
    const float c_log2 = a.scale_log2;

    // One 64-key half: K rows at kt (row-group layout), V rows at vt.
    f16x sacc[kSub];
    // S^T = K Q^T of the tile whose K rows are at kt.
    auto qk = [&](const unsigned char* kt) __attribute__((always_inline)) {
        h8 kop[kSub][kQS];
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int ks = 0; ks < kQS; ++ks)
                kop[st][ks] = *reinterpret_cast<const h8*>(kt + k_rd + st * 2 * kPG * 1024 + ks * 512);
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[st][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kQS; ++ks)
#pragma unroll
            for (int st = 0; st < kSub; ++st)
                sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[st][ks], qv[ks], sacc[st], 0, 0, 0);
    };
    // Softmax and O^T += V^T P^T of the tile whose V rows are at vt.
    auto rest = [&](const unsigned char* vt, int k0) __attribute__((always_inline)) {
        h8 vop[kDT][2 * kSub];
#pragma unroll
        for (int ks = 0; ks < 2 * kSub; ++ks)
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s4v*)(vt + v_rd[dt] + (16 * ks) * kRowB));
                const s4v up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s4v*)(vt + v_rd[dt] + (16 * ks + 8) * kRowB));
                vop[dt][ks] = __builtin_bit_cast(h8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + KT - 1 > w_pos_lo) {
#pragma unroll
            for (int st = 0; st < kSub; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * st + (r >> 2) * 8 + 4 * hi + (r & 3);
                    if (key > row_pos) sacc[st][r] = kNegBig;
                }
        }
        float mv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mv[i] = kNegBig;
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) mv[r & 7] = fmaxf(mv[r & 7], sacc[st][r]);
        float mx = fmaxf(fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])),
                         fmaxf(fmaxf(mv[4], mv[5]), fmaxf(mv[6], mv[7])));
        {
            float ma, mb;
            halves(mx, ma, mb);
            mx = fmaxf(ma, mb) * c_log2;
        }
        const bool grow = mx > m_ref + kSlack;
        if (__ballot(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_sum *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
        }
        h8 pb[2 * kSub];
#pragma unroll
        for (int st = 0; st < kSub; ++st)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][r], c_log2, -m_ref));
                pb[2 * st + (r >> 3)][r & 7] = static_cast<_Float16>(p);
            }
#pragma unroll
        for (int ks = 0; ks < 2 * kSub; ++ks)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const h2 pp = {pb[ks][2 * e2], pb[ks][2 * e2 + 1]};
                l_sum = __builtin_amdgcn_fdot2(pp, kOnes2, l_sum, false);
            }
#pragma unroll
        for (int ks = 0; ks < 2 * kSub; ++ks)
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt)
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[dt][ks], pb[ks], acc_o[dt], 0, 0, 0);
    };

    // Each wave waits for its own loads of the next tile (at most the loads
    // and id fetch issued after them still outstanding), then the workgroup
    // meets.  The wait is the compiler's own instruction, so that
    // its bookkeeping knows which loads have landed.
    constexpr int kAfter = 2 * kInst + 1;            // id fetch + loads of the tile after
    static_assert(kAfter < 16, "vmcnt field");
    auto wait_and_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | kAfter);
        asm volatile("s_barrier" ::: "memory");
    };
    auto stage_of = [&](auto sc) __attribute__((always_inline)) -> unsigned char* {
        if constexpr (std::is_same<decltype(sc), Stage<0>>::value) return st0;
        else if constexpr (std::is_same<decltype(sc), Stage<1>>::value) return st1;
        else return st2;
    };

    // Prologue: tiles 0 and 1 in flight, the ids of tile 2 fetched between
    // them (every iteration fetches ids before it issues loads, so that
    // waiting for a tile's ids never waits for loads issued after them).
    int ids_next;                                     // ids of tile t + 2
    {
        const int ids0 = fetch_ids(0);
        const int ids1 = fetch_ids(KT);
        issue_tile(0, ids0, st0);
        ids_next = fetch_ids(2 * KT);
        issue_tile(KT, ids1, st1);
        wait_and_barrier();
    }
    auto step = [&](auto cur, auto ahead, int t) __attribute__((always_inline)) {
        const int k0 = t * KT;
        const int ids_new = fetch_ids(k0 + 3 * KT);
        __builtin_amdgcn_sched_barrier(0);
        issue_tile(k0 + 2 * KT, ids_next, stage_of(ahead));
        __builtin_amdgcn_sched_barrier(0);
        ids_next = ids_new;
        if (wave_on && k0 <= w_pos_hi) {
            const unsigned char* sp = stage_of(cur);
            qk(sp);
            rest(sp + kTileB, k0);
        }
        wait_and_barrier();
    };
    for (int t = 0; t < n_tiles; t += 3) {
        step(Stage<0>{}, Stage<2>{}, t);
        if (t + 1 >= n_tiles) break;
        step(Stage<1>{}, Stage<0>{}, t + 1);
        if (t + 2 >= n_tiles) break;
        step(Stage<2>{}, Stage<1>{}, t + 2);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    float la, lb;
    halves(l_sum, la, lb);
    const float l_tot = la + lb;
    if (!row_ok) return;
    const float inv = 1.0f / l_tot;
    _Float16* op = reinterpret_cast<_Float16*>(a.out) +
                   (static_cast<size_t>(row_tok) * a.num_q_heads + row_head) * D + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            h4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = static_cast<_Float16>(acc_o[dt][4 * rq + i] * inv);
            *reinterpret_cast<h4*>(op + 32 * dt + 8 * rq) = o;
        }
}

template <int D, int KT, int kWaves, int kNT>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
    const uint64_t cache_bytes = static_cast<uint64_t>(a.num_blocks) * a.block_size * a.num_kv_heads * D * 2;
    PrefillArgs b = a;
    constexpr int kRowsWG = 32 * kNT * kWaves;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int64_t rows = static_cast<int64_t>(a.max_query_len) * G;
    b.tiles_per_seq = static_cast<int32_t>((rows + kRowsWG - 1) / kRowsWG);
    const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * b.tiles_per_seq;
    if (items == 0) return hipSuccess;
    const int64_t grid = (items + 7) / 8 * 8;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    if (kNT == 1 && a.block_size >= 16)
        hipLaunchKernelGGL((prefill_lds_kernel<D, kWaves>), dim3(static_cast<unsigned>(grid)),
                           dim3(kWaves * 64), 0, stream, b);
    else if (cache_bytes <= UINT32_MAX)
        hipLaunchKernelGGL((prefill_kernel<D, KT, kWaves, kNT, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(kWaves * 64), 0, stream, b);
    else
        hipLaunchKernelGGL((prefill_kernel<D, KT, kWaves, kNT, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(kWaves * 64), 0, stream, b);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int head_dim, int block_size) {
    return (head_dim == 64 || head_dim == 128) && block_size > 0 && (block_size & (block_size - 1)) == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs <= 0 || a.max_query_len <= 0) return hipSuccess;
    switch (a.head_dim) {
        case 128: return launch_t<128, 64, 8, 1>(a, stream);
        case 64: return launch_t<64, 64, 8, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa

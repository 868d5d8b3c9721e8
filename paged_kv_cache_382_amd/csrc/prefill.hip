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
// serves all G heads.  A workgroup of kWaves waves owns 32*kWaves rows, 32 a
// wave.  For each tile of KT keys:
//   * the workgroup stages K (row-major, rows padded to D*2+16 bytes) and V
//     (transposed, [d][slot], slot = key with bits 2 and 3 swapped) in LDS;
//     the next tile's global loads are issued before the current tile is
//     consumed;
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
//     8*(l/32) + r%8 of k-step r/8 once V's keys are stored in slot order.
// The output is normalised once and rounded to fp16 (round to nearest even).

#include "kernels.h"

namespace pa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1e30f;
constexpr float kSlack = 8.0f;        // log2 units: probabilities stay below 2^8

// Key position inside a 32-key group -> its column in the transposed V tile.
__device__ __forceinline__ int v_slot(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

// XCD-aware order: consecutive work items (the row tiles of one sequence and
// KV head) go to workgroups that the dispatcher places on the same XCD, so
// they share that XCD's L2 copy of the K/V rows.
__device__ __forceinline__ int work_item(int b, int grid) {
    const int per_xcd = grid >> 3;                   // grid is a multiple of 8
    return (b & 7) * per_xcd + (b >> 3);
}

template <int D, int KT, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void prefill_kernel(PrefillArgs a) {
    constexpr int kThreads = kWaves * 64;
    constexpr int kRowsWG = 32 * kWaves;
    constexpr int kKRow = D * 2 + 16;                 // bytes per K row in LDS
    constexpr int kVRow = KT * 2 + 16;                // bytes per V^T row in LDS
    constexpr int kChunks = D / 8;                    // 16-byte pieces of a row
    constexpr int kKLoads = (KT * kChunks + kThreads - 1) / kThreads;
    constexpr int kVLoads = (KT / 2 * kChunks + kThreads - 1) / kThreads;
    constexpr int kSub = KT / 32;                     // 32-key sub-tiles per tile
    constexpr int kDT = D / 32;                       // 32-wide output column tiles
    constexpr int kQS = D / 16;                       // k-steps of the QK contraction
    __shared__ __align__(16) unsigned char lds_k[KT * kKRow];
    __shared__ __align__(16) unsigned char lds_v[D * kVRow];

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
    const int my_row = row0 + wave * 32 + m;
    const bool row_ok = my_row < rows;
    const int r_eff = row_ok ? my_row : rows - 1;
    const int j = r_eff / G;
    const int hq = g * G + (r_eff - j * G);
    const int first = L - n;                          // position of chunk row 0
    const int pos = first + j;

    // Key range of this wave and of the whole workgroup.
    const int w_row_lo = row0 + wave * 32;
    const bool wave_on = w_row_lo < rows;
    const int w_row_hi = min(w_row_lo + 31, rows - 1);
    const int w_pos_lo = first + w_row_lo / G;
    const int w_pos_hi = first + w_row_hi / G;
    const int g_pos_hi = first + (min(row0 + kRowsWG, rows) - 1) / G;
    const int n_keys = g_pos_hi + 1;
    const int n_tiles = (n_keys + KT - 1) / KT;

    // Q^T operand: row r_eff, dims 16*ks + 8*hi .. +8.
    h8 qv[kQS];
    {
        const _Float16* qp = reinterpret_cast<const _Float16*>(a.q) +
                             (static_cast<size_t>(qs + j) * a.num_q_heads + hq) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < kQS; ++ks) qv[ks] = *reinterpret_cast<const h8*>(qp + 16 * ks);
    }

    const int bs = a.block_size;
    const int* table = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
    const size_t head_off = static_cast<size_t>(g) * D;
    const size_t slot_stride = static_cast<size_t>(a.num_kv_heads) * D;
    const u4 zero4 = {0u, 0u, 0u, 0u};

    // Global address of (key, 16-byte piece c), or null when the key holds no
    // token (past the context, or an out-of-range table entry).
    auto row_ptr = [&](const uint16_t* cache, int key, int c) -> const u4* {
        if (key >= L) return nullptr;
        const int blk = table[key / bs];
        if (blk < 0 || blk >= a.num_blocks) return nullptr;
        const size_t slot = static_cast<size_t>(blk) * bs + key % bs;
        return reinterpret_cast<const u4*>(cache + slot * slot_stride + head_off + 8 * c);
    };

    u4 kreg[kKLoads];
    u4 vreg[kVLoads][2];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int u = 0; u < kKLoads; ++u) {
            const int idx = tid + u * kThreads;
            kreg[u] = zero4;
            if (idx < KT * kChunks) {
                const u4* p = row_ptr(a.k_cache, k0 + idx / kChunks, idx % kChunks);
                if (p) kreg[u] = *p;
            }
        }
#pragma unroll
        for (int u = 0; u < kVLoads; ++u) {
            const int idx = tid + u * kThreads;
            vreg[u][0] = zero4;
            vreg[u][1] = zero4;
            if (idx < KT / 2 * kChunks) {
                const int kp = idx % (KT / 2);
                const int c = idx / (KT / 2);
                const u4* p0 = row_ptr(a.v_cache, k0 + 2 * kp, c);
                const u4* p1 = row_ptr(a.v_cache, k0 + 2 * kp + 1, c);
                if (p0) vreg[u][0] = *p0;
                if (p1) vreg[u][1] = *p1;
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < kKLoads; ++u) {
            const int idx = tid + u * kThreads;
            if (idx < KT * kChunks)
                *reinterpret_cast<u4*>(lds_k + (idx / kChunks) * kKRow + (idx % kChunks) * 16) = kreg[u];
        }
#pragma unroll
        for (int u = 0; u < kVLoads; ++u) {
            const int idx = tid + u * kThreads;
            if (idx < KT / 2 * kChunks) {
                const int kp = idx % (KT / 2);
                const int c = idx / (KT / 2);
                const int key = 2 * kp;
                const int col = (key & ~31) + v_slot(key & 31);
                unsigned char* base = lds_v + (8 * c) * kVRow + col * 2;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned w0 = vreg[u][0][i], w1 = vreg[u][1][i];
                    // d = 8c + 2i and 8c + 2i + 1: (key, key+1) pairs
                    *reinterpret_cast<unsigned*>(base + (2 * i) * kVRow) =
                        (w0 & 0xFFFFu) | (w1 << 16);
                    *reinterpret_cast<unsigned*>(base + (2 * i + 1) * kVRow) =
                        (w0 >> 16) | (w1 & 0xFFFF0000u);
                }
            }
        }
    };

    f16x acc_o[kDT];
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.0f;
    float m_ref = kNegBig;                            // reference max (log2 units)
    float l_sum = 0.0f;                               // this half-wave's keys only
    const float c_log2 = a.scale_log2;

    load_tile(0);
    for (int t = 0; t < n_tiles; ++t) {
        const int k0 = t * KT;
        store_tile();
        __syncthreads();
        if (t + 1 < n_tiles) load_tile(k0 + KT);

        if (wave_on && k0 <= w_pos_hi) {
            // S^T = K Q^T, one 32x32 accumulator per 32-key sub-tile.
            f16x sacc[kSub];
#pragma unroll
            for (int st = 0; st < kSub; ++st) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[st][r] = 0.0f;
                const unsigned char* kb = lds_k + (32 * st + m) * kKRow + 16 * hi;
#pragma unroll
                for (int ks = 0; ks < kQS; ++ks) {
                    const h8 kv = *reinterpret_cast<const h8*>(kb + 32 * ks);
                    sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv, qv[ks], sacc[st], 0, 0, 0);
                }
            }
            // causal mask where the tile reaches past the wave's first row
            if (k0 + KT - 1 > w_pos_lo) {
#pragma unroll
                for (int st = 0; st < kSub; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * st + (r >> 2) * 8 + 4 * hi + (r & 3);
                        if (key > pos) sacc[st][r] = kNegBig;
                    }
            }
            float mx = kNegBig;
#pragma unroll
            for (int st = 0; st < kSub; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[st][r]);
            mx = fmaxf(mx, xor32(mx)) * c_log2;
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
            // probabilities -> fp16 B operands, k-step = (sub-tile, half)
            h8 pb[2 * kSub];
#pragma unroll
            for (int st = 0; st < kSub; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[st][r], c_log2, -m_ref));
                    l_sum += p;
                    pb[2 * st + (r >> 3)][r & 7] = static_cast<_Float16>(p);
                }
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
                const unsigned char* vb = lds_v + (32 * dt + m) * kVRow + 16 * hi;
#pragma unroll
                for (int ks = 0; ks < 2 * kSub; ++ks) {
                    const h8 vv = *reinterpret_cast<const h8*>(vb + 32 * ks);
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv, pb[ks], acc_o[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    const float l_tot = l_sum + xor32(l_sum);
    if (!row_ok) return;
    const float inv = 1.0f / l_tot;
    _Float16* op = reinterpret_cast<_Float16*>(a.out) +
                   (static_cast<size_t>(qs + j) * a.num_q_heads + hq) * D + 4 * hi;
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

template <int D, int KT, int kWaves>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
    PrefillArgs b = a;
    constexpr int kRowsWG = 32 * kWaves;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int64_t rows = static_cast<int64_t>(a.max_query_len) * G;
    b.tiles_per_seq = static_cast<int32_t>((rows + kRowsWG - 1) / kRowsWG);
    const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * b.tiles_per_seq;
    if (items == 0) return hipSuccess;
    const int64_t grid = (items + 7) / 8 * 8;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<D, KT, kWaves>), dim3(static_cast<unsigned>(grid)),
                       dim3(kWaves * 64), 0, stream, b);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs <= 0 || a.max_query_len <= 0) return hipSuccess;
    switch (a.head_dim) {
        case 128: return launch_t<128, 32, 4>(a, stream);
        case 64: return launch_t<64, 64, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa

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
//    the fallback), and section 3 of the vLLM page ties decode speed to
//    memory bandwidth.
//
// What is computed, per sequence s and query head h (KV head g = h / G):
//   out[s][h] = sum_p softmax_p(scale * q[s][h] . K[s,p,g]) V[s,p,g]
// with K/V row p found in physical block table[s][p / BS], row p % BS.
//
// Design (HBM-bound streaming, no matrix cores: G <= 8 query rows never fill
// an MFMA tile):
//  * Work item = (sequence, split-K partition of T tokens, KV head); one
//    workgroup of 4 wave64s per item.  The G query heads sharing the KV head
//    live in registers, so every K/V byte is fetched from HBM once.
//  * Within a partition, 16-token chunks are dealt round-robin to the 4
//    waves.  A K (or V) row of D fp16 is D/8 lanes x 16 bytes, so one
//    global_load_dwordx4 per lane covers 64/(D/8) whole rows (1 KiB per wave
//    instruction, fully coalesced).
//  * Block numbers: each wave loads the table entries of its own chunks into
//    one VGPR (lane k <- chunk k) at the start and reads them back with
//    v_readlane into SGPRs, so the per-load address is a 64-bit scalar base
//    plus a per-lane constant offset.  No LDS round trip, no barrier.
//  * Software pipelining: the next chunk's K and V loads are issued before
//    the current chunk is consumed (two register buffers).
//  * Each 16-lane row group keeps its own online-softmax stream (running max
//    m, sum l, fp32 accumulator of its 8 columns), so the per-chunk work
//    needs only an in-row DPP butterfly for the q.k dot product; the row
//    groups, then the 4 waves (through LDS), are merged once at the end.
//  * Exponentials are exp2 with scale*log2(e) folded into the scores.
//  * Partitions of a sequence beyond the first write fp32 (m, l, o) partials;
//    a reduction kernel merges them.  A sequence that fits one partition is
//    written straight to fp16 by the partition kernel.
//  * Every reduction has a fixed order that depends only on logical token
//    positions, so results are bitwise reproducible and independent of
//    which physical blocks hold the tokens.

#include <type_traits>

#include "kernels.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kWaves = 4;          // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kChunk = 16;         // tokens per chunk
// Occupancy the register allocator may trade down to while keeping two
// 16-token chunks of K and V in flight per wave: 4 waves per SIMD (128 VGPRs)
// for 1-2 query heads per KV head, 3 (168) for 4, 2 (256) for 8.
template <int G>
constexpr int min_waves_per_simd() { return G <= 2 ? 4 : (G == 4 ? 3 : 2); }
constexpr float kNegBig = -1.0e30f;  // start value of a running max
// Word 3 of a gfx9-family buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

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

template <int D>
struct Geometry {
    static constexpr int LPR = D / 8;            // lanes per token row
    static constexpr int RPL = kWave / LPR;      // token rows per wave load
    static constexpr int LPC = kChunk / RPL;     // loads per chunk (K or V)
};

template <int LPC>
struct Frag {
    uint4 k[LPC];
    uint4 v[LPC];
    uint32_t row_ok;   // bit i: this lane's row of load i holds a real token
};

template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves_per_simd<G>())))
void decode_partition_kernel(const DecodeArgs a) {
    using Geo = Geometry<D>;
    constexpr int LPR = Geo::LPR;
    constexpr int RPL = Geo::RPL;
    constexpr int LPC = Geo::LPC;
    constexpr int BPC = BS >= kChunk ? 1 : kChunk / BS;   // blocks per chunk
    static_assert(BS % RPL == 0, "a load must not straddle two blocks");

    __shared__ float s_acc[kWaves][G][D];
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[kWaves][G];

    const int lane = threadIdx.x & (kWave - 1);
    // threadIdx.x / 64 is the same in every lane of a wave; readfirstlane
    // tells the compiler so, which keeps all chunk bookkeeping in SGPRs.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row = lane / LPR;
    const int col = lane % LPR;

    int item = blockIdx.x;
    const int g = item % a.num_kv_heads;
    item /= a.num_kv_heads;
    const int part = item % a.max_parts;
    const int s = item / a.max_parts;

    const int T = a.partition_tokens;
    int L = a.context_lens[s];
    L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
    const int nparts = (L + T - 1) / T;
    const int h0 = g * G;
    const size_t out_row0 = (static_cast<size_t>(s) * a.num_q_heads + h0) * D;

    if (part >= nparts) {
        if (L == 0 && part == 0) {       // empty context: zero output rows
            for (int i = threadIdx.x; i < G * D; i += kThreads) a.out[out_row0 + i] = 0;
        }
        return;
    }

    const int t_begin = part * T;
    const int len = (L - t_begin < T) ? (L - t_begin) : T;
    const int n_chunks = (len + kChunk - 1) / kChunk;
    const int n_local = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;

    // Table entries of this wave's chunks: lane k holds chunk k's blocks.
    int ids[BPC];
    bool bad = false;
    {
        const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq;
        const int c = wave + lane * kWaves;
        const int j0 = (t_begin + c * kChunk) / BS;
#pragma unroll
        for (int e = 0; e < BPC; ++e) {
            int id = -1;
            const int j = j0 + e;
            if (lane < n_local && j * BS < L) {
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

    // This lane's 8 columns of the G query rows.
    half2_t qv[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint4 w = *reinterpret_cast<const uint4*>(a.q + out_row0 + h * D + col * 8);
        qv[h][0] = __builtin_bit_cast(half2_t, w.x);
        qv[h][1] = __builtin_bit_cast(half2_t, w.y);
        qv[h][2] = __builtin_bit_cast(half2_t, w.z);
        qv[h][3] = __builtin_bit_cast(half2_t, w.w);
    }

    const uint32_t row_bytes = static_cast<uint32_t>(a.num_kv_heads) * D * 2;   // one slot
    const uint32_t block_bytes = row_bytes * BS;
    // Per-lane byte offset inside a load: row `row` of the load, 16-byte column `col`.
    const uint32_t lane_off = row * row_bytes + col * 16;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + static_cast<size_t>(g) * D * 2;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + static_cast<size_t>(g) * D * 2;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegBig;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    // Issue the K and V loads of local chunk k (uniform).  Each load goes
    // through a buffer descriptor whose base is the physical block (scalar),
    // with this lane's constant 32-bit offset in a VGPR and the row of the
    // block in an SGPR.  In the masked variant, rows holding no token (ragged
    // tail, bad table entry) still load from a legal address (block 0 stands
    // in for a bad entry) and are dropped in compute(), so issuing never
    // waits for data.
    auto issue = [&](Frag<LPC>& f, int k, auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const int c = wave + k * kWaves;
        const uint32_t tok0 = static_cast<uint32_t>(t_begin + c * kChunk);
        const int nvalid = len - c * kChunk;            // may exceed 16
        f.row_ok = 0;
#pragma unroll
        for (int e = 0; e < BPC; ++e) {
            int blk = __builtin_amdgcn_readlane(ids[e], k);
            const bool blk_ok = blk >= 0;
            if (kMasked) blk = blk_ok ? blk : 0;
            const size_t boff = static_cast<size_t>(blk) * block_bytes;
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char*>(kbase + boff), 0, block_bytes, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char*>(vbase + boff), 0, block_bytes, kRsrcWord3);
            constexpr int kPerBlock = LPC / BPC;        // loads of this chunk in block e
#pragma unroll
            for (int u = 0; u < kPerBlock; ++u) {
                const int i = e * kPerBlock + u;
                const uint32_t in_blk = (tok0 + i * RPL) % BS;
                const int soff = static_cast<int>(in_blk * row_bytes);
                f.k[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(kr, lane_off, soff, 0));
                f.v[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(vr, lane_off, soff, 0));
                if (kMasked) {
                    const bool ok = blk_ok && (i * RPL + row < nvalid);
                    f.row_ok |= ok ? (1u << i) : 0u;
                }
            }
        }
    };

    auto compute = [&](const Frag<LPC>& f, auto masked_tag) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        float sc[LPC][G];
#pragma unroll
        for (int i = 0; i < LPC; ++i) {
            const half2_t k0 = __builtin_bit_cast(half2_t, f.k[i].x);
            const half2_t k1 = __builtin_bit_cast(half2_t, f.k[i].y);
            const half2_t k2 = __builtin_bit_cast(half2_t, f.k[i].z);
            const half2_t k3 = __builtin_bit_cast(half2_t, f.k[i].w);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = __builtin_amdgcn_fdot2(qv[h][0], k0, 0.f, false);
                d = __builtin_amdgcn_fdot2(qv[h][1], k1, d, false);
                d = __builtin_amdgcn_fdot2(qv[h][2], k2, d, false);
                d = __builtin_amdgcn_fdot2(qv[h][3], k3, d, false);
                d = row_sum<LPR>(d) * a.scale_log2;
                if (kMasked && !((f.row_ok >> i) & 1u)) d = -__builtin_inff();
                sc[i][h] = d;
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
#pragma unroll
            for (int i = 0; i < LPC; ++i) {
                const float pr = fast_exp2(sc[i][h] - m_new);
                l[h] += pr;
                uint32_t vw[4] = {f.v[i].x, f.v[i].y, f.v[i].z, f.v[i].w};
                if (kMasked && !((f.row_ok >> i) & 1u)) {
                    // p is 0 here, but 0 * (NaN or Inf) is not: drop the row.
                    vw[0] = vw[1] = vw[2] = vw[3] = 0;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2_t v2 = __builtin_bit_cast(half2_t, vw[j]);
                    acc[h][2 * j] = __builtin_fmaf(pr, static_cast<float>(v2.x), acc[h][2 * j]);
                    acc[h][2 * j + 1] = __builtin_fmaf(pr, static_cast<float>(v2.y), acc[h][2 * j + 1]);
                }
            }
        }
    };

    using Full = std::integral_constant<bool, false>;
    using Masked = std::integral_constant<bool, true>;
    // Chunks this wave owns that are completely inside the context; at most
    // one more (the partition's ragged tail) follows them.
    const int full_chunks = len / kChunk;
    const int n_full = full_chunks > wave ? (full_chunks - wave + kWaves - 1) / kWaves : 0;
    if (!any_bad) {
        if (n_full > 0) {
            Frag<LPC> fa, fb;
            issue(fa, 0, Full{});
            for (int k = 0; k < n_full; k += 2) {
                // The prefetch never runs past the last full chunk: at the
                // end it re-reads that chunk (an L2 hit), so every iteration
                // issues the same loads and the wait counts stay static.
                // The scheduling barriers keep the compiler from sinking the
                // prefetch next to its use, which would serialise latency.
                const int k1 = k + 1 < n_full ? k + 1 : n_full - 1;
                issue(fb, k1, Full{});
                __builtin_amdgcn_sched_barrier(0);
                compute(fa, Full{});
                if (k + 1 >= n_full) break;
                const int k2 = k + 2 < n_full ? k + 2 : n_full - 1;
                issue(fa, k2, Full{});
                __builtin_amdgcn_sched_barrier(0);
                compute(fb, Full{});
            }
        }
        if (n_local > n_full) {
            Frag<LPC> ft;
            issue(ft, n_full, Masked{});
            compute(ft, Masked{});
        }
    } else {
        for (int k = 0; k < n_local; ++k) {
            Frag<LPC> ft;
            issue(ft, k, Masked{});
            compute(ft, Masked{});
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

    // Merge the 4 waves and write either the final fp16 row or the partials.
    for (int o = threadIdx.x; o < G * D; o += kThreads) {
        const int h = o / D;
        const int d = o % D;
        float mm = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = __builtin_fmaxf(mm, s_m[w][h]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(s_m[w][h] - mm);
            num = __builtin_fmaf(f, s_acc[w][h][d], num);
            den = __builtin_fmaf(f, s_l[w][h], den);
        }
        if (nparts == 1) {
            // den is 0 only when no token was read (e.g. every table entry of
            // the partition was out of range); NaN inputs still propagate.
            const float r = den == 0.f ? 0.f : num / den;
            const _Float16 hv = static_cast<_Float16>(r);
            a.out[out_row0 + o] = __builtin_bit_cast(uint16_t, hv);
        } else {
            const size_t prow = (static_cast<size_t>(s) * a.num_q_heads + h0 + h) * a.max_parts + part;
            a.part_o[prow * D + d] = num;
            if (d == 0) {
                a.part_ml[2 * prow] = mm;
                a.part_ml[2 * prow + 1] = den;
            }
        }
    }
}

// Merge split-K partials: one wave per (sequence, query head).
template <int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(const DecodeArgs a) {
    extern __shared__ float s_w[];
    constexpr int PER_LANE = D / kWave;        // 1 or 2 columns per lane
    const int lane = threadIdx.x;
    const int sh = blockIdx.x;                 // s * Hq + h
    const int s = sh / a.num_q_heads;
    const int T = a.partition_tokens;
    int L = a.context_lens[s];
    L = L < 0 ? 0 : (L > a.max_tokens ? a.max_tokens : L);
    const int nparts = (L + T - 1) / T;
    if (nparts <= 1) return;                   // written by the partition kernel

    const float* ml = a.part_ml + static_cast<size_t>(sh) * a.max_parts * 2;
    float mloc = kNegBig;
    for (int i = lane; i < nparts; i += kWave) mloc = __builtin_fmaxf(mloc, ml[2 * i]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) mloc = __builtin_fmaxf(mloc, shfl_xor(mloc, o));
    float den = 0.f;
    for (int i = lane; i < nparts; i += kWave) {
        const float w = fast_exp2(ml[2 * i] - mloc);
        s_w[i] = w;
        den = __builtin_fmaf(w, ml[2 * i + 1], den);
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) den += shfl_xor(den, o);
    __syncthreads();

    const float* po = a.part_o + static_cast<size_t>(sh) * a.max_parts * D + lane * PER_LANE;
    float acc[PER_LANE];
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) acc[e] = 0.f;
    int i = 0;
    for (; i + 4 <= nparts; i += 4) {
        float x[4][PER_LANE];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < PER_LANE; ++e) x[u][e] = po[static_cast<size_t>(i + u) * D + e];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < PER_LANE; ++e) acc[e] = __builtin_fmaf(s_w[i + u], x[u][e], acc[e]);
    }
    for (; i < nparts; ++i)
#pragma unroll
        for (int e = 0; e < PER_LANE; ++e)
            acc[e] = __builtin_fmaf(s_w[i], po[static_cast<size_t>(i) * D + e], acc[e]);

    uint16_t* out = a.out + static_cast<size_t>(sh) * D + lane * PER_LANE;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) {
        const float r = den == 0.f ? 0.f : acc[e] / den;
        out[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
    }
}

template <int D, int BS, int G>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(a.num_seqs) * a.max_parts * a.num_kv_heads;
    hipLaunchKernelGGL((decode_partition_kernel<D, BS, G>), dim3(grid), dim3(kThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.max_parts <= 1) return err;
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(a.num_seqs * a.num_q_heads), dim3(kWave),
                       static_cast<size_t>(a.max_parts) * sizeof(float), stream, a);
    return hipGetLastError();
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.head_dim == 128) return dispatch_block<128>(a, stream);
    if (a.head_dim == 64) return dispatch_block<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa

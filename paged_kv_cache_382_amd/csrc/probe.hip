// Measurement probes: helpers beside the attention path, not steps of it.
//
// Streaming-read probe.  The pages tie decode speed to memory bandwidth
// ("vLLM core architecture ...", section 3, "Continuous batching").  This
// kernel reads a device buffer once, as fast as the device streams reads, so
// that the decode kernel's bandwidth can be set beside what the same device
// reaches with nothing but reads, on the same buffer, in the same run.
// Design: the buffer is cut into equal contiguous ranges, one per workgroup
// (at most 4096 of them, 256 lanes each); every lane keeps 16 non-temporal
// 16-byte loads in flight.  The words are folded with XOR and the result is
// stored only when it equals a fixed constant, so the loads cannot be dropped
// and nothing is written in practice.
//
// Matrix-core probe.  Chunked prefill is a dense contraction on the matrix
// cores ("Deep dive into the nano-vLLM inference engine architecture:
// PagedAttention memory management", section "Deployable configuration
// parameters": prompts are prefilled in chunks).  This kernel issues the
// prefill kernel's fp16 matrix instruction back to back with nothing else to
// do, so that the prefill kernel's rate can be set beside what the same device
// sustains, at the clock it holds under matrix load, in the same run.  Each
// wave keeps four independent accumulation chains of v_mfma_f32_32x32x16_f16
// on register operands; every operand is the caller's value, so each product
// adds 16 * operand^2 to every accumulator, which the kernel checks exactly at
// the end.
//
// Buffer range probe.  The decode and prefill kernels read the cache through
// buffer resources whose range ends at the last row that holds a token (the
// ragged last chunk of a context, the keys a prefill workgroup sees, an
// out-of-range table entry): the rows behind the end must arrive as zeros,
// both for loads into registers and for loads that write LDS directly, and
// the check must cover the scalar offset that the kernels add to every lane's
// offset.  This kernel makes exactly those loads over a caller's buffer, so
// that a test can pin the behaviour the kernels rely on.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_probe.h"

namespace pa {
namespace {

// A lane writes the sink only when the XOR of its words equals this value.
constexpr uint32_t kReadProbeMagic = 0x9E3779B9u;

typedef unsigned int u4 __attribute__((ext_vector_type(4)));
constexpr int kProbeLanes = 256;
constexpr int kProbeUnroll = 16;
constexpr int64_t kProbeMaxGroups = 4096;

__global__ __launch_bounds__(kProbeLanes) void read_probe_kernel(const u4* __restrict__ p, int64_t n_vec,
                                                                 int64_t per_group, uint32_t* sink) {
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * per_group;
    const int64_t end = begin + per_group < n_vec ? begin + per_group : n_vec;
    unsigned acc = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += kProbeLanes * kProbeUnroll) {
        u4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + static_cast<int64_t>(u) * kProbeLanes;
            v[u] = j < end ? __builtin_nontemporal_load(p + j) : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == kReadProbeMagic) *sink = acc;
}

hipError_t launch_read_probe(const void* buf, int64_t n_vec16, uint32_t* sink, hipStream_t stream) {
    if (n_vec16 <= 0) return hipSuccess;
    constexpr int64_t kPerIter = static_cast<int64_t>(kProbeLanes) * kProbeUnroll;
    int64_t groups = (n_vec16 + kPerIter - 1) / kPerIter;
    groups = groups < kProbeMaxGroups ? groups : kProbeMaxGroups;
    const int64_t per_group = (n_vec16 + groups - 1) / groups;
    hipLaunchKernelGGL(read_probe_kernel, dim3(static_cast<unsigned>(groups)), dim3(kProbeLanes), 0, stream,
                       static_cast<const u4*>(buf), n_vec16, per_group, sink);
    return hipGetLastError();
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));
constexpr int kRangeProbeLanes = 64;
constexpr int kMfmaLanes = 512;                  // 8 waves: two per SIMD
constexpr int kMfmaChains = 4;

__global__ __launch_bounds__(kMfmaLanes) void mfma_probe_kernel(int32_t iters, float operand, uint32_t* sink) {
    h8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = static_cast<_Float16>(operand);
    f16x c[kMfmaChains];
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[k][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c[k], 0, 0, 0);
    }
    // Operand 1: every accumulator holds 16 * iters exactly (iters <= 65536).
    const float want = 16.0f * static_cast<float>(iters);
    bool ok = true;
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) ok = ok && c[k][r] == want;
    if (!ok) *sink = 1u;
}

hipError_t launch_mfma_probe(uint32_t* sink, int32_t workgroups, int32_t iters, float operand, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kMfmaLanes), 0, stream,
                       iters, operand, sink);
    return hipGetLastError();
}

constexpr int kRsrcWord3 = 0x00020000;          // 32-bit data format, no swizzle
typedef __attribute__((address_space(3))) void lds_void;

struct RangeProbeArgs {
    const void* buf;
    uint32_t range;
    uint32_t soffset;
    int32_t n;
    uint32_t voff[kRangeProbeLanes];
    uint32_t* out;
};

__global__ __launch_bounds__(kRangeProbeLanes) void range_probe_kernel(RangeProbeArgs a) {
    __shared__ __align__(16) uint32_t tile[kRangeProbeLanes * 4];
    const int j = threadIdx.x;
    // Lanes past n repeat lane 0's offset (every offset was checked against
    // the allocation) and store nothing.
    const uint32_t v = a.voff[j < a.n ? j : 0];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.buf), 0,
                                                                        static_cast<int>(a.range), kRsrcWord3);
    const u4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, v, a.soffset, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)tile, 16, v, a.soffset, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): the LDS writes have landed
    __syncthreads();
    if (j < a.n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a.out[j * 4 + i] = r[i];
            a.out[(a.n + j) * 4 + i] = tile[j * 4 + i];
        }
    }
}

hipError_t launch_range_probe(const RangeProbeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(range_probe_kernel, dim3(1), dim3(kRangeProbeLanes), 0, stream, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream) {
    if (bytes % 16 != 0) return PA_ERR_SHAPE;
    if (bytes == 0) return PA_OK;
    if (!buf || !sink) return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0) return PA_ERR_ALIGN;
    const hipError_t err = pa::launch_read_probe(buf, static_cast<int64_t>(bytes / 16), sink,
                                                 static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_mfma_probe(uint32_t* sink, int32_t workgroups, int32_t iters, float operand,
                                   void* hip_stream) {
    if (workgroups < 0 || workgroups > 65536 || iters < 1 || iters > 65536) return PA_ERR_SHAPE;
    if (workgroups == 0) return PA_OK;
    if (!sink) return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sink) % 4 != 0) return PA_ERR_ALIGN;
    const hipError_t err = pa::launch_mfma_probe(sink, workgroups, iters, operand, static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" pa_status pa_range_probe(const void* buf, size_t alloc_bytes, uint32_t range_bytes, uint32_t soffset,
                                    const uint32_t* voffsets, int32_t n, uint32_t* out, void* hip_stream) {
    if (n < 1 || n > pa::kRangeProbeLanes) return PA_ERR_SHAPE;
    if (!buf || !voffsets || !out) return PA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0 || soffset % 4 != 0)
        return PA_ERR_ALIGN;
    if (range_bytes > alloc_bytes) return PA_ERR_RANGE;
    pa::RangeProbeArgs a{};
    for (int j = 0; j < n; ++j) {
        if (voffsets[j] % 4 != 0) return PA_ERR_ALIGN;
        // Every load stays inside the allocation even without a range check.
        if (static_cast<uint64_t>(voffsets[j]) + soffset + 16 > alloc_bytes) return PA_ERR_RANGE;
        a.voff[j] = voffsets[j];
    }
    a.buf = buf;
    a.range = range_bytes;
    a.soffset = soffset;
    a.n = n;
    a.out = out;
    const hipError_t err = pa::launch_range_probe(a, static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

/*
 * pa_probe.h -- measurement probes of AMD Instinct MI355X (gfx950), built as
 * their own library (paged_kv_cache_382_amd/lib/libpa_probe.so).  Helpers
 * beside the attention library, not steps of the attention path.
 *
 * pa_read_probe -- source: "vLLM core architecture: PagedAttention principle,
 * KV Cache management, continuous batching", section 3 ("Continuous
 * batching"): decode speed is a matter of memory bandwidth.  This call reads a
 * buffer once at the rate the device streams plain reads, so that the decode
 * kernel's bandwidth can be set beside it in the same run on the same memory.
 *
 * pa_mfma_probe -- source: "Deep dive into the nano-vLLM inference engine
 * architecture: PagedAttention memory management", section "Deployable
 * configuration parameters" (prompts are prefilled in chunks): chunked
 * prefill is a dense contraction on the matrix cores.  This call runs the prefill kernel's fp16
 * matrix instruction back to back with nothing else, so that the prefill
 * kernel's rate can be set beside what the device sustains, at the clock it
 * holds under matrix load, in the same run.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*   buf     device, 16-byte aligned, `bytes` readable bytes; read once with
 *           16-byte non-temporal loads spread over the whole device
 *   bytes   a multiple of 16; 0 launches nothing
 *   sink    device uint32, 4-byte aligned: written (with 0x9E3779B9) only if
 *           the XOR of the 32-bit words one lane read equals 0x9E3779B9, so
 *           the loads cannot be optimised away; normally left untouched
 *
 * Enqueued on hip_stream; returns after the launch.  Errors (status codes of
 * pa.h; this library keeps no error text): PA_ERR_SHAPE (bytes not a multiple
 * of 16), PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_HIP (launch failed). */
pa_status pa_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream);

/*   sink        device uint32, 4-byte aligned: set to 1 if any accumulator
 *               differs from 16 * iters (the value for operand 1.0), else
 *               left untouched; so with operand 1.0 it stays as the caller
 *               set it, and any other operand of magnitude above 1 sets it
 *   workgroups  0 .. 65536 workgroups of 8 waves (512 lanes); 0 launches nothing
 *   iters       1 .. 65536 iterations; each wave runs 4 * iters
 *               v_mfma_f32_32x32x16_f16 (32 x 32 x 16 fp16 products, fp32
 *               accumulation) in four independent chains
 *   operand     every A and B element (rounded to fp16)
 *
 * Work of one call: workgroups * 8 * 4 * iters * 32768 flops (a product of
 * 32 x 32 x 16 is 32768 flops).  Enqueued on hip_stream; returns after the
 * launch.  Errors: PA_ERR_SHAPE (counts out of range), PA_ERR_NULL,
 * PA_ERR_ALIGN, PA_ERR_HIP (launch failed). */
pa_status pa_mfma_probe(uint32_t* sink, int32_t workgroups, int32_t iters, float operand, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */

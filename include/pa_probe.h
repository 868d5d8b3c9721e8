/*
 * pa_probe.h -- streaming-read probe of AMD Instinct MI355X (gfx950), built as
 * its own library (paged_kv_cache_382_amd/lib/libpa_probe.so).  A measurement
 * helper beside the attention library, not a step of the attention path.
 *
 * Source: "vLLM core architecture: PagedAttention principle, KV Cache
 * management, continuous batching", section 3 ("Continuous batching"): decode
 * speed is a matter of memory bandwidth.  This call reads a buffer once at the
 * rate the device streams plain reads, so that the decode kernel's bandwidth
 * can be set beside it in the same run on the same memory.
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

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */

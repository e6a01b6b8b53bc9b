/* Measurement helper of libattn.so: an attainable-HBM-bandwidth reference.
 *
 * Not part of the attention path.  The paged decode is bound by HBM reads, and
 * its achieved rate is reported both against the 8 TB/s specification and
 * against what a plain streaming read reaches on the same device; this call is
 * that plain read.
 *
 * Status codes are those of attn.h (attn_status_string describes them).
 */
#ifndef ATTN_MEASURE_H
#define ATTN_MEASURE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `p` once, with 128-bit loads spread
 * over the whole GPU, and fold them into one 32-bit value; that value is
 * written to the device word `sink` only when it equals 0x9e3779b9 (so the
 * loads cannot be dropped, and `sink` is almost never written).
 *   p     device pointer, 16-byte aligned; not modified
 *   bytes a multiple of 16, at least 16
 *   sink  device pointer to 4 writable bytes, owned by the caller
 *   stream hipStream_t (NULL = default stream); asynchronous, no allocation
 * Errors: ATTN_ERR_NULL (p or sink null), ATTN_ERR_SHAPE (bytes), ATTN_ERR_ALIGN
 * (p not 16-byte aligned), ATTN_ERR_DEVICE (current device not gfx950),
 * ATTN_ERR_HIP (launch failed).  Nothing is launched on an error. */
int attn_hbm_read_probe(const void* p, size_t bytes, unsigned int* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MEASURE_H */

/* Measurement helper of libwq (not a step of the layer): the streaming-read
 * ceiling that the layer's weight stream is compared with.  Same library,
 * same conventions as wq.h (device pointers, wq_status results, errors
 * before any launch, asynchronous on `stream`, a hipStream_t or NULL). */
#ifndef WQ_MEASURE_H
#define WQ_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "wq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at `src` once, in 16-byte loads by
 * one short-lived 256-thread workgroup per 8 KiB, and stores nothing but
 * possibly one meaningless word to `sink` (device, 4 bytes) so the loads
 * are kept.  Timing it on data of a
 * workload's size gives the plain-read ceiling at that size.
 *   bytes  > 0, a multiple of 16; src and sink 16-byte aligned.
 * Returns WQ_E_ARG for bytes == 0, bytes % 16 or a NULL pointer, WQ_E_ALIGN
 * for misalignment, WQ_E_HIP for a launch error. */
wq_status wq_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_MEASURE_H */

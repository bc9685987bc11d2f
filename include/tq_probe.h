/*
 * tq_probe.h -- measurement helper shipped with libtq (not part of the method).
 *
 * tq_probe_stream_read reads `bytes` bytes of device memory once, with 16-byte loads
 * spread over the whole GPU, and writes nothing but one word that depends on every
 * byte read.  Timed over a buffer far larger than the 256 MB Infinity Cache it gives
 * the streaming HBM read rate the same box sustains, the practical ceiling for the
 * scan-like decode kernels next to the published 8 TB/s peak.
 *   src     device, 16-byte aligned, `bytes` readable bytes
 *   bytes   multiple of 16, > 0
 *   sink    device uint32[1] (out): a fold of everything read (only so that the reads
 *           cannot be dropped); its value has no meaning
 *   stream  hipStream_t or NULL
 * Returns TQ_OK, TQ_ERR_INVALID (null/misaligned pointer, bad size) or TQ_ERR_HIP.
 */
#ifndef TQ_PROBE_H
#define TQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int tq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_PROBE_H */

/*
 * gqa_probe.h -- measurement probes exported by libgqa_decode.so.
 *
 * Not part of the decode method: two plain streaming kernels that give the
 * measurements of the decode kernels a reference on the same machine.
 *   gqa_probe_copy  copies `bytes` bytes src -> dst; a kernel of known traffic,
 *                   used to scale hardware byte counters (FETCH_SIZE, WRITE_SIZE)
 *                   to bytes.
 *   gqa_probe_read  reads `bytes` bytes and folds them (XOR of 32-bit words) into
 *                   the GQA_PROBE_SINK_WORDS words at `sink` with atomic XORs, so the
 *                   loads cannot be elided (the XOR of all sink words is the XOR of
 *                   all words read, if the sink started zeroed); its rate is the
 *                   achievable HBM read bandwidth, the practical ceiling of the
 *                   bandwidth-bound decode sweep.
 *
 * Pointers are device memory of the current HIP device, owned by the caller.
 * src, dst and bytes must be multiples of 16 (sink: 4-byte aligned, GQA_PROBE_SINK_WORDS
 * uint32 words).  Work is
 * enqueued on `stream` (hipStream_t, NULL = null stream) without synchronising.
 * Returns 0, 1 (NULL pointer), 4 (misaligned) or 7 (HIP error), the same codes
 * as gqa_status in gqa_decode.h.
 */
#ifndef GQA_PROBE_H
#define GQA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#define GQA_PROBE_SINK_WORDS 256

#ifdef __cplusplus
extern "C" {
#endif

int gqa_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

int gqa_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H */

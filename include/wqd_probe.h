/* wqd_probe.h -- C ABI of libwqd_probe.so, a measurement aid beside libwqd.so (not part of the
 * decode path).
 *
 * The ternary vLLM page ("Making a ternary reasoning model fast in vLLM", "A rough speed limit")
 * bounds a batch-1 decode by the time to stream the packed weights once at the memory bandwidth.
 * The pages' byte model only means something against a bandwidth the card reaches in practice, so
 * this library times the plainest stream of the same bytes: every byte read once, with 16-byte
 * nontemporal loads, nothing computed but an XOR that keeps the loads alive.
 */
#ifndef WQD_PROBE_H
#define WQD_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQD_PROBE_API __attribute__((visibility("default")))

/* Read `bytes` bytes of device memory at `buf` once (16-byte aligned; bytes a multiple of 16 KiB)
 * with one persistent launch of `workgroups` workgroups of 1024 threads (0 = one per CU): each wave
 * streams one contiguous share in 1 KiB wave loads, 8 in flight.  `sink` (device, at least
 * workgroups * 1024 * 4 bytes) receives each thread's XOR of its data.  Enqueued on `stream`
 * (a hipStream_t); returns 0, -1 for a bad argument or -5 for a launch failure. */
WQD_PROBE_API int wqd_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t workgroups,
                                 void *stream);

#ifdef __cplusplus
}
#endif
#endif /* WQD_PROBE_H */

/*
 * Measurement aid of libspecverify (not part of the verify step): a plain read
 * of a device buffer in the pattern of the verify step's row-statistics pass,
 * so that a benchmark can report, beside the verify step's bandwidth, what the
 * GPU reaches when it only reads the same number of bytes.
 */
#ifndef SPECVERIFY_PROBE_H
#define SPECVERIFY_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads floor(bytes / 16384) items of 16 KB of `buf` (device memory, 16-byte aligned) with
 * wgs_per_cu (1..32) workgroups of 256 threads per compute unit; workgroup w of G reads the
 * contiguous items [w N / G, (w + 1) N / G), the next item's loads in flight while the current
 * one is consumed.  The data only feed an xor; `sink` (device, one uint32) is written only when
 * that xor equals a fixed unlikely value, which keeps the loads.  Asynchronous on `stream`
 * (hipStream_t, NULL = default); ev_start / ev_stop (hipEvent_t, both or neither) take the
 * dispatch's own start and end timestamps.  Returns SV_OK, SV_EINVAL (NULL or misaligned
 * pointer, wgs_per_cu out of range, fewer than 16384 bytes) or SV_EHIP.
 */
int spec_read_probe(const void* buf, uint64_t bytes, int32_t wgs_per_cu, void* sink, void* stream,
                    void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_PROBE_H */

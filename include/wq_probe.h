/*
 * wq_probe.h - measurement aid of the benchmark (libwq_probe.so), not part of the
 * W4A16 linear's boundary (include/wq.h). The pages give no kernel-level figures;
 * this plain streaming read is the context in which the decode kernels' HBM rate
 * is reported: what a read-only kernel reaches in one launch over the same bytes.
 */
#ifndef WQ_PROBE_H
#define WQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * wq_probe_stream_read - one launch that reads `bytes` bytes of device memory at
 * `src` once, in 16-byte coalesced loads (eight in flight per thread), and writes
 * (almost) nothing: `sink` (a device uint32) is written only if the XOR of all
 * words a block read equals a fixed constant.
 *  src    device pointer, 16-byte aligned; bytes a positive multiple of 16.
 *  Returns 0, -1 (NULL pointer), -2 (size or alignment), -5 (launch failed).
 */
int wq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_PROBE_H */

/*
 * wq_probe.h -- C ABI of the measurement probe library libwq_probe.so (not
 * part of the product path; the benchmark uses it for context figures).
 *
 * Decode-sized products are bound by the bytes they move (exllama discussion
 * "Regarding comment on benchmark memory bandwidth speeds", GPTQ paper quote
 * and turboderp's reply).  The probe gives the time a single launch needs only
 * to read the same number of bytes: the ceiling a GEMV launch of that size can
 * approach.
 */
#ifndef WQ_PROBE_H
#define WQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * wq_probe_stream_read -- read `bytes` bytes of device memory at `buf` once
 * (128-bit non-temporal buffer loads), asynchronously on `stream`
 * (hipStream_t as void*, NULL = default stream).
 *   buf             : device memory, caller-owned, at least `bytes` long
 *   bytes           : > 0, multiple of 16
 *   workgroups      : 1 .. 2^20 workgroups of 256 threads, each reading one
 *                     contiguous chunk (chunks stay below 1 GiB)
 *   loads_in_flight : 2, 4 or 8 16-byte loads per lane per step
 *   sink            : device uint32, written only in the unlikely case that
 *                     the folded words equal one fixed value (keeps the loads)
 * Returns 0 on success, 1 for invalid arguments, 2 when a chunk would reach
 * 1 GiB, 3 when the launch failed.  Nothing is launched on an error.
 */
int wq_probe_stream_read(const void* buf, size_t bytes, int workgroups, int loads_in_flight, uint32_t* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_PROBE_H */

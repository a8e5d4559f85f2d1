/* Measurement helpers of the Q4 weight-matrix product library.
 *
 * Not part of the products: these kernels exist so that a benchmark can put
 * the products' achieved HBM bandwidth next to what a plain streaming read
 * reaches on the same device, in the same process. */
#ifndef Q4_BENCH_H
#define Q4_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes at device pointer `p` (16-byte aligned, bytes a
 * multiple of 16) once, with coalesced 16-byte non-temporal loads, using
 * `groups` workgroups of 256 threads (1 .. 65536) that stride over the
 * buffer. With `sink` NULL nothing is written: a pure read. Otherwise
 * `sink` holds 4 * `groups` 4-byte device words: word 4g + v receives the
 * XOR of the 32-bit words wave v of workgroup g read, so the XOR of all of
 * them is the fold of the whole buffer, and a caller can check that every
 * word was read exactly once (a word missed or read twice changes the fold).
 * The stores cost the kernel's end the write-back of dirty lines that a pure
 * read does not pay.
 * Enqueued on `hip_stream`; returns a
 * q4_status value (Q4_EINVAL for bad arguments, Q4_EALIGN for misalignment,
 * Q4_EHIP if the launch fails). */
int q4_read_probe(const void *p, size_t bytes, uint32_t *sink, int groups, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_BENCH_H */

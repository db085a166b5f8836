/*
 * sv_probe.h -- a measurement aid shipped with the verification library: the plain
 * streaming-read rate that the library's HBM-bound kernels are compared with.  It is no
 * part of the verification method; the benchmark runs it on the same device, on buffers of
 * the size one verification call reads, to report the achieved bandwidth of the
 * verification kernels against what a kernel that only reads can reach.
 */
#ifndef SV_PROBE_H
#define SV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at `buf` once, the way the verification kernels
 * stream logits: one 256-thread workgroup per 32 KiB chunk, 128-bit non-temporal loads,
 * every load of a thread issued before any is used.  Workgroup i adds the 32-bit words
 * of its chunk (wrapping) and writes the sum to out[i], so that no load can be dropped;
 * the sum of out[0 .. n) equals the wrapping sum of every word of the buffer, with
 * n = bytes / 32768.
 *   buf    device pointer, 16-byte aligned; bytes a positive multiple of 32768
 *   out    device pointer to bytes / 32768 uint32 values (written)
 *   stream a hipStream_t (NULL: the default stream); nothing is synchronised.
 * Returns 0 when the launch was enqueued, 1 for a NULL pointer, 2 for a size or
 * alignment outside the above, 7 when the HIP runtime refused the launch. */
int32_t sv_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream);

/* Timeline stamps of spec_verify (its sampling kernel), for measurement.  The library
 * built for timelines (libspec_verify_timeline.so: the same sources compiled with
 * SV_TIMELINE) has the kernels store the wall clock (wall_clock64, 64-bit words) at fixed
 * points of each sequence's path into buf: word 0 when the grid starts; for sequence b,
 * from word 8 + 512 b: first-pass item (row r of the sequence, chunk c) at r*C + c when
 * below 256; 256 the finisher's entry, 257 its last partial in, 258 its draw record out;
 * 260 + i draw item i (chunk c, quarter s: i = 4c + s, i < 96) with the record, 360 + i
 * its segment masses out; 460 the combiner with every mass in; 461 the sequence's drawn
 * token written.  Stamps not reached keep what buf held.  buf (device memory of at least
 * 8 + 512 B words; NULL stops the stamps) is used by later spec_verify calls of this
 * process until replaced.  *clock_khz (nullable) receives the wall clock's rate on the
 * current device.  Returns 0; 1 in the library built without stamps (nothing done); 7 if
 * the HIP runtime did not give the rate. */
int32_t sv_timeline_stamps(void *buf, int32_t *clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* SV_PROBE_H */

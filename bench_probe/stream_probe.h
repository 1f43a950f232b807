/*
 * stream_probe.h -- streaming passes used as the practical bandwidth ceiling
 * that the RMSNorm kernels' figures are compared with.  Measurement only:
 * bench.py and its tests load this library; the RMSNorm library does not.
 *
 * sp_stream_mix: one pass over n16 16-byte vectors of nsrc source and ndst
 * destination streams (caller-owned device buffers of at least 16 * n16
 * bytes each, 16-byte aligned).  Vector i of every source is read
 * (non-temporal); their XOR is written (non-temporal) to vector i of every
 * destination.  With nsrc = 0 the destinations receive the vector index
 * pattern (i, ~i, i, ~i as 32-bit words); with ndst = 0 the XOR of everything
 * read is folded into one word per thread and `sink` (a device pointer to
 * one uint32, required then) is written only if that word equals 0x9E3779B9,
 * which keeps the loads without a store stream.  The pass moves
 * (nsrc + ndst) * 16 * n16 bytes with that read:write mix and no other work.
 *   nsrc 0..4, ndst 0..5, not both 0.
 *   grid 1..65536 work-groups of wgs threads (64, 128, 256, 512 or 1024).
 *   vpt  vectors per thread per stream in flight in each step: 1, 2, 4 or 8.
 *   order
 *     0  grid-stride: step s of work-group b covers the tile s * grid + b of
 *        wgs * vpt vectors;
 *     1  the same window walk with the work-groups renumbered so that each of
 *        the 8 XCDs (work-groups are dispatched to them round-robin) covers a
 *        contiguous part of every window, as the RMSNorm kernels walk rows;
 *     2  each work-group streams one contiguous chunk of about n16 / grid
 *        vectors.
 * src and dst are HOST arrays of nsrc / ndst device pointers.  Returns 0, or
 * 1 (a NULL pointer), 2 (an argument out of range), 4 (a misaligned stream)
 * or 9 (the launch failed); asynchronous on `stream` (a hipStream_t).
 */
#ifndef STREAM_PROBE_H
#define STREAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int sp_stream_mix(const void* const* src, int nsrc, void* const* dst, int ndst, int64_t n16, int grid, int wgs,
                  int vpt, int order, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_PROBE_H */

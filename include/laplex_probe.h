/*
 * laplex_probe.h -- memory-system probes for AMD Instinct MI355X (gfx950),
 * built as their own library (liblaplex_probe.so) beside the LAPLEX operator
 * library.  They are not part of the operator.  They time the streaming
 * patterns its kernels are measured against: a copy in two shapes, a plain
 * read, a plain write, and the data movement of one radix-sort pass without
 * its ranking.
 *
 * Conventions: src and dst are DEVICE pointers owned by the caller, 16-byte
 * aligned, each of at least `bytes` bytes (bytes a multiple of 16, and of
 * 65536 for LAPLEX_PROBE_RUNS).  dst must not overlap src.  Work is enqueued
 * on `stream` and is asynchronous; the return value reports argument errors
 * (and launch errors) synchronously: 0 on success, 2 for a size that is not a
 * valid multiple, 3 for a misaligned pointer, 1 for a NULL pointer, 9 for an
 * unknown kind, 6 for a failed launch (the values of laplex_status).
 */
#ifndef LAPLEX_PROBE_H
#define LAPLEX_PROBE_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  /* dst = src; one 16-byte piece per thread, 256-thread workgroups on
   * 4 KiB chunks, each XCD taking a contiguous range of chunks */
  LAPLEX_PROBE_COPY_1 = 0,
  /* dst = src; eight 16-byte pieces per thread (32 KiB per workgroup), all
   * loads issued before the stores, workgroups in launch order */
  LAPLEX_PROBE_COPY_8 = 1,
  /* reads src (one 16-byte piece per thread, as COPY_1); dst receives, as
   * float, the sum of each 4 KiB chunk (bytes / 4096 floats) */
  LAPLEX_PROBE_READ = 2,
  /* dst filled with the float pattern (1, 2, 3, 4) repeated; src unused */
  LAPLEX_PROBE_WRITE = 3,
  /* a radix pass's data movement without ranking: src holds tiles of 8192
   * 8-byte pairs; pairs 32 d .. 32 d + 31 of tile t go to run (d, t) of dst,
   * which is laid out [256][tiles][32] pairs, so each tile writes 256 runs of
   * 256 bytes into 256 regions (512 threads, 16 pairs each) */
  LAPLEX_PROBE_RUNS = 4
} laplex_probe_kind;

/* Enqueue one probe of `kind` over `bytes` bytes. */
int laplex_probe(int kind, const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAPLEX_PROBE_H */

/* Memory-system probes of the benchmark (libkveprobe.so).  They are not
 * part of the eviction path: they measure the HBM read ceiling that the
 * scorer's passes are compared with, and evict the caches with clean lines
 * before a cold-cache measurement.
 *
 * All pointers are device pointers; every call enqueues one kernel on
 * `stream` and returns without synchronising.  Returns 0, -1 for invalid
 * arguments (nothing launched) or -2 when the launch failed.
 */
#ifndef KVEPROBE_H
#define KVEPROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) from `p` once with 16-byte loads.
 * `sink` must hold kvp_read_sink_words() uint32 (written only in a case that
 * practically never occurs, so the loads cannot be elided). */
int kvp_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);
int kvp_read_sink_words(void);

/* Streams k and v ([Hkv][n][128] bf16 each) through the scorer's ring
 * structure: one 4-wave workgroup per (head, chunk of `chunk` keys), a
 * 2-stage LDS ring of 64-key K and V tiles.  n must be a multiple of chunk,
 * chunk a multiple of 64, and Hkv * n / chunk at most kvp_read_sink_words(). */
int kvp_read_ring(const void* k, const void* v, int Hkv, int n, int chunk, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif

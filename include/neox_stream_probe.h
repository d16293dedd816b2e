/*
 * neox_stream_probe.h -- bandwidth probes that measure what the MI355X's HBM delivers to
 * the access patterns of the ZeRO-1 step, so the step's throughput can be reported as
 * a fraction of an attainable ceiling as well as of the 8 TB/s nameplate.  Not part of
 * the step; used by the benchmark only.
 *
 * Both probes enqueue one kernel on hip_stream and return without waiting.  Pointers
 * are device pointers, 16-byte aligned.  Return: 0, or -1 (bad argument) / -2 (launch
 * failed) with neox_probe_last_error() describing it.
 */
#ifndef NEOX_STREAM_PROBE_H
#define NEOX_STREAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Plain streaming copy: dst[0:bytes) = src[0:bytes), one 16-byte vector per thread,
 * stores non-temporal when nt_stores != 0.  bytes must be a multiple of 16; src and dst
 * must not overlap. */
int neox_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t nt_stores,
                    void* hip_stream);

/* The update kernel's memory access pattern with trivial arithmetic: over n elements
 * (a multiple of 8) it reads a 2-byte gradient and three FP32 arrays and writes the
 * three FP32 arrays in place and a 2-byte copy, 28 bytes per element, with 16-byte
 * vectors, in tiles walked last-to-first.  Launch shape: `threads` per block (64, 128,
 * 256 or 512), `vectors` 8-element vectors per thread (1, 2 or 4; a tile is threads x
 * vectors x 8 elements), at most `blocks_per_cu` blocks per CU (0 = as many as fit;
 * 1..16, enforced by reserving LDS), stores non-temporal when nt_stores != 0.  The
 * arrays' contents are changed.  Unlike the update, a thread may start storing its
 * first vector before the loads of its later vectors return; at 2 or 4 vectors per
 * thread that ordering makes the pattern slower than the update at the same shape, so
 * the ceiling is the best shape, not a fixed one. */
int neox_probe_update_pattern(const void* grad, void* half, float* master, float* exp_avg,
                              float* exp_avg_sq, uint64_t n, int32_t threads, int32_t vectors,
                              int32_t blocks_per_cu, int32_t nt_stores, void* hip_stream);

const char* neox_probe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif

/*
 * mla_probe.h -- measurement probes of libmla_probe.so (gfx950): the rates the chip reaches for the kinds of
 * work the decode path is bound by, measured beside the decode so that its roofline fraction can be read
 * against the achievable rate as well as the vendor peak.  They compute nothing of the method.
 *
 * Conventions: pointers are device memory owned by the caller; every call only enqueues work on `stream`
 * (a hipStream_t, NULL = default stream) and returns 0, or 1 for a bad argument (nothing enqueued), 2 for a
 * grid too small to cover the work, 6 for a failed launch.  The caller times the calls (HIP events).
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) from src with `workgroups` workgroups of 256 threads in a grid-stride
 * loop; each thread writes one folded word to sink[workgroups * 256]. */
int mla_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

/* Reads `rows` rows of row_bytes bytes (a multiple of 16): row r at pool + addr16[r] * 16.  The grid of
 * `workgroups` x 256 threads, 6 chunks of 16 bytes per thread, must cover rows * row_bytes / 16 chunks;
 * sink[workgroups * 256] receives one folded word per thread. */
int mla_probe_row_gather(const void* pool, const uint32_t* addr16, int64_t rows, int32_t row_bytes, uint32_t* sink,
                         int32_t workgroups, void* stream);

/* Runs `iters` rounds of 8 independent v_mfma_f32_16x16x32 (bf16 != 0: bf16 operands, else FP16) in every wave
 * of `workgroups` x 256 threads; out receives workgroups * 256 * 4 floats.  mla_probe_mfma_flops gives the
 * flops of such a call (2 per multiply-add). */
int mla_probe_mfma(int32_t bf16, int32_t iters, float* out, int32_t workgroups, void* stream);
int64_t mla_probe_mfma_flops(int32_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */

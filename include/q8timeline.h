/*
 * q8timeline.h -- per-wave timeline of the narrow matmul (MI355X, gfx950).
 *
 * Exported only by the timeline build of the library,
 * libq8narrow_timeline.so (the same sources compiled with Q8_TIMELINE); the
 * product library libq8narrow.so does not export it and its kernels hold no
 * timing code.  The timeline build exports every entry point of q8narrow.h
 * with the same behaviour and results, bit for bit; its matmul kernels also
 * read the GPU's 100 MHz real-time counter (s_memrealtime) at fixed points
 * of each wave and write those reads to a caller-owned record buffer, so a
 * profile can attribute a launch's time to dispatch, streaming and the
 * epilogue steps.  The extra reads and the record stores make it slightly
 * slower; its times are for attribution, never for the headline figures.
 *
 * Callers: profiling tools.  The timeline library keeps one buffer pointer
 * (process-wide state, unlike q8narrow.h's stateless product library).
 */
#ifndef Q8TIMELINE_H
#define Q8TIMELINE_H

#include <stdint.h>

#include "q8narrow.h"

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_STAMP_WORDS 8 /* uint64 words per wave record */

/* Sets the record buffer of every later matmul launch of this process
 * (q8_matmul_narrow, _ws, _noalloc, _multi, and the fused entry points'
 * matmul workgroups, whose wave index counts from the first matmul
 * workgroup; the DOT4 engine records nothing).  records: device, 8-byte aligned,
 * caller-owned, at least max_waves * Q8_STAMP_WORDS uint64; null or
 * max_waves = 0 switches recording off.  The launch after this call writes
 * the record of its wave i = blockIdx.x * waves_per_workgroup + wave only if
 * i < max_waves; records of waves past that and words never reached keep
 * what the buffer held, so clear it first (a fill kernel, stream-ordered).
 * Each later launch overwrites the records of its waves: set the buffer, run
 * one launch, read it.
 *
 * Record of one wave of the MFMA matmul (ticks of 10 ns):
 *   [0] the wave starts (after the fused producers' branch)
 *   [1] its first chunk's dot is issued (first weights and slots arrived;
 *       for the fused entry points, after its wait for the slots)
 *   [2] its last chunk's dot is issued (streaming done)
 *   [3] its workgroup's partial tiles are in LDS (after the barrier)
 *   [4] single-workgroup tree: Y stores issued;
 *       split: its partial published (stores complete)
 *   [5] single-workgroup tree: Y stores complete;
 *       split: after its arrival at the counter
 *   [6] split, the last split of its row block only: Y stored and counter
 *       rearmed; otherwise 0
 *   [7] bits 0..31 the HW_ID register (wave, SIMD, CU, shader array, shader
 *       engine), bits 32..35 the XCC
 *
 * Returns Q8_ERR_INVALID_ARG for max_waves < 0, or for a null or
 * misaligned buffer with max_waves > 0; else Q8_OK. */
q8_status q8_timeline_set(uint64_t* records, int64_t max_waves);

#ifdef __cplusplus
}
#endif

#endif /* Q8TIMELINE_H */

/*
 * sparsp_measure.h -- measurement support for libsparsp on AMD Instinct MI355X (gfx950).
 *
 * Not operations of the method: these calls let a benchmark report the shader clock the kernels ran at,
 * beside their durations, so that a throughput can be compared with a peak stated at another clock.
 *
 * Conventions as in sparsp.h: extern "C", caller-owned device memory, work enqueued on `stream`, status codes.
 */
#ifndef SPARSP_MEASURE_H
#define SPARSP_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Clock sampler: one 64-thread workgroup that, every `interval_ticks` ticks of the GPU's constant-rate wall
 * clock, records the pair (shader clock counter, wall clock counter) of the compute unit it runs on.  It
 * takes `n_samples` samples and exits: its run time is bounded by n_samples * interval_ticks wall-clock ticks
 * from its start.  Launch it on a stream of its own beside the kernels being measured; it occupies one wave
 * slot of one compute unit.  DEVICE pointer:
 *   samples   [n_samples][2] uint64: {shader clock, wall clock}                              (written)
 * The shader clock frequency over a window is the shader-counter difference divided by the wall-counter
 * difference, times the wall clock rate (sparsp_wall_clock_khz).
 * Errors: SPARSP_ERR_INVALID (NULL samples, n_samples < 2, interval_ticks < 1, or n_samples * interval_ticks
 * above 2^32 ticks); SPARSP_ERR_HIP for a launch failure.
 */
int32_t sparsp_clock_sampler(uint64_t* samples, int32_t n_samples, int32_t interval_ticks, void* stream);

/*
 * Write the wall clock counter to *out (DEVICE pointer) from a one-thread kernel enqueued on `stream`: marks
 * a point in that stream's order on the sampler's time axis.
 * Errors: SPARSP_ERR_INVALID (NULL out); SPARSP_ERR_HIP for a launch failure.
 */
int32_t sparsp_wall_timestamp(uint64_t* out, void* stream);

/*
 * Rate of the wall clock counter of the current device, in kHz (HOST pointer).
 * Errors: SPARSP_ERR_INVALID (NULL khz); SPARSP_ERR_HIP if the runtime cannot report it.
 */
int32_t sparsp_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* SPARSP_MEASURE_H */

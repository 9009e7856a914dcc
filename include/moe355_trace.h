/*
 * libmoe355_trace.so: the diagnostic build of libmoe355 (same calls, same results)
 * whose gate/up grouped GEMM on 128-row tiles records the shader clock (s_memtime,
 * low 32 bits) three times per K step and wave: before the wave's wait for its stage
 * DMAs, after that wait, and after the barrier that publishes the stage.  The clocks
 * of tiles [0, 64) of the last launch are kept, [tile][wave 0..7][step 0..63][3]
 * (uint32; steps past the problem's K blocks hold nothing meaningful).  For the per-step
 * breakdown of the pipeline ("Blockscale FP8 MoE Computation": the grouped GEMM is the
 * layer's hot loop): wait, barrier and compute time of each step.
 */
#ifndef MOE355_TRACE_H
#define MOE355_TRACE_H

#include <stddef.h>
#include <stdint.h>

#include "moe355.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copies the first `count` (<= 64 * 8 * 64 * 3) clocks to host memory; synchronous
 * with the device.  MOE355_EINVAL for a NULL host pointer or a larger count. */
int moe355_phase_trace_read(uint32_t* host, size_t count);

#ifdef __cplusplus
}
#endif

#endif /* MOE355_TRACE_H */

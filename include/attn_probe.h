/*
 * attn_probe.h -- matrix-core throughput probe of the attention library, a
 * measurement utility (not part of the attention computation): the bf16
 * MFMA rate an MI355X sustains with nothing else running, the measured
 * ceiling that the fused kernels are compared with next to the published
 * dense peak ("Attention Mechanism: Computation & Memory Patterns", section
 * 4: the fused pattern should run close to the compute-bound peak).
 */
#ifndef ATTN_PROBE_H_
#define ATTN_PROBE_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueues one probe kernel on `stream`: `workgroups` workgroups of 4 waves,
 * each wave running `iters` trips of independent bf16 MFMA accumulation
 * chains on register operands (shape 0: v_mfma_f32_32x32x16_bf16, 16 per
 * trip; shape 1: v_mfma_f32_16x16x32_bf16, 32 per trip).  sink: caller-owned
 * device float array of workgroups * 256 elements (one value per thread is
 * written so that the work is not optimised away).  Errors: shape not 0/1
 * (ATTN_ERR_ARG), workgroups outside 1..2^20 or iters outside 1..2^31-1
 * (ATTN_ERR_SHAPE), sink NULL or misaligned, launch failure.
 */
attn_status attn_probe_mfma(int shape, int64_t workgroups, int64_t iters,
                            float* sink, hipStream_t stream);

/* FLOPs one attn_probe_mfma call with these arguments performs (0 if they
 * are invalid). */
double attn_probe_mfma_flops(int shape, int64_t workgroups, int64_t iters);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H_ */

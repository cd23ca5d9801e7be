/* On-device peak probes for MI355X (gfx950): the rates the roofline
 * fractions of the SSA kernels are also quoted against, measured on the card
 * that runs them.  Not part of the method: a plain bf16 MFMA loop (the
 * matrix-core ceiling of the routing and attention contractions) and a plain
 * streaming read of device memory (the HBM ceiling of the gather).
 *
 * Conventions as in ssa.h: device pointers, `stream` is a hipStream_t passed
 * as void*, calls are asynchronous on it; the caller times them (HIP events
 * on the same stream) and owns every buffer.  Errors: SSA_ERR_INVALID_ARGUMENT
 * for a null pointer or a non-positive count, SSA_ERR_HIP for a launch error.
 */
#ifndef SSA_MI355X_SSA_PROBES_H
#define SSA_MI355X_SSA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include "ssa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core loop: `workgroups` workgroups of 4 waves, each wave
 * issuing iters x 16 v_mfma_f32_32x32x16_bf16 on 4 independent accumulator
 * chains (32768 flops each).  out: float32 [workgroups], written (a sum of the
 * accumulators, so the loop cannot be elided).  *flops (host) receives the
 * flops the launch performs. */
ssa_status ssa_probe_mfma_bf16(float* out, int32_t workgroups, int32_t iters, double* flops,
                               void* stream);

/* Streaming read of `bytes` bytes at `buf` (16-byte aligned, bytes a multiple
 * of 16) by `workgroups` workgroups of 256 threads, grid-stride, eight 16-byte
 * nontemporal loads in flight per thread.  out: uint32 [workgroups * 256], written (an XOR
 * of what each thread read). */
ssa_status ssa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* out, int32_t workgroups,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSA_MI355X_SSA_PROBES_H */

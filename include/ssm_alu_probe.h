/*
 * ssm_alu_probe.h -- vector-ALU rate probes for gfx950 (libssm_alu_probe.so).
 *
 * A measurement tool beside the scan library, not part of it: the benchmark
 * uses it to price its vector-ALU floors with rates measured on the device
 * (wall time of a launch with a known instruction count) instead of a
 * nominal peak.  The scan's recurrence issues, per state update, one
 * exponential and four plain FP32 operations; these probes time exactly such
 * instructions.
 */
#ifndef SSM_ALU_PROBE_H_
#define SSM_ALU_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Instructions each lane executes in one probe launch of this kind
 * (kinds 2 and 4 count all five instructions of a group). */
int64_t ssm_probe_instructions_per_lane(int kind, int64_t iters);

/*
 * Enqueue one probe launch on hip_stream: one workgroup per compute unit,
 * waves_per_simd (1..4) waves on each of its 4 SIMDs, every lane running
 * `iters` iterations of independent register chains of one instruction kind:
 * 0 = v_fma_f32, 1 = v_exp_f32, 2 = one v_exp_f32 then four v_fma_f32 (each
 * on another chain), 3 = v_mul_f32, 4 = the recurrence's pattern per state
 * (v_mul, v_exp_f32, v_mul, state v_fma_f32, output v_fma_f32).  out (device, out_elems >= CUs * 256 * waves_per_simd fp32)
 * receives one value per lane; *workgroups (host) the workgroup count.
 * Returns 0, 1 on invalid arguments (nothing enqueued), 2 on a HIP error.
 * The caller times the launch (HIP events on the same stream).
 */
int ssm_probe_valu(int kind, int waves_per_simd, int64_t iters, float *out, int64_t out_elems,
                   int *workgroups, void *hip_stream);

/*
 * Enqueue `workgroups` workgroups of `threads` threads (64..1024) that request
 * lds_bytes of LDS each; every wave writes, at out[workgroup * waves + wave]
 * (device int, out_elems >= workgroups * ceil(threads / 64)), the SIMD it
 * runs on (bits 1:0) and its compute unit within the shader array (bits 7:4),
 * read from the HW_ID hardware register.  Returns 0, 1 on invalid arguments
 * (nothing enqueued), 2 on a HIP error.
 */
int ssm_probe_wave_placement(int threads, int lds_bytes, int workgroups, int *out, int64_t out_elems,
                             void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_ALU_PROBE_H_ */

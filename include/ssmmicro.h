/*
 * ssmmicro.h -- C ABI of libssmmicro.so: instruction-rate and bandwidth
 * probes of the GPU that the scan kernels' ALU ceilings are derived from.
 *
 * The selective scan's cost at dstate 16 is set by the plain fp32 VALU
 * issue rate, the transcendental (v_exp_f32) rate, and whether the two
 * overlap (the pages give no figures for any of this; the GPU cost-model
 * section of the Triton vector-addition tutorial names compute, memory and
 * overhead as the three limits).  Each probe launches `blocks` workgroups of
 * 256 threads (four waves, one per SIMD of a compute unit), so
 * blocks = 256 * k places about k waves on every SIMD of a 256-CU device.
 *
 * Probes (`kind`):
 *   SSM_MB_FMA      8 independent v_fma_f32 chains, 128 per loop iteration
 *   SSM_MB_EXP      8 independent v_exp_f32 chains, 128 per iteration
 *   SSM_MB_MIX      the scan step on 4 states, 8 timesteps per iteration:
 *                   per (timestep, state) a multiply, an exp, a multiply and
 *                   two FMAs (4 plain + 1 transcendental), plus one add per
 *                   timestep for the running sum of y: 136 plain and 32 exps
 *                   per iteration
 *   SSM_MB_DPP      8 independent v_mul_f32 with a row_newbcast DPP operand,
 *                   128 per iteration
 *   SSM_MB_LDS_BC   16 ds_read_b128 per iteration, every lane the same address
 *   SSM_MB_LDS_LIN  16 ds_read_b128 per iteration, lane i at 16*i bytes
 *   SSM_MB_LDS_W32  16 ds_write_b32 per iteration, lane i at 4*i bytes
 *   SSM_MB_SIN      8 independent v_sin_f32 chains, 128 per iteration (the
 *                   complex scan's decay takes a sine and a cosine per
 *                   (timestep, state) besides its exp)
 *   SSM_MB_MIXMM    SSM_MB_MIX with each timestep's products B * (delta' u)
 *                   taken by one v_mfma_f32_16x16x4_f32 (an outer product of
 *                   16 states and 16 channels): 104 plain, 32 exps and 8
 *                   MFMAs per iteration; whether the matrix core's work
 *                   overlaps the VALU stream
 *   SSM_MB_COPY     device copy of `iters` 16-byte vectors per thread (grid
 *                   stride, four loads in flight; iters a multiple of 4),
 *                   src = buf, dst = buf + half: bandwidth probe
 *
 * `out` (device, float) receives blocks*256 floats (keeps the work alive;
 * for SSM_MB_COPY it is the buffer, 2 * blocks * 256 * iters * 16 bytes).
 * `clk` (device, 4 x uint64) receives, from thread 0 of block 0, the
 * s_memtime and s_memrealtime counters at its start and its end.
 * Asynchronous on hip_stream; returns 0, 3 for an unknown kind or a
 * non-positive size, 4 for a HIP launch error.
 */
#ifndef SSMMICRO_H
#define SSMMICRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SSM_MB_FMA = 0,
  SSM_MB_EXP = 1,
  SSM_MB_MIX = 2,
  SSM_MB_DPP = 3,
  SSM_MB_LDS_BC = 4,
  SSM_MB_LDS_LIN = 5,
  SSM_MB_LDS_W32 = 6,
  SSM_MB_COPY = 7,
  SSM_MB_SIN = 8,
  SSM_MB_MIXMM = 9
};

int ssm_microbench(int32_t kind, int32_t blocks, int32_t iters, float *out, uint64_t *clk,
                   void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SSMMICRO_H */

/*
 * mlp_ceiling.h -- measurement probe (not part of the inference boundary): the FP16 MFMA throughput
 * the device sustains on random operands, used by the benchmark as a second roofline denominator
 * beside the spec peak.  Built into its own library, libmlp_ceiling.so.
 */
#ifndef MLP_CEILING_H
#define MLP_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch of a loop of independent v_mfma_f32_32x32x16_f16 instructions (8 per iteration,
 * each 32,768 FLOP) on `stream`, 256 threads per workgroup.
 *   valu_per_mfma  0, 6 or 7: independent packed-FP16 VALU instructions issued after each MFMA
 *   grid           workgroups (4 per compute unit = 4 waves per SIMD)
 *   operands       device buffer of at least 32,768 bytes of FP16 data (the MFMA operands)
 *   out            device buffer of grid * 256 floats (keeps the results live)
 *   clk            device buffer of 2 uint64: shader-clock cycles and 100 MHz ticks of one wave
 *   iters          loop iterations, >= 1
 * Returns 0, -1 for a bad argument, -5 if the launch failed. */
int mlp_ceiling_launch(int valu_per_mfma, int grid, const void *operands, float *out, uint64_t *clk, int iters,
                       void *stream);

/* Enqueue one launch of an empty kernel (`grid` workgroups of 64 threads that do nothing) on `stream`:
 * the fixed cost of one dispatch, timed the same way as the inference kernel.
 * Returns 0, -1 if grid < 1, -5 if the launch failed. */
int mlp_ceiling_empty_launch(int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLP_CEILING_H */

// mlp_ceiling.hip -- measured FP16 MFMA ceiling of the device, for the benchmark's roofline.
//
// The spec peak (2,516.6 TFLOP/s dense FP16 on MI355X) assumes the 2.4 GHz clock.  With random
// operands the MFMA pipe draws enough power that the clock drops well below that, so the benchmark
// also reports its kernel against what the chip sustains on the same kind of data: a loop of
// independent v_mfma_f32_32x32x16_f16 instructions (eight per iteration, four accumulators, operands
// cycled through eight fragments of random FP16 data), optionally with K independent packed-FP16
// VALU instructions after each MFMA (the fused kernel's epilogue needs between six and seven per
// MFMA; the conversion, multiply and max it uses each take the same issue time).
// The instruction stream is written as inline assembly so that the count and order are exact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mlp_ceiling.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16x __attribute__((ext_vector_type(16)));

#define MLPC_MFMA(acc, A, B) "v_mfma_f32_32x32x16_f16 " acc ", " A ", " B ", " acc "\n"
#define MLPC_PK(r) "v_pk_mul_f16 " r ", " r ", %[s]\n"
#define MLPC_STEP(acc, A, B)                                                                       \
    MLPC_MFMA(acc, A, B)                                                                           \
    ".if %[k] > 0\n" MLPC_PK("%[v0]") ".endif\n" ".if %[k] > 1\n" MLPC_PK("%[v1]") ".endif\n"      \
    ".if %[k] > 2\n" MLPC_PK("%[v2]") ".endif\n" ".if %[k] > 3\n" MLPC_PK("%[v3]") ".endif\n"      \
    ".if %[k] > 4\n" MLPC_PK("%[v4]") ".endif\n" ".if %[k] > 5\n" MLPC_PK("%[v5]") ".endif\n"      \
    ".if %[k] > 6\n" MLPC_PK("%[v6]") ".endif\n"

template <int K>
__global__ __launch_bounds__(256) void mfma_loop(const h8 *src, float *out, uint64_t *clk, int iters)
{
    const int l = threadIdx.x;
    const h8 a0 = src[l], a1 = src[l + 256], a2 = src[l + 512], a3 = src[l + 768];
    const h8 b0 = src[l + 1024], b1 = src[l + 1280], b2 = src[l + 1536], b3 = src[l + 1792];
    f16x c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    h2 v0 = (h2)(_Float16)1, v1 = v0, v2 = v0, v3 = v0, v4 = v0, v5 = v0, v6 = v0;
    const h2 s = (h2)((_Float16)0.999f);
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        asm volatile(MLPC_STEP("%[c0]", "%[a0]", "%[b0]") MLPC_STEP("%[c1]", "%[a1]", "%[b1]")
                     MLPC_STEP("%[c2]", "%[a2]", "%[b2]") MLPC_STEP("%[c3]", "%[a3]", "%[b3]")
                     MLPC_STEP("%[c0]", "%[a1]", "%[b2]") MLPC_STEP("%[c1]", "%[a2]", "%[b3]")
                     MLPC_STEP("%[c2]", "%[a3]", "%[b0]") MLPC_STEP("%[c3]", "%[a0]", "%[b1]")
                     : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3), [v0] "+v"(v0), [v1] "+v"(v1),
                       [v2] "+v"(v2), [v3] "+v"(v3), [v4] "+v"(v4), [v5] "+v"(v5), [v6] "+v"(v6)
                     : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3), [b0] "v"(b0), [b1] "v"(b1),
                       [b2] "v"(b2), [b3] "v"(b3), [s] "v"(s), [k] "i"(K));
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    const f16x c = c0 + c1 + c2 + c3;
    out[blockIdx.x * blockDim.x + threadIdx.x] = c[0] + c[9] + (float)(v0[0] + v1[1] + v2[0] + v3[1] + v4[0] + v5[1] + v6[0]);
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        clk[0] = t1 - t0;  // shader clock cycles of one wave
        clk[1] = r1 - r0;  // 100 MHz reference ticks over the same interval
    }
}

__global__ __launch_bounds__(64) void empty_kernel() {}

}  // namespace

extern "C" int mlp_ceiling_launch(int valu_per_mfma, int grid, const void *operands, float *out, uint64_t *clk,
                                  int iters, void *stream)
{
    if (grid < 1 || iters < 1 || !operands || !out || !clk)
        return -1;
    switch (valu_per_mfma) {
    case 0: hipLaunchKernelGGL(mfma_loop<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const h8 *)operands, out, clk, iters); break;
    case 6: hipLaunchKernelGGL(mfma_loop<6>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const h8 *)operands, out, clk, iters); break;
    case 7: hipLaunchKernelGGL(mfma_loop<7>, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const h8 *)operands, out, clk, iters); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int mlp_ceiling_empty_launch(int grid, void *stream)
{
    if (grid < 1)
        return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// mlp_registry.h -- the table of compiled kernel instances and how the host launches them.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "mlp.h"

namespace mlpk {

enum Layout { kRowMajor = 0, kPacked = 1, kPackedFp8 = 2 };
enum Act { kVector = 0, kScalarised = 1 };

// Everything one launch needs; passed by value as the kernel argument.
struct LaunchArgs {
    const uint16_t *x;     // [batch][w0] FP16
    uint16_t *y;           // [batch][wL] FP16
    const uint8_t *image;  // device weight image
    int64_t batch;
    int32_t w0;            // caller's input width (row stride of x)
    int32_t wL;            // caller's output width (row stride of y)
};

struct KernelEntry {
    const char *name;
    int n_layers;
    int widths[MLP_FUSED_DEEP_MAX_LAYERS + 1];  // exact instance: the widths it serves; generic: all 64 or all 128 (any shape within)
    bool generic;
    int layout;
    int act;
    int threads;        // threads per workgroup
    int rows_per_wave;  // rows one wave evaluates per loop iteration
    bool weights_in_lds;
    hipError_t (*launch)(const LaunchArgs &, int grid, hipStream_t);
    const void *func;   // kernel symbol, for occupancy queries
    bool vec_io;        // generic instance with vector I/O: input width % 8 == 0, output width % 4 == 0 only
};

// All compiled instances: the FP16 kernels and the FP8 ones.
const KernelEntry *registry(int *count);
const KernelEntry *registry_fp8(int *count);

}  // namespace mlpk

/*
 * mlp_testing.h -- test hooks of the MLP inference library (not part of the inference interface).
 *
 * Conventions as in mlp.h: MLP_OK or a negative mlp_status, host-side validation first.
 */
#ifndef MLP_TESTING_H
#define MLP_TESTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Run the work items of mlp_pack_weights_device's conversion kernel on the host: the same per-item
 * code the kernel runs on the GPU ("Row-major versus InferencingOptimal weights": the one-time
 * conversion recorded into the command stream), here reading host weights and writing a host image,
 * so that its output and every write's extent can be checked on a machine without a GPU.
 *   n_layers, widths, weights, biases, layout  as for mlp_pack_host (every layout the device
 *               conversion serves: packed, row-major, FP8)
 *   host_dst    receives the image; dst_bytes must equal mlp_packed_size
 *   exact_cover set to 1 if every byte of the image was written exactly once and nothing outside it,
 *               else 0 (the image is then incomplete)
 * Host only; no HIP call.  Errors: INVALID_ARGUMENT, UNSUPPORTED. */
int mlp_testing_pack_device_on_host(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                                    const uint16_t *const *biases, int layout, void *host_dst, size_t dst_bytes,
                                    int *exact_cover);

/* The kernel mlp_pack_weights would select for this shape and layout, by the name mlp_kernel_name
 * reports once it is packed: a dedicated or generic fused instance, or the layer-by-layer path.
 *   name  receives the NUL-terminated name (truncated to cap - 1 characters)
 * Host only; no HIP call.  Errors: INVALID_ARGUMENT, UNSUPPORTED (as mlp_packed_size). */
int mlp_testing_plan_kernel(int n_layers, const int32_t *widths, int layout, char *name, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* MLP_TESTING_H */

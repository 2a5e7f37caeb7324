// mlp_pack.h -- host-side construction of the device weight images (see mlp_layout.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mlp_registry.h"

namespace mlpk {

// Bytes of the image for a kernel computing with widths kernel_widths[0..n_layers].
size_t image_bytes(int n_layers, const int *kernel_widths, int layout);

// Write the image for the caller's net (widths[0..n_layers], weights[l] = [widths[l+1]][widths[l]]
// FP16 row-major, biases[l] = [widths[l+1]] FP16) as consumed by a kernel computing with
// kernel_widths (each >= the caller's width; the excess is zero).  dst must hold image_bytes().
void pack_image(int n_layers, const int *widths, const int *kernel_widths, const uint16_t *const *weights,
                const uint16_t *const *biases, int layout, uint8_t *dst);

}  // namespace mlpk

// mlp_pack.h -- host-side construction of the device weight images (see mlp_layout.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "mlp_registry.h"

namespace mlpk {

// Bytes of the image for a kernel computing with widths kernel_widths[0..n_layers].
size_t image_bytes(int n_layers, const int *kernel_widths, int layout);

// Write the image for the caller's net (widths[0..n_layers], weights[l] = [widths[l+1]][widths[l]]
// FP16 row-major, biases[l] = [widths[l+1]] FP16) as consumed by a kernel computing with
// kernel_widths (each >= the caller's width; the excess is zero).  dst must hold image_bytes().
void pack_image(int n_layers, const int *widths, const int *kernel_widths, const uint16_t *const *weights,
                const uint16_t *const *biases, int layout, uint8_t *dst);

// Everything the device packer needs, per layer l (kernel argument, passed by value).  Work items
// [0, first[l]) write the first section (packed: A-fragment slices; row-major: 16-byte chunks of W;
// FP8: 32-byte lane slices of the A fragments), [first[l], mid[l]) the FP8 scale codes (empty for
// the FP16 layouts), [mid[l], items[l]) the biases; a_off / s_off / b_off are the byte offsets of
// the sections.
constexpr int kPackMaxLayers = 16;  // layers one conversion launch takes: every fused network
struct PackArgs {
    const uint16_t *w[kPackMaxLayers];
    const uint16_t *b[kPackMaxLayers];
    int win[kPackMaxLayers], wout[kPackMaxLayers], mt[kPackMaxLayers], kb[kPackMaxLayers];
    int narrow[kPackMaxLayers];  // 1: the narrow last-layer layout of mlp_layout.h (packed layout, one output tile)
    uint32_t a_off[kPackMaxLayers], s_off[kPackMaxLayers], b_off[kPackMaxLayers], first[kPackMaxLayers],
        mid[kPackMaxLayers], items[kPackMaxLayers];
    int layout;
    int natural;  // 1: every layer in natural K order (the layered image), 0: the fused kernels' order
    uint8_t *dst;
};

// Fill everything but w, b and dst for the caller's widths and the kernel's widths kw (a fused network:
// n_layers <= kPackMaxLayers).
void fill_pack_args(int n_layers, const int *widths, const int *kw, int layout, PackArgs &p);

// The layered path's image (mlp_layered.h): bytes, and the host packer.  Layers are packed one after
// another; layer_offset(l) is where layer l starts.
size_t layered_image_bytes(int n_layers, const int *widths);
size_t layered_layer_offset(const int *widths, int l);
void pack_layered(int n_layers, const int *widths, const uint16_t *const *weights, const uint16_t *const *biases,
                  uint8_t *dst);
// Fill args for layers l0 .. l0 + count - 1 (count <= 8) of the layered image (natural K order).
void fill_pack_args_layered(const int *widths, int l0, int count, PackArgs &p);

// Enqueue the device packer on `stream`: it writes the image pack_image would write, from device
// copies of the weights (p.w, p.b) into p.dst.
hipError_t launch_pack(const PackArgs &p, int n_layers, hipStream_t stream);

// Run the device packer's work items on the host, from host weights (p.w, p.b) into dst (bytes long),
// marking each byte written in `written` (bytes entries): false if any item writes outside
// [0, bytes) or onto a byte written before (the kernel's own per-item code, checked on the CPU).
bool pack_items_on_host(const PackArgs &p, int n_layers, uint8_t *dst, size_t bytes, std::vector<uint8_t> &written);

}  // namespace mlpk

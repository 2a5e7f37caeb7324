// mlp_pack.cpp -- one-time conversion of row-major FP16 weights into a device weight image.
//
// "Row-major versus InferencingOptimal weights": the same FP16 row-major matrices are converted
// once, before inference, into a layout chosen for the hardware; the conversion is paid only when
// the weights change.  Here the target is the MFMA-fragment order described in mlp_layout.h.  The
// conversion is a pure permutation and zero padding of FP16 bit patterns; the only arithmetic is the
// exact widening of each FP16 bias to FP32 (the accumulator's initial value).
#include <string.h>

#include "mlp_layered.h"
#include "mlp_layout.h"
#include "mlp_pack.h"

namespace mlpk {

static float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

size_t image_bytes(int n_layers, const int *kernel_widths, int layout)
{
    return layout == kPacked ? mlpl::pk_bytes(kernel_widths, n_layers) : mlpl::rm_bytes(kernel_widths, n_layers);
}

void pack_image(int n_layers, const int *widths, const int *kw, const uint16_t *const *weights,
                const uint16_t *const *biases, int layout, uint8_t *dst)
{
    const size_t total = image_bytes(n_layers, kw, layout);
    memset(dst, 0, total);
    for (int l = 0; l < n_layers; ++l) {
        const int win = widths[l], wout = widths[l + 1];
        const uint16_t *W = weights[l];
        const uint16_t *b = biases[l];
        if (layout == kRowMajor) {
            // Verbatim copies: the kernel reads the canonical matrices as they are.
            memcpy(dst + mlpl::rm_w_off(kw, l), W, (size_t)win * wout * 2);
            memcpy(dst + mlpl::rm_b_off(kw, l), b, (size_t)wout * 2);
            continue;
        }
        const int MT = mlpl::m_tiles(kw, l), KB = mlpl::k_blocks(kw, l);
        uint16_t *A = (uint16_t *)(dst + mlpl::pk_a_off(kw, l));
        for (int mt = 0; mt < MT; ++mt)
            for (int kb = 0; kb < KB; ++kb)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane / 32, m = lane % 32;
                    const int r = mlpl::kTileM * mt + m;
                    uint16_t *frag = A + ((size_t)(mt * KB + kb) * 64 + lane) * 8;
                    for (int j = 0; j < 8; ++j) {
                        const int f = mlpl::slot_feature(l, kb, g, j);
                        frag[j] = (r < wout && f < win) ? W[(size_t)r * win + f] : 0;
                    }
                }
        float *B = (float *)(dst + mlpl::pk_b_off(kw, l));
        for (int mt = 0; mt < MT; ++mt)
            for (int g = 0; g < 2; ++g)
                for (int j = 0; j < 16; ++j) {
                    const int r = mlpl::acc_feature(mt, g, j);
                    B[mt * 32 + g * 16 + j] = r < wout ? half_bits_to_float(b[r]) : 0.0f;
                }
    }
}

size_t layered_layer_offset(const int *widths, int l)
{
    size_t o = 0;
    for (int i = 0; i < l; ++i)
        o += layered_layer_bytes(widths[i], widths[i + 1]);
    return o;
}

size_t layered_image_bytes(int n_layers, const int *widths) { return layered_layer_offset(widths, n_layers); }

void pack_layered(int n_layers, const int *widths, const uint16_t *const *weights, const uint16_t *const *biases,
                  uint8_t *dst)
{
    memset(dst, 0, layered_image_bytes(n_layers, widths));
    for (int l = 0; l < n_layers; ++l) {
        const int win = widths[l], wout = widths[l + 1];
        const int MT = layered_kout(wout) / 32, KB = layered_kin(win) / 16;
        const uint16_t *W = weights[l];
        const uint16_t *b = biases[l];
        uint8_t *base = dst + layered_layer_offset(widths, l);
        uint16_t *A = (uint16_t *)base;
        for (int mt = 0; mt < MT; ++mt)
            for (int kb = 0; kb < KB; ++kb)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane / 32, r = 32 * mt + lane % 32;
                    uint16_t *frag = A + ((size_t)(mt * KB + kb) * 64 + lane) * 8;
                    for (int j = 0; j < 8; ++j) {
                        const int f = 16 * kb + 8 * g + j;  // natural K order
                        frag[j] = (r < wout && f < win) ? W[(size_t)r * win + f] : 0;
                    }
                }
        float *B = (float *)(base + layered_a_bytes(win, wout));
        for (int mt = 0; mt < MT; ++mt)
            for (int g = 0; g < 2; ++g)
                for (int j = 0; j < 16; ++j) {
                    const int r = mlpl::acc_feature(mt, g, j);
                    B[mt * 32 + g * 16 + j] = r < wout ? half_bits_to_float(b[r]) : 0.0f;
                }
    }
}

}  // namespace mlpk

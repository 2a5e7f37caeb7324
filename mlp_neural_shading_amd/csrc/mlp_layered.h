// mlp_layered.h -- the layer-by-layer path for networks beyond the fused kernels (widths > 128, or
// more than 8 layers, or more than 16 when every width is at most 64): geometry of its weight image
// and the per-layer kernel launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mlpk {

// Padded widths of the layered image: every layer's K (input width) to a multiple of 64 (an even
// number of the kernel's 32-deep K steps), every layer's M (output width) to a multiple of 128 (the
// kernel's workgroup tile).
inline int layered_kin(int w) { return (w + 63) / 64 * 64; }
inline int layered_kout(int w) { return (w + 127) / 128 * 128; }

// Per layer l, in order: A fragments [kout/32][kin/16][64 lanes][8 halves] (natural K order: slot
// (kb, g, j) holds input feature 16 kb + 8 g + j), then FP32 bias tiles [kout/32][2][16] (entry
// (mt, g, j) = b[32 mt + 8 (j / 4) + 4 g + j % 4]).  Zero outside the real matrix.
inline size_t layered_a_bytes(int win, int wout) { return (size_t)(layered_kout(wout) / 32) * (layered_kin(win) / 16) * 1024; }
inline size_t layered_b_bytes(int wout) { return (size_t)(layered_kout(wout) / 32) * 128; }
inline size_t layered_layer_bytes(int win, int wout) { return layered_a_bytes(win, wout) + layered_b_bytes(wout); }

// Everything one layer launch needs (kernel argument, by value).
struct LayerArgs {
    const uint16_t *x;  // [rows][ldx] FP16, columns 0..win-1 used
    int64_t ldx;
    uint16_t *y;        // [rows][ldy] FP16, columns 0..wout-1 written
    int64_t ldy;
    const uint8_t *a;   // this layer's A fragments
    const float *bias;  // this layer's bias tiles
    int64_t rows;
    int64_t row_tiles;  // ceil(rows / layered_rows_per_tile())
    int win, wout;      // real widths
    int kin, kout;      // padded widths (layered_kin / layered_kout)
    int act;            // 1: leaky ReLU after the rounding; 0: none (last layer)
    int vec_x;          // 1: rows of x are 16-byte aligned (ldx % 8 == 0, x aligned)
    int vec_y;          // 1: rows of y are 8-byte aligned (ldy % 4 == 0, y aligned)
    int cus;            // compute units of the device (sizes the persistent grid)
};

hipError_t launch_layer(const LayerArgs &p, hipStream_t stream);

// A run of consecutive layers of one chain width (256, 128 or 64) in one launch: each workgroup keeps
// its 256 rows' activations in LDS from the first layer's input to the last layer's output, so only
// the chain's input and output pass through device memory.
constexpr int kChainMaxLayers = 64;
struct ChainArgs {
    const uint16_t *x;  // [rows][ldx] FP16: the first layer's input, kin[0] columns, rows 16-byte aligned
    int64_t ldx;
    uint16_t *y;        // [rows][ldy] FP16: the last layer's wout_last outputs, rows 16-byte aligned (may be x)
    int64_t ldy;
    int width;          // the chain's width: 256, 128 or 64 (outputs computed per layer)
    int wout_last;      // outputs stored from the last layer: a multiple of 8, at most width
    const uint8_t *image;  // the layered weight image
    int64_t rows;
    int64_t row_tiles;     // ceil(rows / 256)
    int n;                 // layers in the chain, 2 .. kChainMaxLayers
    int act_last;          // 1: leaky ReLU after the chain's last layer too
    uint64_t off[kChainMaxLayers];  // byte offset of each layer's A fragments in the image
    int kin[kChainMaxLayers];       // each layer's padded K: 128..256 (width 256), 64 or 128 (128), 64 (64)
};

// The narrowest chain width a layer (real widths win -> wout) can run in, or 0: 256 for 256 padded
// outputs and a padded K of 128..256; 64 for at most 64 outputs and K of 64 (the image pads its
// outputs to 128; the chain skips the zero half); 128 for 128 padded outputs and K of at most 128.
// A chain runs at the widest class of its layers: a 64 layer also runs in a 128-wide chain (its
// outputs 64..127 then computed as the exact zeros of the padded weights), never in a 256-wide one.
inline int layered_chain_class(int win, int wout)
{
    const int kout = layered_kout(wout), kin = layered_kin(win);
    if (kout == 256 && kin >= 128 && kin <= 256)
        return 256;
    if (wout <= 64 && kin == 64)
        return 64;
    if (kout == 128 && kin <= 128)
        return 128;
    return 0;
}

// Whether a layer of class k can join a chain that starts with a layer of class k0 (both non-zero).
inline bool layered_chain_joins(int k0, int k) { return k0 == 256 ? k == 256 : k == 64 || k == 128; }

// Whether the layer-by-layer path runs a whole network (widths w[0..n]) as one chain of 128 or 64
// padded outputs, given input and output rows that are 16-byte aligned (as mlp_infer requires):
// every layer in the chain classes, the input width its own padding, the output width a multiple of
// 8, at most kChainMaxLayers layers.
inline bool layered_one_narrow_chain(int n, const int32_t *w)
{
    if (n < 2 || n > kChainMaxLayers || w[0] != layered_kin(w[0]) || w[n] % 8 != 0)
        return false;
    const int k0 = layered_chain_class(w[0], w[1]);
    if (k0 != 64 && k0 != 128)
        return false;
    for (int l = 0; l < n; ++l)
        if (!layered_chain_joins(k0, layered_chain_class(w[l], w[l + 1])))
            return false;
    return true;
}

hipError_t launch_chain(const ChainArgs &c, hipStream_t stream);

// Rows one workgroup covers (the row tile).
int layered_rows_per_tile();

}  // namespace mlpk

// mlp_pack_device.hip -- the one-time weight conversion as a stream-ordered device kernel.
//
// "Row-major versus InferencingOptimal weights": the conversion from the canonical FP16 row-major
// matrices to the optimal layout can be recorded into the GPU's command stream and run there, from
// weights already resident on the device, instead of on the host.  This kernel writes exactly the
// image the host packer (mlp_pack.cpp) writes -- the same permutation and zero padding of FP16 bit
// patterns and the same exact widening of the biases to FP32 -- so either can feed the inference
// kernels.  One thread writes one 16-byte A-fragment slice (packed) or one 16-byte chunk
// (row-major); one thread writes each 64-byte half of a bias tile.
#include <hip/hip_runtime.h>

#include "mlp_layered.h"
#include "mlp_layout.h"
#include "mlp_pack.h"

namespace mlpk {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(PackArgs p)
{
    const int l = blockIdx.y;
    const int win = p.win[l], wout = p.wout[l];
    const uint16_t *W = p.w[l];
    const uint16_t *b = p.b[l];
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < p.items[l]; i += gridDim.x * blockDim.x) {
        if (p.layout == kPacked) {
            if (i < p.first[l]) {  // A fragments [mt][kb][lane][8]
                const int lane = (int)(i % 64), frag = (int)(i / 64);
                const int kb = frag % p.kb[l], mt = frag / p.kb[l];
                const int g = lane / 32;
                // a narrow last layer has one tile whose lanes carry outputs 0..3 twice (or zeros)
                const int nr = mlpl::narrow_row(lane);
                const int r = p.narrow[l] ? (nr >= 0 ? nr : wout) : mlpl::kTileM * mt + lane % 32;
                uint16_t v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int f = p.natural ? 16 * kb + 8 * g + j : mlpl::slot_feature(l, kb, g, j);
                    v[j] = (r < wout && f < win) ? W[(size_t)r * win + f] : 0;
                }
                *(uint4 *)(p.dst + p.a_off[l] + (size_t)i * 16) = __builtin_bit_cast(uint4, v);
            } else {  // bias tiles [mt][g][16] FP32
                const int k = (int)(i - p.first[l]), mt = k / 2, g = k % 2;
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    // narrow: floats 0..3 and 4..7 of the tile are b[0..3], the rest zero
                    const int r = p.narrow[l] ? (g == 0 && j < 8 ? j % 4 : wout) : mlpl::acc_feature(mt, g, j);
                    v[j] = r < wout ? (float)__builtin_bit_cast(_Float16, b[r]) : 0.0f;
                }
                float4 *d = (float4 *)(p.dst + p.b_off[l] + (size_t)(mt * 32 + g * 16) * 4);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    d[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            }
        } else {  // row-major: W [wout][win] then b [wout], each padded to 16 bytes
            const bool in_w = i < p.first[l];
            const uint32_t c = in_w ? i : i - p.first[l];
            const uint32_t n = in_w ? (uint32_t)wout * win : (uint32_t)wout;
            const uint16_t *src = in_w ? W : b;
            uint16_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = 8 * c + j < n ? src[8 * c + j] : 0;
            *(uint4 *)(p.dst + (in_w ? p.a_off[l] : p.b_off[l]) + (size_t)c * 16) = __builtin_bit_cast(uint4, v);
        }
    }
}

}  // namespace

void fill_pack_args(int n_layers, const int *widths, const int *kw, int layout, PackArgs &p)
{
    p.layout = layout;
    p.natural = 0;
    for (int l = 0; l < n_layers; ++l) {
        p.win[l] = widths[l];
        p.wout[l] = widths[l + 1];
        p.narrow[l] = layout == kPacked && l == n_layers - 1 && mlpl::narrow_last(kw, n_layers);
        p.mt[l] = mlpl::m_tiles(kw, l);
        p.kb[l] = mlpl::k_blocks(kw, l);
        if (layout == kPacked) {
            p.a_off[l] = (uint32_t)mlpl::pk_a_off(kw, l);
            p.b_off[l] = (uint32_t)mlpl::pk_b_off(kw, l);
            p.first[l] = (uint32_t)(p.mt[l] * p.kb[l] * 64);
            p.items[l] = p.first[l] + (uint32_t)(p.mt[l] * 2);
        } else {
            p.a_off[l] = (uint32_t)mlpl::rm_w_off(kw, l);
            p.b_off[l] = (uint32_t)mlpl::rm_b_off(kw, l);
            p.first[l] = (uint32_t)(mlpl::rm_w_bytes(kw, l) / 16);
            p.items[l] = p.first[l] + (uint32_t)(mlpl::rm_b_bytes(kw, l) / 16);
        }
    }
}

void fill_pack_args_layered(const int *widths, int l0, int count, PackArgs &p)
{
    p.layout = kPacked;
    p.natural = 1;
    for (int i = 0; i < count; ++i) {
        const int win = widths[l0 + i], wout = widths[l0 + i + 1];
        const size_t off = layered_layer_offset(widths, l0 + i);
        p.win[i] = win;
        p.wout[i] = wout;
        p.narrow[i] = 0;
        p.mt[i] = layered_kout(wout) / 32;
        p.kb[i] = layered_kin(win) / 16;
        p.a_off[i] = (uint32_t)off;
        p.b_off[i] = (uint32_t)(off + layered_a_bytes(win, wout));
        p.first[i] = (uint32_t)(p.mt[i] * p.kb[i] * 64);
        p.items[i] = p.first[i] + (uint32_t)(p.mt[i] * 2);
    }
}

hipError_t launch_pack(const PackArgs &p, int n_layers, hipStream_t stream)
{
    uint32_t most = 0;
    for (int l = 0; l < n_layers; ++l)
        most = p.items[l] > most ? p.items[l] : most;
    const int blocks = (int)((most + 255) / 256);
    hipLaunchKernelGGL(pack_kernel, dim3(blocks, n_layers), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mlpk

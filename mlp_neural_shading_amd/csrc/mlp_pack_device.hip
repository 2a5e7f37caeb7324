// mlp_pack_device.hip -- the one-time weight conversion as a stream-ordered device kernel.
//
// "Row-major versus InferencingOptimal weights": the conversion from the canonical FP16 row-major
// matrices to the optimal layout can be recorded into the GPU's command stream and run there, from
// weights already resident on the device, instead of on the host.  This kernel writes exactly the
// image the host packer (mlp_pack.cpp) writes -- the same permutation and zero padding of FP16 bit
// patterns, the same exact widening of the biases to FP32, and for the FP8 layout the same row scales
// and E4M3 codes -- so either can feed the inference kernels.  One work item writes one 16-byte
// A-fragment slice (packed) or one 16-byte chunk (row-major) or one lane's 32-byte slice of an FP8
// fragment or one lane's 4 scale codes; one writes each 64-byte half of a bias tile.
//
// The work of one item is a host-and-device function with the destination behind a writer: the
// kernel writes device memory, and pack_items_on_host runs the same function over every item into a
// host buffer through a writer that checks each write's extent (see mlp_pack.h), so the kernel's
// offsets and contents are checked on the CPU against the host packer.
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include <vector>

#include "mlp_layered.h"
#include "mlp_layout.h"
#include "mlp_pack.h"

namespace mlpk {

namespace {

__host__ __device__ inline float half_value(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// E_r of a weight row for the FP8 layout: the smallest E with max |w| <= 448 * 2^E (0 for a zero row).
__host__ __device__ inline int fp8_row_exponent(const uint16_t *row, int n)
{
    float amax = 0.0f;
    for (int k = 0; k < n; ++k)
        amax = fmaxf(amax, fabsf(half_value(row[k])));
    if (amax == 0.0f)
        return 0;
    int E = -40;  // a nonzero binary16 magnitude is at least 2^-24 > 448 * 2^-33
    while (amax > ldexpf(448.0f, E))
        ++E;
    return E;
}

// OCP E4M3 code nearest to v (ties to the even code), the host packer's rounding: values in
// (448, 464] give 448, larger ones NaN.  Binade [2^e, 2^(e+1)) for e in -6..8 has 8 steps of 2^(e-3);
// below 2^-6 the steps are 2^-9 (subnormals).  Every scaling here is by a power of two, so exact.
__host__ __device__ inline uint8_t e4m3_code(float v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    const float a = fabsf(v);
    if (!(a <= 464.0f))
        return sign | 0x7f;
    if (a >= 448.0f)
        return sign | 0x7e;
    if (a < 0.015625f)
        return sign | (uint8_t)rintf(a * 512.0f);  // 0 .. 8; 8 is 2^-6 (exponent field 1)
    int e2 = 0;
    frexpf(a, &e2);
    const int e = e2 - 1;                          // a in [2^e, 2^(e+1))
    const int r = (int)rintf(ldexpf(a, 3 - e));    // 8 .. 16 (16: the next binade)
    return sign | (uint8_t)(((e + 7) << 3) + r - 8);
}

// The work of item i of layer l, written through `out` (out(byte offset, pointer, bytes)).
template <class Out>
__host__ __device__ inline void pack_item(const PackArgs &p, int l, uint32_t i, Out &out)
{
    const int win = p.win[l], wout = p.wout[l];
    const uint16_t *W = p.w[l];
    const uint16_t *b = p.b[l];
    if (p.layout == kPackedFp8) {
        if (i < p.first[l]) {  // A fragments [mt][kb][lane][32 bytes]
            const int lane = (int)(i % 64), frag = (int)(i / 64);
            const int kb = frag % p.kb[l], mt = frag / p.kb[l];
            const int g = lane / 32, r = mlpl::kTileM * mt + lane % 32;
            const int E = r < wout ? fp8_row_exponent(W + (size_t)r * win, win) : 0;
            alignas(16) uint8_t v[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int f = mlpl::f8_slot_feature(l, kb, g, j);
                v[j] = (r < wout && f < win) ? e4m3_code(ldexpf(half_value(W[(size_t)r * win + f]), -E)) : 0;
            }
            out(p.a_off[l] + (size_t)i * 32, v, 32);
        } else if (i < p.mid[l]) {  // scale codes [ceil(MT / 4)][lane][4]: byte k of lane (g, m) is row 32 (4 q + k) + m
            const uint32_t k = i - p.first[l];
            const int lane = (int)(k % 64), q = (int)(k / 64);
            alignas(16) uint8_t v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 32 * (4 * q + t) + lane % 32;
                v[t] = (uint8_t)(127 + (r < wout ? fp8_row_exponent(W + (size_t)r * win, win) : 0));
            }
            out(p.s_off[l] + (size_t)k * 4, v, 4);
        } else {  // bias tiles [mt][g][16] FP32, as in the FP16 image
            const int k = (int)(i - p.mid[l]), mt = k / 2, g = k % 2;
            alignas(16) float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = mlpl::acc_feature(mt, g, j);
                v[j] = r < wout ? half_value(b[r]) : 0.0f;
            }
            out(p.b_off[l] + (size_t)(mt * 32 + g * 16) * 4, v, 64);
        }
    } else if (p.layout == kPacked) {
        if (i < p.first[l]) {  // A fragments [mt][kb][lane][8]
            const int lane = (int)(i % 64), frag = (int)(i / 64);
            const int kb = frag % p.kb[l], mt = frag / p.kb[l];
            const int g = lane / 32;
            // a narrow last layer has one tile whose lanes carry outputs 0..3 twice (or zeros)
            const int nr = mlpl::narrow_row(lane);
            const int r = p.narrow[l] ? (nr >= 0 ? nr : wout) : mlpl::kTileM * mt + lane % 32;
            alignas(16) uint16_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int f = p.natural ? 16 * kb + 8 * g + j : mlpl::slot_feature(l, kb, g, j);
                v[j] = (r < wout && f < win) ? W[(size_t)r * win + f] : 0;
            }
            out(p.a_off[l] + (size_t)i * 16, v, 16);
        } else {  // bias tiles [mt][g][16] FP32
            const int k = (int)(i - p.first[l]), mt = k / 2, g = k % 2;
            alignas(16) float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                // narrow: floats 0..3 and 4..7 of the tile are b[0..3], the rest zero
                const int r = p.narrow[l] ? (g == 0 && j < 8 ? j % 4 : wout) : mlpl::acc_feature(mt, g, j);
                v[j] = r < wout ? half_value(b[r]) : 0.0f;
            }
            out(p.b_off[l] + (size_t)(mt * 32 + g * 16) * 4, v, 64);
        }
    } else {  // row-major: W [wout][win] then b [wout], each padded to 16 bytes
        const bool in_w = i < p.first[l];
        const uint32_t c = in_w ? i : i - p.first[l];
        const uint32_t n = in_w ? (uint32_t)wout * win : (uint32_t)wout;
        const uint16_t *src = in_w ? W : b;
        alignas(16) uint16_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = 8 * c + j < n ? src[8 * c + j] : 0;
        out((in_w ? p.a_off[l] : p.b_off[l]) + (size_t)c * 16, v, 16);
    }
}

// Device writer: whole 16-byte stores where the piece is 16-byte aligned, else 4-byte ones.
struct DeviceOut {
    uint8_t *dst;
    __device__ void operator()(size_t off, const void *src, int bytes) const
    {
        if (bytes % 16 == 0) {
            for (int k = 0; k < bytes; k += 16)
                *(uint4 *)(dst + off + k) = *(const uint4 *)((const uint8_t *)src + k);
        } else {
            for (int k = 0; k < bytes; k += 4)
                *(uint32_t *)(dst + off + k) = *(const uint32_t *)((const uint8_t *)src + k);
        }
    }
};

__global__ __launch_bounds__(256) void pack_kernel(PackArgs p)
{
    const int l = blockIdx.y;
    DeviceOut out{p.dst};
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < p.items[l]; i += gridDim.x * blockDim.x)
        pack_item(p, l, i, out);
}

// Host writer for pack_items_on_host: refuses a write outside the image or onto bytes already written.
struct CheckedHostOut {
    uint8_t *dst;
    size_t bytes;
    std::vector<uint8_t> *written;
    bool ok = true;
    void operator()(size_t off, const void *src, int n)
    {
        if (off + (size_t)n > bytes || off % 4 != 0) {
            ok = false;
            return;
        }
        for (int k = 0; k < n; ++k) {
            if ((*written)[off + k])
                ok = false;
            (*written)[off + k] = 1;
        }
        memcpy(dst + off, src, (size_t)n);
    }
};

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
        if (layout == kPackedFp8) {
            p.kb[l] = mlpl::f8_k_blocks(kw, l);
            p.a_off[l] = (uint32_t)mlpl::f8_a_off(kw, l);
            p.s_off[l] = (uint32_t)mlpl::f8_s_off(kw, l);
            p.b_off[l] = (uint32_t)mlpl::f8_b_off(kw, l);
            p.first[l] = (uint32_t)(p.mt[l] * p.kb[l] * 64);
            p.mid[l] = p.first[l] + (uint32_t)((p.mt[l] + 3) / 4 * 64);
            p.items[l] = p.mid[l] + (uint32_t)(p.mt[l] * 2);
        } else if (layout == kPacked) {
            p.kb[l] = mlpl::k_blocks(kw, l);
            p.a_off[l] = (uint32_t)mlpl::pk_a_off(kw, l);
            p.s_off[l] = 0;
            p.b_off[l] = (uint32_t)mlpl::pk_b_off(kw, l);
            p.first[l] = (uint32_t)(p.mt[l] * p.kb[l] * 64);
            p.mid[l] = p.first[l];
            p.items[l] = p.first[l] + (uint32_t)(p.mt[l] * 2);
        } else {
            p.kb[l] = mlpl::k_blocks(kw, l);
            p.a_off[l] = (uint32_t)mlpl::rm_w_off(kw, l);
            p.s_off[l] = 0;
            p.b_off[l] = (uint32_t)mlpl::rm_b_off(kw, l);
            p.first[l] = (uint32_t)(mlpl::rm_w_bytes(kw, l) / 16);
            p.mid[l] = p.first[l];
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
        p.s_off[i] = 0;
        p.b_off[i] = (uint32_t)(off + layered_a_bytes(win, wout));
        p.first[i] = (uint32_t)(p.mt[i] * p.kb[i] * 64);
        p.mid[i] = p.first[i];
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

bool pack_items_on_host(const PackArgs &p, int n_layers, uint8_t *dst, size_t bytes, std::vector<uint8_t> &written)
{
    CheckedHostOut out{dst, bytes, &written};
    for (int l = 0; l < n_layers; ++l)
        for (uint32_t i = 0; i < p.items[l]; ++i)
            pack_item(p, l, i, out);
    return out.ok;
}

}  // namespace mlpk

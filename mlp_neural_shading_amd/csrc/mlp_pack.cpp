// mlp_pack.cpp -- one-time conversion of row-major FP16 weights into a device weight image.
//
// "Row-major versus InferencingOptimal weights": the same FP16 row-major matrices are converted
// once, before inference, into a layout chosen for the hardware; the conversion is paid only when
// the weights change.  Here the target is the MFMA-fragment order described in mlp_layout.h.  The
// conversion is a pure permutation and zero padding of FP16 bit patterns; the only arithmetic is the
// exact widening of each FP16 bias to FP32 (the accumulator's initial value).
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "mlp_layered.h"
#include "mlp_layout.h"
#include "mlp_pack.h"

namespace mlpk {

static float half_bits_to_float(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

size_t image_bytes(int n_layers, const int *kernel_widths, int layout)
{
    if (layout == kPackedFp8)
        return mlpl::f8_bytes(kernel_widths, n_layers);
    return layout == kPacked ? mlpl::pk_bytes(kernel_widths, n_layers) : mlpl::rm_bytes(kernel_widths, n_layers);
}

// ---- FP8 (OCP E4M3) weights ---------------------------------------------------------------------

// The 127 non-negative finite E4M3 values in code order (increasing): code c = (e << 3) | f is
// f/8 * 2^-6 for e = 0 and (1 + f/8) * 2^(e-7) otherwise; code 0x7f is NaN.
static const double *e4m3_table()
{
    static double t[127];
    static bool init = false;
    if (!init) {
        for (int c = 0; c < 127; ++c) {
            const int e = c >> 3, f = c & 7;
            t[c] = e == 0 ? f / 8.0 / 64.0 : (1.0 + f / 8.0) * std::ldexp(1.0, e - 7);
        }
        init = true;
    }
    return t;
}

// Nearest E4M3 code to v (ties to the even code); magnitudes above 464 give NaN.  The packer only
// converts values it has scaled to at most 448.
static uint8_t e4m3_nearest(double v)
{
    const double *t = e4m3_table();
    const uint8_t sign = std::signbit(v) ? 0x80 : 0;
    const double a = std::fabs(v);
    if (!(a <= 464.0))
        return sign | 0x7f;
    if (a >= t[126])  // 448 .. 464: nearer 448 than the unrepresentable 480 (464 ties to even)
        return sign | 0x7e;
    const int hi = (int)(std::lower_bound(t, t + 127, a) - t);  // first value >= a
    if (t[hi] == a)
        return sign | (uint8_t)hi;
    const int lo = hi - 1;
    const double dlo = a - t[lo], dhi = t[hi] - a;
    const int c = dlo < dhi ? lo : dhi < dlo ? hi : (lo % 2 == 0 ? lo : hi);
    return sign | (uint8_t)c;
}

// Scale exponent of a weight row: the smallest E with max |w| <= 448 * 2^E (0 for a zero row).
static int f8_row_exponent(const uint16_t *row, int n)
{
    float amax = 0.0f;
    for (int k = 0; k < n; ++k)
        amax = std::max(amax, std::fabs(half_bits_to_float(row[k])));
    if (amax == 0.0f)
        return 0;
    int E = 0;
    while ((double)amax > std::ldexp(448.0, E))
        ++E;
    while ((double)amax <= std::ldexp(448.0, E - 1))
        --E;
    return E;
}

static void pack_fp8(int n_layers, const int *widths, const int *kw, const uint16_t *const *weights,
                     const uint16_t *const *biases, uint8_t *dst)
{
    for (int l = 0; l < n_layers; ++l) {
        const int win = widths[l], wout = widths[l + 1];
        const uint16_t *W = weights[l];
        const uint16_t *b = biases[l];
        const int MT = mlpl::m_tiles(kw, l), KB = mlpl::f8_k_blocks(kw, l);
        std::vector<int> E(MT * 32, 0);
        for (int r = 0; r < wout; ++r)
            E[r] = f8_row_exponent(W + (size_t)r * win, win);
        uint8_t *A = dst + mlpl::f8_a_off(kw, l);
        for (int mt = 0; mt < MT; ++mt)
            for (int kb = 0; kb < KB; ++kb)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane / 32, r = mlpl::kTileM * mt + lane % 32;
                    uint8_t *frag = A + ((size_t)(mt * KB + kb) * 64 + lane) * 32;
                    for (int j = 0; j < 32; ++j) {
                        const int f = mlpl::f8_slot_feature(l, kb, g, j);
                        frag[j] = (r < wout && f < win)
                                      ? e4m3_nearest(std::ldexp((double)half_bits_to_float(W[(size_t)r * win + f]), -E[r]))
                                      : 0;
                    }
                }
        uint8_t *S = dst + mlpl::f8_s_off(kw, l);
        for (int q = 0; q < (MT + 3) / 4; ++q)
            for (int lane = 0; lane < 64; ++lane)
                for (int i = 0; i < 4; ++i) {
                    const int r = 32 * (4 * q + i) + lane % 32;
                    S[((size_t)q * 64 + lane) * 4 + i] = (uint8_t)(127 + (r < (int)E.size() ? E[r] : 0));
                }
        float *B = (float *)(dst + mlpl::f8_b_off(kw, l));
        for (int mt = 0; mt < MT; ++mt)
            for (int g = 0; g < 2; ++g)
                for (int j = 0; j < 16; ++j) {
                    const int r = mlpl::acc_feature(mt, g, j);
                    B[mt * 32 + g * 16 + j] = r < wout ? half_bits_to_float(b[r]) : 0.0f;
                }
    }
}

void pack_image(int n_layers, const int *widths, const int *kw, const uint16_t *const *weights,
                const uint16_t *const *biases, int layout, uint8_t *dst)
{
    const size_t total = image_bytes(n_layers, kw, layout);
    memset(dst, 0, total);
    if (layout == kPackedFp8) {
        pack_fp8(n_layers, widths, kw, weights, biases, dst);
        return;
    }
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
        if (l == n_layers - 1 && mlpl::narrow_last(kw, n_layers)) {
            // [kb][lane][8]: output narrow_row(lane) over the slots of group lane / 32, both sample halves
            for (int kb = 0; kb < KB; ++kb)
                for (int lane = 0; lane < 64; ++lane) {
                    const int r = mlpl::narrow_row(lane), g = lane / 32;
                    uint16_t *frag = A + ((size_t)kb * 64 + lane) * 8;
                    for (int j = 0; j < 8; ++j) {
                        const int f = mlpl::slot_feature(l, kb, g, j);
                        frag[j] = (r >= 0 && r < wout && f < win) ? W[(size_t)r * win + f] : 0;
                    }
                }
            float *B = (float *)(dst + mlpl::pk_b_off(kw, l));
            for (int a = 0; a < 2; ++a)
                for (int r = 0; r < wout; ++r)
                    B[4 * a + r] = half_bits_to_float(b[r]);
            continue;
        }
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

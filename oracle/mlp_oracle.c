/*
 * mlp_oracle.c -- TEST INFRASTRUCTURE ONLY.  The CPU oracle for fused FP16 MLP inference.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load this library.
 * The product path (the HIP library under mlp_neural_shading_amd/) never calls it, links it or
 * includes anything from here, and this file includes nothing from there.
 *
 * What it computes ("Profiling neural material inference", section "Experiment setup"): one
 * complete evaluation of an eight-affine-layer network per input row, every row independent.
 * Per layer l (weights W_l stored [out][in] row-major, biases b_l):
 *     acc_j = f32(b_l[j]);  acc_j += f32(W_l[j][i]) * f32(h[i])  for i ascending, in binary32;
 *     y_j   = RNE16(acc_j);
 *     between layers (every layer but the last): y_j = max(y_j, y_j * half(0.01)) in binary16,
 *     the vector form of the leaky ReLU given in section "Bad versus good activation".
 * FP16 storage with FP32 accumulation is the mixed-precision convention described on
 * "Working with Cooperative Matrices", section "Hardware Constraints and Capabilities".
 * The readings taken where the pages are silent (weight orientation, bias placement, rounding
 * mode, summation order, no activation after the output layer) are listed with the design notes.
 *
 * Deliberately plain: single thread, scalar loops, no blocking, no reordering, its own
 * IEEE 754 binary16 codec written from the format's definition (1 sign bit, 5 exponent bits
 * with bias 15, 10 fraction bits; subnormals have exponent field 0 and value f * 2^-24).
 * Build with -O2 -fno-fast-math -ffp-contract=off.  (Every fp16 x fp16 product is exact in
 * binary32 -- 11 + 11 significant bits -- so contraction could not change a result anyway.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------------------- */
/* binary16 codec                                                                           */
/* ---------------------------------------------------------------------------------------- */

/* Exact widening binary16 -> binary32 (every binary16 value is a binary32 value). */
float oracle_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    float mag;
    if (e == 0) {
        mag = ldexpf((float)f, -24); /* subnormal (or zero): f * 2^-24 */
    } else if (e == 31) {
        mag = f ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* binary32 -> binary16, round to nearest, ties to even (the IEEE default rounding).
 *
 * Let q be the spacing of binary16 values in the binade of |x| (2^-24 below 2^-14, where the
 * subnormals live, else 2^(e-10) for |x| in [2^e, 2^(e+1))).  Then |x|/q is exact in double,
 * rint() rounds it to the nearest integer with ties to even (default rounding mode), and the
 * rounded magnitude r*q is re-encoded.  A carry r == 2048 (or r == 1024 from the subnormal
 * range) lands exactly on the next binade's encoding, and a carry out of the largest binade
 * lands on the infinity encoding 0x7c00. */
uint16_t oracle_f32_to_f16(float x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xfe00 : 0x7e00);
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs((double)x);
    if (isinf(x))
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        const double r = rint(a / ldexp(1.0, -24)); /* 0 .. 1024 */
        return sign | (uint16_t)r;                  /* 1024 encodes 2^-14 (exponent field 1) */
    }
    int e2;
    frexp(a, &e2);        /* a = m * 2^e2, m in [0.5, 1)  =>  a in [2^(e2-1), 2^e2) */
    const int e = e2 - 1; /* a in [2^e, 2^(e+1)) */
    if (e > 15)
        return sign | 0x7c00;
    const double r = rint(a / ldexp(1.0, e - 10)); /* 1024 .. 2048 */
    const uint32_t bits = ((uint32_t)(e + 15) << 10) + (uint32_t)(r - 1024.0);
    return sign | (uint16_t)(bits >= 0x7c00 ? 0x7c00 : bits);
}

/* ---------------------------------------------------------------------------------------- */
/* activation                                                                               */
/* ---------------------------------------------------------------------------------------- */

/* half(0.01): 0.01 rounded to binary16 = 0x211f = 1311 * 2^-17 = 0.01000213623046875. */
#define ORACLE_SLOPE_BITS 0x211fu

/* Leaky ReLU in binary16, the whole-vector form max(v, v * half(0.01)): the product of two
 * binary16 values is exact in binary32, so RNE16 of it is the single binary16 rounding of the
 * product. */
uint16_t oracle_leaky_f16(uint16_t v)
{
    const float fv = oracle_f16_to_f32(v);
    const uint16_t scaled = oracle_f32_to_f16(fv * oracle_f16_to_f32(ORACLE_SLOPE_BITS));
    const float fs = oracle_f16_to_f32(scaled);
    return (fs > fv) ? scaled : v;
}

/* ---------------------------------------------------------------------------------------- */
/* the network                                                                              */
/* ---------------------------------------------------------------------------------------- */

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1 };

#define ORACLE_MAX_WIDTH 4096

/* Evaluate rows [0, rows) of x (row-major [rows][widths[0]], binary16 bits) through the net and
 * write y (row-major [rows][widths[n_layers]]).  weights[l] is [widths[l+1]][widths[l]] row-major,
 * biases[l] is [widths[l+1]]; all binary16 bits.  Leaky ReLU follows every layer except the last. */
int oracle_mlp_forward(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                       const uint16_t *const *biases, int64_t rows, const uint16_t *x, uint16_t *y)
{
    if (n_layers < 1 || !widths || !weights || !biases || rows < 0 || (rows > 0 && (!x || !y)))
        return ORACLE_BAD_ARG;
    for (int l = 0; l <= n_layers; ++l)
        if (widths[l] < 1 || widths[l] > ORACLE_MAX_WIDTH)
            return ORACLE_BAD_ARG;

    uint16_t h[ORACLE_MAX_WIDTH], next[ORACLE_MAX_WIDTH];
    const int w_in0 = widths[0], w_out_last = widths[n_layers];
    for (int64_t r = 0; r < rows; ++r) {
        memcpy(h, x + r * w_in0, sizeof(uint16_t) * (size_t)w_in0);
        for (int l = 0; l < n_layers; ++l) {
            const int w_in = widths[l], w_out = widths[l + 1];
            const uint16_t *W = weights[l];
            const uint16_t *b = biases[l];
            for (int j = 0; j < w_out; ++j) {
                float acc = oracle_f16_to_f32(b[j]);
                for (int i = 0; i < w_in; ++i)
                    acc = acc + oracle_f16_to_f32(W[(size_t)j * w_in + i]) * oracle_f16_to_f32(h[i]);
                uint16_t o = oracle_f32_to_f16(acc);
                if (l + 1 < n_layers)
                    o = oracle_leaky_f16(o);
                next[j] = o;
            }
            memcpy(h, next, sizeof(uint16_t) * (size_t)w_out);
        }
        memcpy(y + r * w_out_last, h, sizeof(uint16_t) * (size_t)w_out_last);
    }
    return ORACLE_OK;
}

/* Row subset: evaluate the rows listed in row_index (each an index into x) and write them, in
 * list order, to y ([count][widths[n_layers]]).  Used to check sampled rows of large batches. */
int oracle_mlp_forward_rows(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                            const uint16_t *const *biases, const uint16_t *x, int64_t count,
                            const int64_t *row_index, uint16_t *y)
{
    if (n_layers < 1 || !widths || count < 0 || (count > 0 && (!x || !y || !row_index)))
        return ORACLE_BAD_ARG;
    const int w0 = widths[0], wl = widths[n_layers];
    for (int64_t k = 0; k < count; ++k) {
        const int rc = oracle_mlp_forward(n_layers, widths, weights, biases, 1,
                                          x + row_index[k] * w0, y + k * wl);
        if (rc != ORACLE_OK)
            return rc;
    }
    return ORACLE_OK;
}

/* Array forms of the codec and activation, so the tests can sweep every bit pattern. */
void oracle_f32_to_f16_array(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_f16(in[i]);
}

void oracle_f16_to_f32_array(int64_t n, const uint16_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f32(in[i]);
}

void oracle_leaky_f16_array(int64_t n, const uint16_t *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_leaky_f16(in[i]);
}

/* ---------------------------------------------------------------------------------------- */
/* the FP8 variant                                                                          */
/* ---------------------------------------------------------------------------------------- */
/*
 * A lower-precision form of the same network (beyond the FP16 path, the pages point to lower
 * precisions and to block-scaled formats that carry one power-of-two scale per block of elements).
 * Readings taken here, listed with the design notes:
 *   - format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 fraction bits; subnormals
 *     f * 2^-9; the code S.1111.111 is NaN, there is no infinity, the largest finite value is 448);
 *   - conversion to E4M3: round to nearest, ties to even; a magnitude above 464 (the midpoint
 *     between 448 and the next, unrepresentable step 480) becomes NaN -- no saturation;
 *   - weights: each output row r of W_l gets the power of two 2^E_r with the smallest E_r such that
 *     max_k |W_l[r][k]| <= 448 * 2^E_r (E_r = 0 for an all-zero row); q = E4M3(W / 2^E_r);
 *   - activations: each layer's input h (binary16) is stored as x8 = E4M3(16 * h);
 *   - layer: acc = f32(b[r]) + sum_k (q[r][k] * 2^E_r) * (x8[k] * 2^-4) in binary32, k ascending
 *     (every product is exact in binary32), then RNE16 and the binary16 leaky ReLU as in the FP16
 *     network, none after the last layer.
 */

/* Value of an E4M3 code. */
float oracle_e4m3_to_f32(uint8_t c)
{
    const int sign = (c >> 7) & 1, e = (c >> 3) & 0xf, f = c & 7;
    float mag;
    if (e == 0xf && f == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexpf((float)f, -9); /* f/8 * 2^-6 */
    else
        mag = ldexpf((float)(8 + f), e - 10); /* (1 + f/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* binary32 -> E4M3, nearest even, NaN above 464 (same scheme as the binary16 encoder: the
 * magnitude over the binade's spacing is exact in double and rint() rounds it, ties to even). */
uint8_t oracle_f32_to_e4m3(float x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    if (isnan(x))
        return sign | 0x7f;
    const double a = fabs((double)x);
    if (a > 464.0)
        return sign | 0x7f;
    if (a < ldexp(1.0, -6)) {
        const double r = rint(a / ldexp(1.0, -9)); /* 0 .. 8; 8 encodes 2^-6 (exponent field 1) */
        return sign | (uint8_t)r;
    }
    int e2;
    frexp(a, &e2);
    const int e = e2 - 1;                        /* a in [2^e, 2^(e+1)), e in -6 .. 8 */
    const double r = rint(a / ldexp(1.0, e - 3)); /* 8 .. 16 */
    return sign | (uint8_t)(((e + 7) << 3) + (int)(r - 8.0));
}

/* E_r of a weight row of binary16 values: the smallest E with max |w| <= 448 * 2^E. */
int oracle_fp8_row_exponent(const uint16_t *row, int n)
{
    double amax = 0.0;
    for (int k = 0; k < n; ++k) {
        const double a = fabs((double)oracle_f16_to_f32(row[k]));
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0)
        return 0;
    int E = -60;
    while (amax > ldexp(448.0, E))
        ++E;
    return E;
}

/* The FP8 network on rows of x (binary16 bits), as described above. */
int oracle_mlp_forward_fp8(int n_layers, const int32_t *widths, const uint16_t *const *weights,
                           const uint16_t *const *biases, int64_t rows, const uint16_t *x, uint16_t *y)
{
    if (n_layers < 1 || !widths || !weights || !biases || rows < 0 || (rows > 0 && (!x || !y)))
        return ORACLE_BAD_ARG;
    for (int l = 0; l <= n_layers; ++l)
        if (widths[l] < 1 || widths[l] > ORACLE_MAX_WIDTH)
            return ORACLE_BAD_ARG;
    /* quantise every layer's weights once */
    float *wq[64];
    if (n_layers > 64)
        return ORACLE_BAD_ARG;
    for (int l = 0; l < n_layers; ++l) {
        const int win = widths[l], wout = widths[l + 1];
        wq[l] = (float *)malloc(sizeof(float) * (size_t)win * wout);
        for (int r = 0; r < wout; ++r) {
            const uint16_t *row = weights[l] + (size_t)r * win;
            const int E = oracle_fp8_row_exponent(row, win);
            for (int k = 0; k < win; ++k) {
                const uint8_t q = oracle_f32_to_e4m3(ldexpf(oracle_f16_to_f32(row[k]), -E));
                wq[l][(size_t)r * win + k] = ldexpf(oracle_e4m3_to_f32(q), E);
            }
        }
    }
    uint16_t h[ORACLE_MAX_WIDTH], next[ORACLE_MAX_WIDTH];
    float xq[ORACLE_MAX_WIDTH];
    for (int64_t r = 0; r < rows; ++r) {
        memcpy(h, x + r * widths[0], sizeof(uint16_t) * widths[0]);
        for (int l = 0; l < n_layers; ++l) {
            const int win = widths[l], wout = widths[l + 1];
            for (int k = 0; k < win; ++k)
                xq[k] = ldexpf(oracle_e4m3_to_f32(oracle_f32_to_e4m3(16.0f * oracle_f16_to_f32(h[k]))), -4);
            for (int j = 0; j < wout; ++j) {
                float acc = oracle_f16_to_f32(biases[l][j]);
                for (int k = 0; k < win; ++k)
                    acc = acc + wq[l][(size_t)j * win + k] * xq[k];
                uint16_t v = oracle_f32_to_f16(acc);
                if (l + 1 < n_layers)
                    v = oracle_leaky_f16(v);
                next[j] = v;
            }
            memcpy(h, next, sizeof(uint16_t) * wout);
        }
        memcpy(y + r * widths[n_layers], h, sizeof(uint16_t) * widths[n_layers]);
    }
    for (int l = 0; l < n_layers; ++l)
        free(wq[l]);
    return ORACLE_OK;
}

/* Array forms of the E4M3 codec (for the exhaustive checks). */
void oracle_f32_to_e4m3_array(int64_t n, const float *x, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_e4m3(x[i]);
}

void oracle_e4m3_to_f32_array(int64_t n, const uint8_t *c, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_to_f32(c[i]);
}

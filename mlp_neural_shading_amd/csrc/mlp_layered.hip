// mlp_layered.hip -- networks beyond the fused kernels: layer-by-layer MFMA GEMMs with the fused
// epilogue.
//
// The fused kernels keep a whole network's weights in LDS and its activations in registers, which
// bounds them to widths <= 128 and 8 layers.  Wider or deeper networks run here, one kernel per layer:
//   Y[r][o] = act(RNE16(b[o] + sum_k W[o][k] * X[r][k]))   (FP16 x FP16 products, FP32 accumulation;
//   act = the leaky ReLU max(v, v * half(0.01)) in FP16 for every layer but the last)
// -- the same arithmetic as the fused path ("Profiling neural material inference", "Experiment
// setup" and "Bad versus good activation"), with the activations between layers in device memory.
//
// Tiling (v_mfma_f32_32x32x16_f16, weights = A operand, rows = B operand, as in the fused kernel):
//   - a workgroup (4 waves) computes 128 outputs x 128 rows; wave (wm, wn) the 64 x 64 quarter
//     (wm, wn), i.e. 2 x 2 MFMA tiles, so every A and B fragment read from LDS feeds two MFMAs;
//   - K advances 32 at a time; the next 32 are loaded from global memory into registers while the
//     current ones are multiplied, then written to the other half of a double-buffered LDS tile;
//   - the weight image is fragment-ordered per layer (natural K order: slot (kb, g, j) = feature
//     16 kb + 8 g + j), so a fragment is one 16-byte LDS read per lane; the activation tile is kept
//     as rows of 32 halves padded to 40 (80-byte stride: 16 consecutive rows start 4 banks apart,
//     "Optimization Techniques", "Avoiding Bank Conflicts");
//   - the bias is the C operand of the first MFMA of each output tile; the epilogue converts FP32 ->
//     FP16 (nearest even), applies the leaky ReLU on packed FP16 and stores 4 outputs per lane.
//   - workgroups are numbered so that each XCD takes a contiguous run of (row tile, output tile)
//     pairs, output tiles fastest: the workgroups that share a row tile share that XCD's L2.
#include <hip/hip_runtime.h>

#include "mlp_layered.h"

namespace mlpk {

namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;         // outputs per workgroup
constexpr int kBN = 128;         // rows per workgroup
constexpr int kBK = 32;          // K per step
constexpr int kThreads = 256;    // 4 waves
constexpr int kRowHalves = 40;   // LDS row of the activation tile: 32 halves + 8 of padding
constexpr int kABytes = (kBM / 32) * (kBK / 16) * 1024;  // 8 fragments of 1 KB
constexpr int kBBytes = kBN * kRowHalves * 2;            // 10 KB

__device__ __forceinline__ _Float16 slope() { return __builtin_bit_cast(_Float16, (unsigned short)0x211f); }

// One 16-byte chunk (8 halves) of row `row`, columns c .. c+7 of X; zero past the rows or columns.
__device__ __forceinline__ h8 load_x8(const LayerArgs &p, int64_t row, int c)
{
    h8 v = (h8)(_Float16)0;
    if (row >= p.rows)
        return v;
    const _Float16 *xr = (const _Float16 *)p.x + row * p.ldx;
    if (p.vec_x && c + 8 <= p.win)
        return *(const h8 *)(xr + c);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (c + j < p.win)
            v[j] = xr[c + j];
    return v;
}

// Four waves per SIMD (128 registers, no spills; four 36 KB workgroups per CU): more workgroups
// in flight hide more of the operand loads' latency (-2.5 % on 1024-wide layers, -4 % on 256-wide
// ones against three).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void layer_gemm(LayerArgs p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kABytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kBBytes];

    // Workgroup -> (row tile, output tile): XCD x = b % 8 takes the x-th contiguous run of tiles.
    const int64_t n_out = p.kout / kBM;
    const int64_t n_tiles = p.row_tiles * n_out;
    const int64_t per_xcd = (n_tiles + 7) / 8;
    const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= n_tiles)
        return;  // whole workgroup: no barrier has been reached yet
    const int64_t rt = t / n_out;
    const int ot = (int)(t % n_out);
    const int64_t row0 = rt * kBN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, n = lane & 31;
    const int KB = p.kin / 16;  // fragments per output tile of the image
    const int steps = p.kin / kBK;

    // Global sources of this thread's share of a K step: two A chunks and two B chunks of 16 bytes.
    //   A: chunk q = tid + 256 i (i = 0, 1) of the 8 KB tile: fragment f = q / 64 = (mt, kb) with
    //      mt = f / 2, kb = f % 2, lane slice q % 64 (the LDS tile keeps this order).
    //   B: row s = tid / 2, columns 16 (tid % 2) + 8 i.
    const uint8_t *a_tile = p.a + (size_t)(ot * (kBM / 32)) * KB * 1024;
    const int bs = tid >> 1, bc = (tid & 1) * 16;

    // Named registers rather than arrays indexed in helper lambdas: the compiler placed those in
    // scratch memory.
    uint4 ra0, ra1;
    h8 rb0, rb1;
    const int fa0 = tid >> 6, fa1 = (tid + kThreads) >> 6;  // fragments (mt, kb) = (f >> 1, f & 1)
    const size_t lane16 = (size_t)(tid & 63) * 16;
#define MLPL_LOAD_STEP(step)                                                                                   \
    do {                                                                                                       \
        ra0 = *(const uint4 *)(a_tile + ((size_t)(fa0 >> 1) * KB + (step) * 2 + (fa0 & 1)) * 1024 + lane16);  \
        ra1 = *(const uint4 *)(a_tile + ((size_t)(fa1 >> 1) * KB + (step) * 2 + (fa1 & 1)) * 1024 + lane16);  \
        rb0 = load_x8(p, row0 + bs, (step) * kBK + bc);                                                        \
        rb1 = load_x8(p, row0 + bs, (step) * kBK + bc + 8);                                                    \
    } while (0)
#define MLPL_STORE_STEP(buf)                                                                                   \
    do {                                                                                                       \
        *(uint4 *)(lds_a[buf] + tid * 16) = ra0;                                                               \
        *(uint4 *)(lds_a[buf] + (tid + kThreads) * 16) = ra1;                                                  \
        *(h8 *)(lds_b[buf] + (bs * kRowHalves + bc) * 2) = rb0;                                                \
        *(h8 *)(lds_b[buf] + (bs * kRowHalves + bc + 8) * 2) = rb1;                                            \
    } while (0)

    // Bias tiles of this wave's two output tiles (the C operand of the first MFMA).
    f16x acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int mtg = ot * (kBM / 32) + 2 * wm + i;  // output tile in the layer
        const f4 *bt = (const f4 *)(p.bias + mtg * 32 + g * 16);
        const f4 b0 = bt[0], b1 = bt[1], b2 = bt[2], b3 = bt[3];
        f16x b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = b0[j];
            b[4 + j] = b1[j];
            b[8 + j] = b2[j];
            b[12 + j] = b3[j];
        }
        acc[i][0] = b;
        acc[i][1] = b;
    }

    MLPL_LOAD_STEP(0);
    MLPL_STORE_STEP(0);
    __syncthreads();
    for (int step = 0; step < steps; ++step) {
        const int buf = step & 1;
        if (step + 1 < steps)
            MLPL_LOAD_STEP(step + 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            h8 af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[i] = *(const h8 *)(lds_a[buf] + (((2 * wm + i) * 2 + kb) * 64 + lane) * 16);
                bf[i] = *(const h8 *)(lds_b[buf] + ((64 * wn + 32 * i + n) * kRowHalves + kb * 16 + 8 * g) * 2);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (step + 1 < steps) {
            MLPL_STORE_STEP(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: lane (g, n) holds, for row 64 wn + 32 j + n, outputs 32 mt + 8 q + 4 g + i.
    const h4 s4 = (h4)slope();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int cbase = (ot * (kBM / 32) + 2 * wm + i) * 32 + 4 * g;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t row = row0 + 64 * wn + 32 * j + n;
            if (row >= p.rows)
                continue;
            _Float16 *yr = (_Float16 *)p.y + row * p.ldy;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = cbase + 8 * q;
                const f4 part = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                h4 v = __builtin_convertvector(part, h4);  // nearest even
                if (p.act)
                    v = __builtin_elementwise_max(v, v * s4);
                if (p.vec_y && c + 4 <= p.wout) {
                    *(h4 *)(yr + c) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c + e < p.wout)
                            yr[c + e] = v[e];
                }
            }
        }
    }
#undef MLPL_LOAD_STEP
#undef MLPL_STORE_STEP
}

}  // namespace

hipError_t launch_layer(const LayerArgs &p, hipStream_t stream)
{
    const int64_t tiles = p.row_tiles * (p.kout / kBM);
    hipLaunchKernelGGL(layer_gemm, dim3((unsigned)((tiles + 7) / 8 * 8)), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

int layered_rows_per_tile() { return kBN; }

}  // namespace mlpk

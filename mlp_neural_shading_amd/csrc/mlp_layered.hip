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
//   - a workgroup (4 waves) computes 128 outputs x 256 rows; each wave owns 64 rows (two 32-row
//     sample tiles) and all 128 outputs (four output tiles), so every A fragment read from LDS feeds
//     two MFMAs and every B fragment four;
//   - the rows are the B operand straight from global memory: lane (g, n) loads the 16 bytes of row
//     n at columns 16 kb + 8 g .. + 8, one K step ahead, so activations never pass through LDS (no
//     other wave uses them).  Rows past the batch load the last row instead; their outputs are
//     never stored, and each output row depends on its own input row only;
//   - the weights are shared by the four waves through a double-buffered LDS tile, K advancing 32 at
//     a time: each step's tile is requested two steps ahead into one of two sets of staging
//     registers and stored into LDS at the end of the step before it is used; the weight image is
//     fragment-ordered per layer (natural K order: slot (kb, g, j) = feature
//     16 kb + 8 g + j), so a fragment is one 16-byte LDS read per lane;
//   - the bias is the C operand of the first MFMA of each output tile; the epilogue converts FP32 ->
//     FP16 (nearest even), applies the leaky ReLU on packed FP16 and stores 4 outputs per lane.
//   - workgroups are numbered so that each XCD takes a contiguous run of (row tile, output tile)
//     pairs, output tiles fastest: the workgroups that read the same rows share that XCD's L2.
#include <hip/hip_runtime.h>

#include "mlp_layered.h"

namespace mlpk {

namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;         // outputs per workgroup
constexpr int kBN = 256;         // rows per workgroup (64 per wave)
constexpr int kBK = 32;          // K per step
constexpr int kThreads = 256;    // 4 waves
constexpr int kABytes = (kBM / 32) * (kBK / 16) * 1024;  // 8 fragments of 1 KB

__device__ __forceinline__ _Float16 slope() { return __builtin_bit_cast(_Float16, (unsigned short)0x211f); }

// One 16-byte chunk (8 halves) of a row, columns c .. c+7; zero past the row's win columns.  WHOLE:
// the rows are 16-byte aligned and win equals the padded K, so every chunk is one load.
template <bool WHOLE>
__device__ __forceinline__ h8 load_x8(const LayerArgs &p, const _Float16 *xr, int c)
{
    if (WHOLE || (p.vec_x && c + 8 <= p.win))
        return *(const h8 *)(xr + c);
    h8 v = (h8)(_Float16)0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (c + j < p.win)
            v[j] = xr[c + j];
    return v;
}

// Two waves per SIMD: the 128 accumulator registers, two steps of B fragments, the eight A fragments
// of a step and two sets of weight staging need ~240 registers per lane.
template <bool WHOLE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void layer_gemm(LayerArgs p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kABytes];

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
    const int g = lane >> 5, n = lane & 31;
    const int KB = p.kin / 16;  // fragments per output tile of the image
    const int steps = p.kin / kBK;

    // This thread's share of a K step of the weight tile: chunk q = tid + 256 i (i = 0, 1) of the
    // 8 KB tile, fragment f = q / 64 = (mt, kb) with mt = f / 2, kb = f % 2, lane slice q % 64 (the
    // LDS tile keeps this order).
    const uint8_t *a_tile = p.a + (size_t)(ot * (kBM / 32)) * KB * 1024;
    const int fa0 = tid >> 6, fa1 = (tid + kThreads) >> 6;
    const size_t lane16 = (size_t)(tid & 63) * 16;
    // This lane's two rows (sample tiles j = 0, 1), clamped to the batch.
    const _Float16 *xr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t row = row0 + 64 * wave + 32 * j + n;
        xr[j] = (const _Float16 *)p.x + (row < p.rows ? row : p.rows - 1) * p.ldx;
    }

    // Named registers rather than arrays indexed in helper lambdas: the compiler placed those in
    // scratch memory.
    uint4 ra0, ra1, rb0, rb1;  // weight staging of the even (ra) and the odd (rb) K steps
    h8 bc[2][2], bn[2][2];  // [kb][j]: B fragments of the even and the odd K steps
#define MLPL_LOAD_A(R0, R1, step)                                                                              \
    do {                                                                                                       \
        R0 = *(const uint4 *)(a_tile + ((size_t)(fa0 >> 1) * KB + (step) * 2 + (fa0 & 1)) * 1024 + lane16);   \
        R1 = *(const uint4 *)(a_tile + ((size_t)(fa1 >> 1) * KB + (step) * 2 + (fa1 & 1)) * 1024 + lane16);   \
    } while (0)
#define MLPL_LOAD_B(dst, step)                                                                                 \
    do {                                                                                                       \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                                       \
            _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                      \
                dst[kb][j] = load_x8<WHOLE>(p, xr[j], (step) * kBK + 16 * kb + 8 * g);                         \
    } while (0)
#define MLPL_STORE_A(R0, R1, buf)                                                                              \
    do {                                                                                                       \
        *(uint4 *)(lds_a[buf] + tid * 16) = R0;                                                                \
        *(uint4 *)(lds_a[buf] + (tid + kThreads) * 16) = R1;                                                   \
    } while (0)

    // Bias tiles of the four output tiles (the C operand of the first MFMA).
    f16x acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int mtg = ot * (kBM / 32) + i;  // output tile in the layer
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

    // One K step: multiply with CUR (this step's B fragments) and the LDS tile `buf`.  A step with a
    // successor first requests the next step's rows (into NXT) and, with two successors, the weights
    // two steps ahead (into the staging set RL, stored a step ago); it ends by storing the next step's
    // weights (RS, requested a step ago) into the other LDS tile.  The K loop alternates the B buffers
    // and the staging sets and has no branch inside, so no fragment is copied and each load is first
    // waited for where it is used.  Scheduling barriers hold the loads at the top of the step and the
    // LDS store at its end: otherwise the compiler moves them next to each other and the store waits
    // a full round trip.
#define MLPL_MFMAS(step, CUR)                                                                                  \
    do {                                                                                                       \
        const int buf = (step) & 1;                                                                            \
        h8 af[2][4];                                                                                           \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                                       \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
                af[kb][i] = *(const h8 *)(lds_a[buf] + ((i * 2 + kb) * 64 + lane) * 16);                       \
        /* all eight fragment reads in flight before the first MFMA: left to itself the compiler */          \
        /* interleaves them in pairs, and each pair waits out the LDS latency */                                \
        asm volatile("" ::"v"(af[0][0]), "v"(af[0][1]), "v"(af[0][2]), "v"(af[0][3]), "v"(af[1][0]),           \
                     "v"(af[1][1]), "v"(af[1][2]), "v"(af[1][3]));                                             \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                                       \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
                _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kb][i], CUR[kb][j], acc[i][j], 0, 0, 0); \
    } while (0)
#define MLPL_STEP(step, CUR, NXT, RL0, RL1, RS0, RS1, LOADA)                                                   \
    do {                                                                                                       \
        if (LOADA)                                                                                             \
            MLPL_LOAD_A(RL0, RL1, (step) + 2);                                                                 \
        MLPL_LOAD_B(NXT, (step) + 1);                                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
        MLPL_MFMAS(step, CUR);                                                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
        MLPL_STORE_A(RS0, RS1, ((step) & 1) ^ 1);                                                              \
        __syncthreads();                                                                                       \
    } while (0)

    // kin is a multiple of 64, so the number of steps is even (and at least 2).
    MLPL_LOAD_A(ra0, ra1, 0);
    MLPL_LOAD_A(rb0, rb1, 1);
    MLPL_LOAD_B(bc, 0);
    MLPL_STORE_A(ra0, ra1, 0);
    __syncthreads();
    for (int step = 0; step + 2 < steps; step += 2) {
        MLPL_STEP(step, bc, bn, ra0, ra1, rb0, rb1, true);
        MLPL_STEP(step + 1, bn, bc, rb0, rb1, ra0, ra1, true);
    }
    MLPL_STEP(steps - 2, bc, bn, ra0, ra1, rb0, rb1, false);
    MLPL_MFMAS(steps - 1, bn);

    // Epilogue: lane (g, n) holds, for row 64 wave + 32 j + n, outputs 32 mt + 8 q + 4 g + i.
    const h4 s4 = (h4)slope();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int cbase = (ot * (kBM / 32) + i) * 32 + 4 * g;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t row = row0 + 64 * wave + 32 * j + n;
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
#undef MLPL_LOAD_A
#undef MLPL_LOAD_B
#undef MLPL_STORE_A
#undef MLPL_MFMAS
#undef MLPL_STEP
}

}  // namespace

hipError_t launch_layer(const LayerArgs &p, hipStream_t stream)
{
    const int64_t tiles = p.row_tiles * (p.kout / kBM);
    const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
    if (p.vec_x && p.win == p.kin)
        hipLaunchKernelGGL(layer_gemm<true>, grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(layer_gemm<false>, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

int layered_rows_per_tile() { return kBN; }

}  // namespace mlpk

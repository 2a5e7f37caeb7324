// mlp_layered.hip -- networks beyond the fused kernels: layer-by-layer MFMA GEMMs with the fused
// epilogue.
//
// The fused kernels keep a whole network's weights in LDS and its activations in registers, which
// bounds them to widths <= 128 and 8 layers.  Wider or deeper networks run here, one kernel per layer:
//   Y[r][o] = act(RNE16(b[o] + sum_k W[o][k] * X[r][k]))   (FP16 x FP16 products, FP32 accumulation;
//   act = the leaky ReLU max(v, v * half(0.01)) in FP16 for every layer but the last)
// -- the same arithmetic as the fused path ("Profiling neural material inference", "Experiment
// setup" and "Bad versus good activation"), with the activations between layers in device memory
// (within a chain of 256-wide layers, in LDS).
//
// Three forms (v_mfma_f32_32x32x16_f16, weights = A operand, rows = B operand, as in the fused
// kernel): runs of consecutive layers with 256 padded outputs and K of 128..256 go through one
// launch that keeps the row tile's activations in LDS (layer_chain, described before it); other
// layers whose padded output width is a multiple of 256 and whose rows are whole 16-byte chunks run
// on a 256 x 256 workgroup tile with both operands staged through LDS (layer_gemm_big); every other
// layer on this 128 x 256 one:
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

    // Epilogue: lane (g, n) holds, for row 64 wave + 32 j + n, outputs 32 mt + 8 q + 4 g + i.  Without
    // the activation the slope is 1: max(v, v * 1) is v bit for bit, and no select per register.
    const h4 s4 = p.act ? (h4)slope() : (h4)(_Float16)1.0f;
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

// ---- the large tile: 256 outputs x 256 rows per workgroup -------------------------------------
//
// For layers whose padded output width is a multiple of 256 and whose rows are whole 16-byte chunks
// (win equal to the padded K, rows 16-byte aligned).  Four waves in a 2 x 2 grid, each computing 128
// outputs x 128 rows (4 x 4 MFMA tiles, 256 accumulator registers: one wave per SIMD, the
// accumulators in AGPRs).  Both operands go through LDS, K advancing 32 per stage, two stages of LDS:
//   - weights: the stage's 16 fragments of the image ([8 output tiles][2 K blocks], 1 KB each, in
//     fragment order), read back with one 16-byte LDS read per lane;
//   - rows: 256 rows x 64 bytes; chunk c (16 bytes, K = 8 c .. 8 c + 7) of row r sits at
//     r * 64 + 16 (c ^ ((r / 4) % 4)), so the 16 lanes of a fragment read that share a K chunk hit 16
//     different bank groups (rows 4 apart land 16 bytes apart);
//   - every thread loads 8 chunks of 16 bytes per stage (4 of weights, 4 of rows, coalesced) two
//     stages ahead into registers and stores them into LDS at the end of the stage before; a weight
//     tile is read from LDS by the two waves that share its outputs, a row tile by the two that share
//     its rows.
// Per stage a wave reads 16 fragments from LDS (8 KB) and issues 32 MFMAs (1,024 MFMA cycles).
namespace bigtile {

constexpr int BM = 256, BN = 256, BK = 32, THREADS = 256;
constexpr int MTW = 4, NTW = 4;       // 32 x 32 tiles per wave
constexpr int A_STAGE = BM * BK * 2;  // 16 fragments of 1 KB
constexpr int B_STAGE = BN * BK * 2;  // 256 rows x 64 bytes
constexpr int STAGE = A_STAGE + B_STAGE;

// TWO: K has exactly two stages (kin = 64); otherwise at least four, so the K loop below runs at least
// once (a loop that may run zero times made the compiler park the accumulators in scratch around it).
// FULL: every padded output column is stored (wout = kout) and the output rows are 16-byte aligned.
// PP: the stage split around its barrier (below), for K of at least 32 stages.
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format: range-checked byte offsets
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

template <bool TWO, bool FULL, bool PP>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void layer_gemm_big(LayerArgs p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE];

    // Workgroup -> (row tile, output tile), output tiles fastest; XCD x = b % 8 takes a contiguous run.
    const int n_out = p.kout / BM;
    const int64_t n_tiles = p.row_tiles * n_out;
    const int64_t per_xcd = (n_tiles + 7) / 8;
    const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= n_tiles)
        return;  // whole workgroup, before any barrier
    const int64_t rt = t / n_out;
    const int ot = (int)(t % n_out);
    const int64_t row0 = rt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, n = lane & 31;
    const int KB = p.kin / 16;
    const int steps = p.kin / BK;  // even: kin is a multiple of 64

    // This thread's loads: weight fragment f = wave + 4 i of the stage (output tile f / 2, K block
    // f % 2), and row group q = wave + 4 i (rows 16 q .. 16 q + 15, this lane's row 16 q + lane / 4 and
    // its chunk slot lane % 4, holding chunk (lane % 4) ^ ((row / 4) % 4)).
    const uint8_t *a_src = p.a + ((size_t)ot * (BM / 32) * KB) * 1024 + lane * 16;
    const _Float16 *x_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = 16 * (wave + 4 * i) + (lane >> 2);
        const int64_t row = row0 + rl < p.rows ? row0 + rl : p.rows - 1;  // past the batch: a valid row, never stored
        x_src[i] = (const _Float16 *)p.x + row * p.ldx + 8 * ((lane & 3) ^ ((rl >> 2) & 3));
    }
    // Fragment reads: weights at (f * 64 + lane) * 16; rows at row * 64 + 16 ((2 kb + g) ^ ((n / 4) % 4)).
    const int a_rd = lane * 16 + wm * MTW * 2 * 1024;
    const int b_rd0 = A_STAGE + (wn * NTW * 32 + n) * 64 + 16 * ((0 + g) ^ ((n >> 2) & 3));
    const int b_rd1 = A_STAGE + (wn * NTW * 32 + n) * 64 + 16 * ((2 + g) ^ ((n >> 2) & 3));

    // Staging registers of the even (E) and the odd (O) stages, named one by one: arrays indexed in
    // unrolled loops were placed in LDS by the compiler (it promotes private arrays to LDS when the
    // workgroup leaves room), which turned every load into a load, a wait and an LDS store.
    uint4 Ea0, Ea1, Ea2, Ea3, Eb0, Eb1, Eb2, Eb3, Oa0, Oa1, Oa2, Oa3, Ob0, Ob1, Ob2, Ob3;
    const _Float16 *x0 = x_src[0], *x1 = x_src[1], *x2 = x_src[2], *x3 = x_src[3];
#define BIG_LDA(R, i, stage)                                                                                   \
    R = *(const uint4 *)(a_src + ((size_t)((wave + 4 * (i)) >> 1) * KB + 2 * (stage) + ((wave + 4 * (i)) & 1)) * 1024)
#define BIG_LOAD(P, stage)                                                                                     \
    do {                                                                                                       \
        BIG_LDA(P##a0, 0, stage);                                                                              \
        BIG_LDA(P##a1, 1, stage);                                                                              \
        BIG_LDA(P##a2, 2, stage);                                                                              \
        BIG_LDA(P##a3, 3, stage);                                                                              \
        P##b0 = *(const uint4 *)(x0 + (stage) * BK);                                                           \
        P##b1 = *(const uint4 *)(x1 + (stage) * BK);                                                           \
        P##b2 = *(const uint4 *)(x2 + (stage) * BK);                                                           \
        P##b3 = *(const uint4 *)(x3 + (stage) * BK);                                                           \
    } while (0)
#define BIG_STORE(P, buf)                                                                                      \
    do {                                                                                                       \
        uint8_t *d = lds[buf] + wave * 1024 + lane * 16;                                                       \
        *(uint4 *)(d + 0 * 4096) = P##a0;                                                                      \
        *(uint4 *)(d + 1 * 4096) = P##a1;                                                                      \
        *(uint4 *)(d + 2 * 4096) = P##a2;                                                                      \
        *(uint4 *)(d + 3 * 4096) = P##a3;                                                                      \
        *(uint4 *)(d + A_STAGE + 0 * 4096) = P##b0;                                                            \
        *(uint4 *)(d + A_STAGE + 1 * 4096) = P##b1;                                                            \
        *(uint4 *)(d + A_STAGE + 2 * 4096) = P##b2;                                                            \
        *(uint4 *)(d + A_STAGE + 3 * 4096) = P##b3;                                                            \
    } while (0)

    // Accumulators start at the bias tiles (the C operand of the first MFMA).
    f16x acc[MTW][NTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int mtg = ot * (BM / 32) + wm * MTW + mt;
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
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
            acc[mt][nt] = b;
    }

    // The fragments of one K block (4 of weights, 4 of rows).  BIG_FRAGS reads them together and
    // waits for them (the empty asm: left alone the compiler reads one weight fragment at a time and
    // each waits out the LDS latency); BIG_READ only requests them.
#define BIG_READ(A0, A1, A2, A3, B0, B1, B2, B3, buf, kb)                                                     \
    do {                                                                                                       \
        const uint8_t *la = lds[buf] + a_rd + (kb) * 1024;                                                     \
        const uint8_t *lb = lds[buf] + ((kb) ? b_rd1 : b_rd0);                                                 \
        A0 = *(const h8 *)(la + 0 * 2048);                                                                     \
        A1 = *(const h8 *)(la + 1 * 2048);                                                                     \
        A2 = *(const h8 *)(la + 2 * 2048);                                                                     \
        A3 = *(const h8 *)(la + 3 * 2048);                                                                     \
        B0 = *(const h8 *)(lb + 0 * 2048);                                                                     \
        B1 = *(const h8 *)(lb + 1 * 2048);                                                                     \
        B2 = *(const h8 *)(lb + 2 * 2048);                                                                     \
        B3 = *(const h8 *)(lb + 3 * 2048);                                                                     \
    } while (0)
#define BIG_FRAGS(A0, A1, A2, A3, B0, B1, B2, B3, buf, kb)                                                     \
    do {                                                                                                       \
        BIG_READ(A0, A1, A2, A3, B0, B1, B2, B3, buf, kb);                                                     \
        asm volatile("" ::"v"(A0), "v"(A1), "v"(A2), "v"(A3), "v"(B0), "v"(B1), "v"(B2), "v"(B3));             \
    } while (0)
// Scheduling groups for half a stage: eight times one MFMA, then one LDS read.
#define PP_MIX_READS8()                                                                                        \
    do {                                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                                     \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                 \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                 \
        }                                                                                                      \
    } while (0)
#define BIG_ROW(mt, A, B0, B1, B2, B3)                                                                         \
    do {                                                                                                       \
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B0, acc[mt][0], 0, 0, 0);                       \
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B1, acc[mt][1], 0, 0, 0);                       \
        acc[mt][2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B2, acc[mt][2], 0, 0, 0);                       \
        acc[mt][3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B3, acc[mt][3], 0, 0, 0);                       \
    } while (0)
#define BIG_MFMAS16(A0, A1, A2, A3, B0, B1, B2, B3)                                                             \
    do {                                                                                                       \
        BIG_ROW(0, A0, B0, B1, B2, B3);                                                                        \
        BIG_ROW(1, A1, B0, B1, B2, B3);                                                                        \
        BIG_ROW(2, A2, B0, B1, B2, B3);                                                                        \
        BIG_ROW(3, A3, B0, B1, B2, B3);                                                                        \
    } while (0)
    h8 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3;  // K block 0 of a stage
    h8 qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3;  // K block 1
    // Stage s (staging set P = s % 2, LDS buffer s % 2): request stage s + 2 into P (LOAD), multiply
    // stage s (its block 0 fragments were read at the end of the stage before), store stage s + 1
    // (staging set Q, requested a stage ago) into the other buffer (STORE), barrier, read the next
    // stage's block 0.  The loop body has no branch (the last two stages are peeled): branches inside it
    // made the compiler move accumulators between AGPRs and VGPRs around them.
#define BIG_STEP(P, Q, buf, LOAD, STORE)                                                                       \
    do {                                                                                                       \
        if (LOAD)                                                                                              \
            BIG_LOAD(P, s + 2);                                                                                \
        BIG_FRAGS(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3, buf, 1);                                             \
        BIG_MFMAS16(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3);                                                   \
        BIG_MFMAS16(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3);                                                   \
        if (STORE) {                                                                                           \
            BIG_STORE(Q, (buf) ^ 1);                                                                           \
            __syncthreads();                                                                                   \
            BIG_FRAGS(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, (buf) ^ 1, 0);                                   \
        }                                                                                                      \
    } while (0)
    // The same stage split around its barrier, for deep K (PP): the block 1 fragments of stage s are
    // read and stage s + 1 is stored into the other buffer while the 16 MFMAs of block 0 run (one
    // MFMA, then one LDS read; then one MFMA, one LDS store and one global load, stage s + 2's); after
    // the barrier, the block 0 fragments of stage s + 1 are read while block 1's 16 MFMAs run.  The
    // MFMA pipe then never waits for a whole block of reads, and the wave issues its memory work
    // between MFMAs; scheduling groups fix that interleave.  -11 % on 1024-wide and -10 % on 2048-wide
    // layers, none on 512-wide (16 stages), +7 % on 256-wide (8 stages).
#define PP_STEP(P, Q, buf, LOAD, STORE)                                                                       \
    do {                                                                                                       \
        if (LOAD)                                                                                              \
            BIG_LOAD(P, s + 2);                                                                                \
        BIG_READ(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3, buf, 1);                                              \
        if (STORE)                                                                                             \
            BIG_STORE(Q, (buf) ^ 1);                                                                           \
        BIG_MFMAS16(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3);                                                   \
        PP_MIX_READS8();                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                                     \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                 \
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                                                 \
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                                 \
        }                                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
        if (STORE) {                                                                                           \
            __syncthreads();                                                                                   \
            BIG_READ(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, (buf) ^ 1, 0);                                    \
        }                                                                                                      \
        BIG_MFMAS16(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3);                                                   \
        PP_MIX_READS8();                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                                                       \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
    } while (0)

    BIG_LOAD(E, 0);
    BIG_LOAD(O, 1);
    BIG_STORE(E, 0);
    __syncthreads();
    int s = 0;
    if constexpr (PP) {
        BIG_READ(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, 0, 0);
        do {
            PP_STEP(E, O, 0, true, true);
            ++s;
            PP_STEP(O, E, 1, true, true);
            ++s;
        } while (s + 2 < steps);
        PP_STEP(E, O, 0, false, true);
        PP_STEP(O, E, 1, false, false);
    } else {
        BIG_FRAGS(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, 0, 0);
        if constexpr (!TWO) {
            do {  // stages s and s + 1, both followed by two more
                BIG_STEP(E, O, 0, true, true);
                ++s;
                BIG_STEP(O, E, 1, true, true);
                ++s;
            } while (s + 2 < steps);
        }
        BIG_STEP(E, O, 0, false, true);  // stage steps - 2
        BIG_STEP(O, E, 1, false, false);  // stage steps - 1
    }

    // Epilogue through LDS (free once every wave has finished its last stage): each wave writes its
    // 128 outputs x 128 rows as FP16 after the rounding and the activation, 64 rows at a time, into a
    // 16 KB region of its own (row r, outputs 8 k .. 8 k + 3 in 8-byte chunk c = 2 k' at
    // r * 256 + 8 (c ^ (r % 32)): the 32 rows a write touches fall in 32 different bank pairs), then
    // reads it back row by row and stores 16 bytes per lane, whole 256-byte row segments.  The writes
    // have no condition (lane (g, n) of tile (mt, nt) holds outputs 32 mt + 8 q + 4 g + i of row
    // 32 nt + n); only the stores check the batch and the output width, on a few registers, so the
    // 256 accumulators stream out of the AGPRs instead of being spilled around branches.
    __syncthreads();
    const h4 s4 = p.act ? (h4)slope() : (h4)(_Float16)1.0f;  // slope 1: max(v, v * 1) is v
    uint8_t *ob = &lds[0][0] + wave * 16384;
    const bool vec16 = p.ldy % 8 == 0 && ((uintptr_t)p.y & 15) == 0;
    const int ldy2 = (int)p.ldy * 2;  // FULL only: at most 256 rows x 8 KB past the resource's base
    const int64_t left = p.rows - row0;
    const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
        (_Float16 *)p.y + row0 * p.ldy, 0, (int)((left < BN ? left : BN) * p.ldy * 2), RSRC_WORD3);
#define BIG_OUT_TILE(mt, nt, u)                                                                                \
    do {                                                                                                       \
        const int rl = 32 * (u) + n;                                                                           \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                                        \
            const f4 part = {acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]}; \
            h4 v = __builtin_convertvector(part, h4); /* nearest even */                                       \
            v = __builtin_elementwise_max(v, v * s4);                                                          \
            const int c = 8 * (mt) + 2 * q + g;                                                                \
            *(h4 *)(ob + rl * 256 + 8 * (c ^ (rl & 31))) = v;                                                  \
        }                                                                                                      \
    } while (0)
// Every padded output is stored (FULL): the 16 row quads of a half go out as buffer stores against a
// resource spanning this tile's rows within the batch, so rows past the batch fall outside it and
// write nothing, with no branch: the LDS reads then issue back to back instead of one read, one wait
// and one store at a time under a branch per row quad.
#define BIG_OUT_STORES(h)                                                                                      \
    do {                                                                                                       \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                                       \
            const int rl = 4 * i + (lane >> 4);                                                                \
            const uint2 lo = *(const uint2 *)(ob + rl * 256 + 8 * ((2 * k) ^ (rl & 31)));                      \
            const uint2 hi = *(const uint2 *)(ob + rl * 256 + 8 * ((2 * k + 1) ^ (rl & 31)));                  \
            __builtin_amdgcn_raw_buffer_store_b128(u4{lo.x, lo.y, hi.x, hi.y}, out_rs,                         \
                                                   (wn * NTW * 32 + 64 * (h) + rl) * ldy2 + 2 * col, 0, 0);    \
        }                                                                                                      \
    } while (0)
#define BIG_OUT_HALF(h)                                                                                        \
    do {                                                                                                       \
        _Pragma("unroll") for (int mt = 0; mt < MTW; ++mt) {                                                   \
            BIG_OUT_TILE(mt, 2 * (h), 0);                                                                      \
            BIG_OUT_TILE(mt, 2 * (h) + 1, 1);                                                                  \
        }                                                                                                      \
        const int k = lane & 15;                                                                               \
        const int col = ot * BM + wm * MTW * 32 + 8 * k;                                                       \
        if constexpr (FULL) {                                                                                  \
            BIG_OUT_STORES(h);                                                                                 \
        } else                                                                                                 \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                                       \
            const int rl = 4 * i + (lane >> 4);                                                                \
            const int64_t row = row0 + wn * NTW * 32 + 64 * (h) + rl;                                          \
            const uint2 lo = *(const uint2 *)(ob + rl * 256 + 8 * ((2 * k) ^ (rl & 31)));                      \
            const uint2 hi = *(const uint2 *)(ob + rl * 256 + 8 * ((2 * k + 1) ^ (rl & 31)));                  \
            if (row < p.rows) {                                                                                \
                _Float16 *yr = (_Float16 *)p.y + row * p.ldy + col;                                            \
                if (vec16 && col + 8 <= p.wout) {                                                              \
                    *(uint4 *)yr = make_uint4(lo.x, lo.y, hi.x, hi.y);                                         \
                } else {                                                                                       \
                    const uint4 w = make_uint4(lo.x, lo.y, hi.x, hi.y);                                        \
                    const h8 v8 = __builtin_bit_cast(h8, w);                                                   \
                    _Pragma("unroll") for (int e = 0; e < 8; ++e) if (col + e < p.wout) yr[e] = v8[e];         \
                }                                                                                              \
            }                                                                                                  \
        }                                                                                                      \
    } while (0)
    BIG_OUT_HALF(0);
    BIG_OUT_HALF(1);
#undef BIG_LDA
#undef BIG_LOAD
#undef BIG_STORE
#undef BIG_FRAGS
#undef BIG_ROW
#undef BIG_READ
#undef PP_MIX_READS8
#undef PP_STEP
#undef BIG_MFMAS16
#undef BIG_STEP
#undef BIG_OUT_TILE
#undef BIG_OUT_HALF
#undef BIG_OUT_STORES
}

// ---- chains of layers: the row tile's activations stay in LDS ---------------------------------
//
// For consecutive layers whose padded output width is CW (256; 128 or 64 for narrow deep nets) and
// whose K is at most CW (64 for CW = 64), one workgroup of NW waves takes 256 rows through all the
// chain's layers; wave w computes CW / 2 outputs (half w % 2) x 512 / NW rows (group w / 2), as
// CW / 64 x 16 / NW MFMA tiles.  CW = 256 runs eight waves of 128 outputs x 64 rows (128 accumulators,
// two waves per SIMD in the one workgroup per CU that its 160 KB of LDS allow: 8-9 % faster than four
// waves of 256 accumulators, one per SIMD, whose barrier and epilogue waits no other wave covered);
// CW = 128 four waves of 64 x 128 (128 accumulators, two workgroups per CU); CW = 64 four of 32 x 128
// (64, up to four workgroups).  The activations live in an LDS tile of 256 rows x CW features (row
// r's 16-byte chunk k, features 8 k .. 8 k + 7, at r * 2 CW + 16 (k ^ sw(r)) with sw(r) = r % (CW / 8),
// or (r / 2) % 8 for CW = 64: the 16 rows that one 256-byte LDS cycle of a fragment read serves hit 16
// distinct slots of the 64 banks), which the first layer's input rows are copied into and the last
// layer's outputs are copied out of; only the weights stream in, through two stages of CW x 32 K per
// step, as in the tile above.  A layer's epilogue (nearest-even rounding, the leaky ReLU) writes its
// outputs back into the tile, where the padded outputs (zero weights and bias) are exact zeros for
// the next layer's padded K.  At CW = 64 the image's outputs 64..127 of each layer (padded to 128, all
// zero) are skipped.  Device-memory traffic per chain: its input and its output, instead of every
// layer's, which makes such nets bound by the MFMA pipe instead of HBM.
constexpr int chain_waves_per_simd(int cw, int nw) { return cw == 64 ? 4 : cw == 128 ? 2 : nw / 4; }

template <int CW, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(chain_waves_per_simd(CW, NW),
                                                                          chain_waves_per_simd(CW, NW))))
void layer_chain(ChainArgs c)
{
    constexpr int TH = 64 * NW;         // threads per workgroup
    constexpr int NTC = 16 / NW;        // 32-row tiles per wave
    constexpr int MTC = CW / 64;        // output tiles per wave
    constexpr int NA = CW * 4 / TH;     // 16-byte weight chunks per thread per stage
    static_assert((NW == 4 || NW == 8) && NA >= 1 && NA <= 4, "a stage is 1 to 4 chunks per thread");
    constexpr int ROWB = CW * 2;        // bytes per activation row
    constexpr int NCH = CW / 8;         // 16-byte chunks per activation row
    constexpr int SWZ = NCH - 1;
    constexpr int SWS = CW < 128 ? 1 : 0;  // sw(r) = (r >> SWS) & SWZ
    constexpr int KOUT = CW < 128 ? 128 : CW;  // the image's padded outputs per layer
    constexpr int A_ST = CW * BK * 2;   // weight stage bytes
    __shared__ __attribute__((aligned(16))) uint8_t act[BN * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t ast[2][A_ST];

    const int64_t rt = blockIdx.x;
    if (rt >= c.row_tiles)
        return;  // whole workgroup, before any barrier
    const int64_t row0 = rt * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 5, n = lane & 31;

    // The first layer's input: 16-byte chunks of the tile's rows (rows past the batch repeat the last
    // row; their outputs are never stored).
    {
        const int kc = c.kin[0] / 8;
        for (int i = tid; i < BN * kc; i += TH) {
            const int r = i / kc, k = i - r * kc;
            const int64_t row = row0 + r < c.rows ? row0 + r : c.rows - 1;
            const uint4 v = *(const uint4 *)(c.x + row * c.ldx + 8 * k);
            *(uint4 *)(act + r * ROWB + 16 * (k ^ ((r >> SWS) & SWZ))) = v;
        }
    }

    const h4 s4 = (h4)slope();
    // B fragment rows of this lane: tile nt's row wn * 32 NTC + 32 nt + n, whose chunk k sits at
    // row * ROWB + 16 (k ^ sw(n)) (sw of the row depends on n alone).
    const int b_row = (wn * NTC * 32 + n) * ROWB;
    const int b_swz = (n >> SWS) & SWZ;
    const int a_rd = lane * 16 + wm * MTC * 2 * 1024;
    uint4 Ea0, Ea1, Ea2, Ea3, Oa0, Oa1, Oa2, Oa3;
    h8 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3;
    h8 qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3;
    f16x acc[MTC][NTC];

    // Weight stages: a_src / KB describe the layer being computed; its first two stages are loaded
    // before it starts (for layer 0 here, for the others during the last two K steps of the layer
    // before, into the staging registers those steps no longer use).  Thread chunk i of a stage is
    // fragment f = wave + NW i (output tile f / 2, K block f % 2).
    const uint8_t *a_src = c.image + c.off[0] + lane * 16;
    int KB = c.kin[0] / 16;
#define CH_LDA(R, i, stage)                                                                                    \
    R = *(const uint4 *)(a_src + ((size_t)((wave + NW * (i)) >> 1) * KB + 2 * (stage) + ((wave + NW * (i)) & 1)) * 1024)
#define CH_LDN(R, i, stage)                                                                                    \
    R = *(const uint4 *)(a_nx + ((size_t)((wave + NW * (i)) >> 1) * KB_nx + 2 * (stage) + ((wave + NW * (i)) & 1)) * 1024)
#define CH_LOAD(P, stage)                                                                                      \
    do {                                                                                                       \
        CH_LDA(P##a0, 0, stage);                                                                               \
        if constexpr (NA > 1)                                                                                  \
            CH_LDA(P##a1, 1, stage);                                                                           \
        if constexpr (NA > 2) {                                                                                \
            CH_LDA(P##a2, 2, stage);                                                                           \
            CH_LDA(P##a3, 3, stage);                                                                           \
        }                                                                                                      \
    } while (0)
#define CH_LOADN(P, stage)                                                                                     \
    do {                                                                                                       \
        CH_LDN(P##a0, 0, stage);                                                                               \
        if constexpr (NA > 1)                                                                                  \
            CH_LDN(P##a1, 1, stage);                                                                           \
        if constexpr (NA > 2) {                                                                                \
            CH_LDN(P##a2, 2, stage);                                                                           \
            CH_LDN(P##a3, 3, stage);                                                                           \
        }                                                                                                      \
    } while (0)
#define CH_STORE(P, buf)                                                                                       \
    do {                                                                                                       \
        uint8_t *d = ast[buf] + wave * 1024 + lane * 16;                                                       \
        *(uint4 *)(d + 0 * NW * 1024) = P##a0;                                                                 \
        if constexpr (NA > 1)                                                                                  \
            *(uint4 *)(d + 1 * NW * 1024) = P##a1;                                                             \
        if constexpr (NA > 2) {                                                                                \
            *(uint4 *)(d + 2 * NW * 1024) = P##a2;                                                             \
            *(uint4 *)(d + 3 * NW * 1024) = P##a3;                                                             \
        }                                                                                                      \
    } while (0)
// K block kbg of the layer (16 features): weight fragments from stage buffer buf (its block kbg % 2),
// row fragments from the activation tile, requested together (the waits fall where they are used).
#define CH_READ(A0, A1, A2, A3, B0, B1, B2, B3, buf, kbg)                                                      \
    do {                                                                                                       \
        const uint8_t *la = ast[buf] + a_rd + ((kbg) & 1) * 1024;                                              \
        const uint8_t *lb = act + b_row + 16 * ((2 * (kbg) + g) ^ b_swz);                                      \
        A0 = *(const h8 *)(la + 0 * 2048);                                                                     \
        if constexpr (MTC > 1)                                                                                 \
            A1 = *(const h8 *)(la + 1 * 2048);                                                                 \
        if constexpr (MTC > 2) {                                                                               \
            A2 = *(const h8 *)(la + 2 * 2048);                                                                 \
            A3 = *(const h8 *)(la + 3 * 2048);                                                                 \
        }                                                                                                      \
        B0 = *(const h8 *)(lb + 0 * 32 * ROWB);                                                                \
        B1 = *(const h8 *)(lb + 1 * 32 * ROWB);                                                                \
        if constexpr (NTC > 2) {                                                                               \
            B2 = *(const h8 *)(lb + 2 * 32 * ROWB);                                                            \
            B3 = *(const h8 *)(lb + 3 * 32 * ROWB);                                                            \
        }                                                                                                      \
    } while (0)
#define CH_ROW(mt, A, B0, B1, B2, B3)                                                                          \
    do {                                                                                                       \
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B0, acc[mt][0], 0, 0, 0);                       \
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B1, acc[mt][1], 0, 0, 0);                       \
        if constexpr (NTC > 2) {                                                                               \
            acc[mt][2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B2, acc[mt][2], 0, 0, 0);                   \
            acc[mt][3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B3, acc[mt][3], 0, 0, 0);                   \
        }                                                                                                      \
    } while (0)
#define CH_MFMAS(A0, A1, A2, A3, B0, B1, B2, B3)                                                               \
    do {                                                                                                       \
        CH_ROW(0, A0, B0, B1, B2, B3);                                                                         \
        if constexpr (MTC > 1)                                                                                 \
            CH_ROW(1, A1, B0, B1, B2, B3);                                                                     \
        if constexpr (MTC > 2) {                                                                               \
            CH_ROW(2, A2, B0, B1, B2, B3);                                                                     \
            CH_ROW(3, A3, B0, B1, B2, B3);                                                                     \
        }                                                                                                      \
    } while (0)
    // per K block: MTC + NTC fragment reads and MTC x NTC MFMAs; per stage NA weight chunks per thread
    constexpr int RD = MTC + NTC, NM = MTC * NTC;
    CH_LOAD(E, 0);
    CH_LOAD(O, 1);

    for (int l = 0; l < c.n; ++l) {
        const uint8_t *A = c.image + c.off[l];
        const int steps = KB / 2;  // 2 (CW = 128 or 64), 4, 6 or 8
        // the next layer's weights (the last layer reloads its own, unused: no branch)
        const int ln = l + 1 < c.n ? l + 1 : l;
        const uint8_t *a_nx = c.image + c.off[ln] + lane * 16;
        const int KB_nx = c.kin[ln] / 16;
        const f4 *bias = (const f4 *)(A + (size_t)(KOUT / 32) * KB * 1024);  // after the fragments
#pragma unroll
        for (int mt = 0; mt < MTC; ++mt) {
            const f4 *bt = bias + (wm * MTC + mt) * 8 + g * 4;
            const f4 b0 = bt[0], b1 = bt[1], b2 = bt[2], b3 = bt[3];
            f16x b;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = b0[j];
                b[4 + j] = b1[j];
                b[8 + j] = b2[j];
                b[12 + j] = b3[j];
            }
#pragma unroll
            for (int nt = 0; nt < NTC; ++nt)
                acc[mt][nt] = b;
        }
        __syncthreads();  // the tile holds this layer's input; every wave is done with the stages
        CH_STORE(E, 0);
        __syncthreads();
// Stage s split around its barrier (as PP_STEP above): block 1's fragments are read and the next
// stage's weights stored while block 0's MFMAs run, the next stage's block 0 after the barrier while
// block 1's run; LOADN requests weights two stages ahead (in the last two steps, the next layer's
// first two stages).  -1.6 % on 16 layers of 256 against the unsplit order.
#define CH_SPLIT(P, Q, buf, LOADN, STORE)                                                                      \
    do {                                                                                                       \
        LOADN;                                                                                                 \
        CH_READ(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3, buf, 2 * s + 1);                                       \
        if (STORE)                                                                                             \
            CH_STORE(Q, (buf) ^ 1);                                                                            \
        CH_MFMAS(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3);                                                      \
        if constexpr (CW >= 128) {                                                                             \
            _Pragma("unroll") for (int i_ = 0; i_ < RD; ++i_) {                                                \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
            }                                                                                                  \
            _Pragma("unroll") for (int i_ = 0; i_ < NA; ++i_) {                                                \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                                             \
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                             \
            }                                                                                                  \
            _Pragma("unroll") for (int i_ = 0; i_ < NM - RD - NA; ++i_)                                        \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
        }                                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
        if (STORE) {                                                                                           \
            __syncthreads();                                                                                   \
            CH_READ(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, (buf) ^ 1, 2 * s + 2);                             \
        }                                                                                                      \
        CH_MFMAS(qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3);                                                      \
        if constexpr (CW >= 128) {                                                                             \
            _Pragma("unroll") for (int i_ = 0; i_ < RD; ++i_) {                                                \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                             \
            }                                                                                                  \
            _Pragma("unroll") for (int i_ = 0; i_ < NM - RD; ++i_)                                             \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                             \
        }                                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                                     \
    } while (0)
        CH_READ(pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, 0, 0);
        int s = 0;
        if (CW == 256 || (CW == 128 && steps > 2)) {  // K of 128..256 (the 256-wide chain always: no branch there)
            do {
                CH_SPLIT(E, O, 0, CH_LOAD(E, s + 2), true);
                ++s;
                CH_SPLIT(O, E, 1, CH_LOAD(O, s + 2), true);
                ++s;
            } while (s + 2 < steps);
        }
        CH_SPLIT(E, O, 0, CH_LOADN(E, 0), true);
        ++s;
        CH_SPLIT(O, E, 1, CH_LOADN(O, 1), false);
#undef CH_SPLIT
        __syncthreads();  // every wave has read its row fragments of this layer

        // Epilogue into the tile: lane (g, n) of tile (mt, nt) holds outputs 32 mt + 8 q + 4 g + i of
        // row 32 nt + n (within the wave's row group): features 8 k + 4 g .. + 3 of chunk
        // k = (NCH / 2) wm + 4 mt + q.
        // A layer without the activation (the chain's last, unless act_last) takes slope 1, for which
        // max(v, v * 1) is v bit for bit: one uniform select per layer instead of one per register.
        const h4 sl = l + 1 < c.n || c.act_last ? s4 : (h4)(_Float16)1.0f;
#pragma unroll
        for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTC; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f4 part = {acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2],
                                     acc[mt][nt][4 * q + 3]};
                    h4 v = __builtin_convertvector(part, h4);  // nearest even
                    v = __builtin_elementwise_max(v, v * sl);
                    const int k = (NCH / 2) * wm + 4 * mt + q;
                    *(h4 *)(act + b_row + nt * 32 * ROWB + 16 * (k ^ b_swz) + 8 * g) = v;
                }
        a_src = a_nx;
        KB = KB_nx;
    }
#undef CH_LDA
#undef CH_LDN
#undef CH_LOAD
#undef CH_LOADN
#undef CH_STORE
#undef CH_ROW
#undef CH_READ
#undef CH_MFMAS
    __syncthreads();

    // The last layer's outputs: its first c.wout_last features (a multiple of 8) of each row within
    // the batch, in 16-byte chunks; thread tid copies chunk tid % NCH of every (TH / NCH)-th row.
    const int k = tid % NCH;
    if (8 * k < c.wout_last)
        for (int r = tid / NCH; r < BN; r += TH / NCH)
            if (row0 + r < c.rows)
                *(uint4 *)(c.y + (row0 + r) * c.ldy + 8 * k) = *(const uint4 *)(act + r * ROWB + 16 * (k ^ ((r >> SWS) & SWZ)));
}

}  // namespace bigtile

}  // namespace

bool layer_big_tile(const LayerArgs &p) { return p.kout % bigtile::BM == 0 && p.vec_x && p.win == p.kin; }

hipError_t launch_layer(const LayerArgs &p, hipStream_t stream)
{
    if (layer_big_tile(p)) {
        const int64_t tiles = ((p.rows + bigtile::BN - 1) / bigtile::BN) * (p.kout / bigtile::BM);
        LayerArgs q = p;
        q.row_tiles = (p.rows + bigtile::BN - 1) / bigtile::BN;
        const int steps = p.kin / bigtile::BK;
        const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
        const bool full = p.wout == p.kout && p.ldy % 8 == 0 && ((uintptr_t)p.y & 15) == 0;
        const bool pp = steps >= 32;  // K >= 1024
        auto *k = steps == 2 ? (full ? bigtile::layer_gemm_big<true, true, false> : bigtile::layer_gemm_big<true, false, false>)
                  : pp ? (full ? bigtile::layer_gemm_big<false, true, true> : bigtile::layer_gemm_big<false, false, true>)
                       : (full ? bigtile::layer_gemm_big<false, true, false> : bigtile::layer_gemm_big<false, false, false>);
        hipLaunchKernelGGL(k, grid, dim3(bigtile::THREADS), 0, stream, q);
        return hipGetLastError();
    }
    const int64_t tiles = p.row_tiles * (p.kout / kBM);
    const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
    if (p.vec_x && p.win == p.kin)
        hipLaunchKernelGGL(layer_gemm<true>, grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(layer_gemm<false>, grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_chain(const ChainArgs &c, hipStream_t stream)
{
    if (c.width == 256)
        hipLaunchKernelGGL((bigtile::layer_chain<256, 8>), dim3((unsigned)c.row_tiles), dim3(512), 0, stream, c);
    else if (c.width == 128)
        hipLaunchKernelGGL((bigtile::layer_chain<128, 4>), dim3((unsigned)c.row_tiles), dim3(bigtile::THREADS), 0, stream, c);
    else if (c.width == 64)
        hipLaunchKernelGGL((bigtile::layer_chain<64, 4>), dim3((unsigned)c.row_tiles), dim3(bigtile::THREADS), 0, stream, c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int layered_rows_per_tile() { return kBN; }

}  // namespace mlpk

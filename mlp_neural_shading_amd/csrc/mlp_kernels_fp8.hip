// mlp_kernels_fp8.hip -- the FP8 variant of the fused kernel (gfx950 v_mfma_f32_32x32x64_f8f6f4).
//
// The same network as mlp_kernels.hip at lower precision: weights and each layer's input in OCP
// E4M3, products accumulated in FP32 with the bias as the C operand, then the same FP32 -> FP16
// rounding and FP16 leaky ReLU max(v, v * half(0.01)) ("Profiling neural material inference",
// "Bad versus good activation").  Scaling follows the block-scaled formats: every weight row carries
// a power-of-two scale (an E8M0 code in the image, applied by the MFMA's A-operand scale), and the
// activations are stored as E4M3(16 h) and scaled back by the B-operand scale 2^-4.
//
// Structure as in the FP16 kernel (persistent grid, the image staged once per workgroup into LDS,
// tiles of NT x 32 rows per wave, output tiles software-pipelined), with these differences:
//   - one MFMA covers 64 input features (32 bytes of A and of B per lane);
//   - the epilogue of output tile mt converts to FP16, applies the leaky ReLU and converts to E4M3
//     with v_cvt_scalef32_pk_fp8_f16 (scale 1/16, i.e. E4M3(16 v)); tiles 2 kb and 2 kb + 1 fill the
//     next layer's block kb in the same lanes (slot order in mlp_layout.h), no data movement;
//   - the caller's FP16 input rows are loaded one tile ahead and converted to E4M3 when used.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mlp_layout.h"
#include "mlp_registry.h"

namespace mlpk {
namespace f8 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s2 __attribute__((ext_vector_type(2)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kScaleB = 127 - 4;  // E8M0 code of 2^-4: the activations are stored as E4M3(16 h)

__device__ __forceinline__ _Float16 slope() { return __builtin_bit_cast(_Float16, (unsigned short)0x211f); }

// D = C + sum_k (A[k] * 2^(sa_row - 127)) * (B[k] * 2^-4); SEL picks lane's scale byte.
template <int SEL>
__device__ __forceinline__ f16x mfma8(i8 a, i8 b, f16x c, int sa)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, sa, 0, kScaleB);
}

// Four FP16 values -> four E4M3 codes of 16 v (bytes 0..3 in order).
__device__ __forceinline__ int to_e4m3x4(h4 v)
{
    const s2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16((s2)(short)0, __builtin_shufflevector(v, v, 0, 1), 1.0f / 16, false);
    const s2 both = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, __builtin_shufflevector(v, v, 2, 3), 1.0f / 16, true);
    return __builtin_bit_cast(int, both);
}

template <int... W>
struct Net {
    static constexpr int L = sizeof...(W) - 1;
    static constexpr int w[sizeof...(W)] = {W...};
    static constexpr int MT(int l) { return mlpl::m_tiles(w, l); }
    static constexpr int KB(int l) { return mlpl::f8_k_blocks(w, l); }
    static constexpr size_t bytes() { return mlpl::f8_bytes(w, L); }
};

template <class N, int NT>
struct Body {
    static constexpr int L = N::L;
    static constexpr int KB0 = N::KB(0);
    static_assert(N::w[0] % 8 == 0, "the FP8 kernels read the input rows 8 halves at a time");
    static constexpr bool kVecOut = N::w[L] % 4 == 0;
    static_assert(kVecOut, "the FP8 kernels store 4 outputs at a time");

    // ---- weights from LDS ----------------------------------------------------------------------

    template <int l>
    static __device__ __forceinline__ i8 a_frag(const uint8_t *lds, int mt, int kb, int lane)
    {
        const uint8_t *p = lds + mlpl::f8_a_off(N::w, l) + ((size_t)(mt * N::KB(l) + kb) * 64 + lane) * 32;
        const i4 lo = *(const i4 *)p, hi = *(const i4 *)(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    template <int l>
    static __device__ __forceinline__ f16x bias_tile(const uint8_t *lds, int mt, int lane)
    {
        const f4 *p = (const f4 *)(lds + mlpl::f8_b_off(N::w, l) + mt * mlpl::kBiasTileBytes + (lane >> 5) * 64);
        const f4 b0 = p[0], b1 = p[1], b2 = p[2], b3 = p[3];
        f16x b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = b0[j];
            b[4 + j] = b1[j];
            b[8 + j] = b2[j];
            b[12 + j] = b3[j];
        }
        return b;
    }

    template <int l>
    static __device__ __forceinline__ int scale_word(const uint8_t *lds, int mt, int lane)
    {
        return *(const int *)(lds + mlpl::f8_s_off(N::w, l) + ((mt / 4) * 64 + lane) * 4);
    }

    template <int l>
    static __device__ __forceinline__ void fetch(const uint8_t *lds, int mt, i8 (&af)[N::KB(l)], f16x &bias, int &sc,
                                                 int lane)
    {
        constexpr int KB = N::KB(l);  // a constant expression, so the loop fully unrolls
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            af[kb] = a_frag<l>(lds, mt, kb, lane);
        bias = bias_tile<l>(lds, mt, lane);
        sc = scale_word<l>(lds, mt, lane);
    }

    // ---- one layer ----------------------------------------------------------------------------

    template <int l, int MTI>
    static __device__ __forceinline__ void mfmas(const i8 (&af)[N::KB(l)], const i8 (&Bin)[N::KB(l)][NT],
                                                 const f16x &bias, int sc, f16x (&acc)[NT])
    {
        constexpr int KB = N::KB(l);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = mfma8<MTI % 4>(af[kb], Bin[kb][t], kb == 0 ? bias : acc[t], sc);
    }

    // FP32 -> FP16 (nearest even) -> leaky ReLU -> E4M3(16 v): tile MTI fills half MTI % 2 of block
    // MTI / 2 of the next layer's B operand.
    template <int KBN, int MTI>
    static __device__ __forceinline__ void epilogue(const f16x (&acc)[NT], i8 (&Bout)[KBN][NT])
    {
        const h4 s = (h4)slope();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 part = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
                const h4 v = __builtin_convertvector(part, h4);
                Bout[MTI / 2][t][4 * (MTI % 2) + q] = to_e4m3x4(__builtin_elementwise_max(v, v * s));
            }
    }

    template <int t>
    static __device__ __forceinline__ void store_tile(const f16x (&acc)[NT], int mt, const LaunchArgs &a,
                                                      int64_t row0, int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const int64_t row = row0 + 32 * t + n;
        if (row < a.batch) {
            constexpr int wl = N::w[L];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 32 * mt + 8 * q + 4 * g;
                const f4 part = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
                if (32 * mt + 8 * q < wl && c < wl)
                    *(h4 *)((_Float16 *)a.y + row * wl + c) = __builtin_convertvector(part, h4);
            }
        }
    }

    template <int... T>
    static __device__ __forceinline__ void store_outputs(const f16x (&acc)[NT], int mt, const LaunchArgs &a,
                                                         int64_t row0, int lane, std::integer_sequence<int, T...>)
    {
        (store_tile<T>(acc, mt, a, row0, lane), ...);
    }

    static constexpr int next_blocks(int l) { return l + 1 == L ? 1 : N::KB(l + 1); }

    template <int l, int mt>
    static __device__ __forceinline__ void tile_step(const uint8_t *lds, const i8 (&Bin)[N::KB(l)][NT],
                                                     i8 (&af)[N::KB(l)], f16x &bias, int &sc,
                                                     i8 (&Bout)[next_blocks(l)][NT], f16x (&prev)[NT],
                                                     const LaunchArgs &a, int64_t row0, int lane)
    {
        constexpr int MT = N::MT(l);
        i8 afn[N::KB(l)];
        f16x biasn;
        int scn;
        if constexpr (mt + 1 < MT)
            fetch<l>(lds, mt + 1, afn, biasn, scn, lane);
        f16x acc[NT];
        mfmas<l, mt>(af, Bin, bias, sc, acc);
        if constexpr (l + 1 == L) {
            store_outputs(acc, mt, a, row0, lane, std::make_integer_sequence<int, NT>());
        } else {
            if constexpr (mt > 0)
                epilogue<next_blocks(l), mt - 1>(prev, Bout);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                prev[t] = acc[t];
        }
        if constexpr (mt + 1 < MT) {
            constexpr int KB = N::KB(l);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                af[kb] = afn[kb];
            bias = biasn;
            sc = scn;
        }
    }

    template <int l, int... MTS>
    static __device__ __forceinline__ void layer_tiles(const uint8_t *lds, const i8 (&Bin)[N::KB(l)][NT],
                                                       i8 (&Bout)[next_blocks(l)][NT], const LaunchArgs &a,
                                                       int64_t row0, int lane, std::integer_sequence<int, MTS...>)
    {
        i8 af[N::KB(l)];
        f16x bias;
        int sc;
        fetch<l>(lds, 0, af, bias, sc, lane);
        f16x prev[NT];
        (tile_step<l, MTS>(lds, Bin, af, bias, sc, Bout, prev, a, row0, lane), ...);
        if constexpr (l + 1 < L)
            epilogue<next_blocks(l), N::MT(l) - 1>(prev, Bout);
    }

    template <int l>
    static __device__ __forceinline__ void layer(const uint8_t *lds, const i8 (&Bin)[N::KB(l)][NT], const LaunchArgs &a,
                                                 int64_t row0, int lane)
    {
        // Keep each layer inside its own stretch of the instruction stream: without these barriers
        // the scheduler requests the whole network's weights up front and defers the conversions,
        // and runs out of registers.  The barriers take every block of the layer's input as an
        // operand, so neither they nor the reads after them can move above the previous layer's
        // epilogues.
        constexpr int KBI = N::KB(l);
#pragma unroll
        for (int kb = 0; kb < KBI; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                asm volatile("" ::"v"(Bin[kb][t]) : "memory");
        constexpr int KBN = next_blocks(l);
        i8 Bout[KBN][NT];
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                Bout[kb][t] = (i8)0;  // an odd number of output tiles leaves half of the last block empty
        layer_tiles<l>(lds, Bin, Bout, a, row0, lane, std::make_integer_sequence<int, N::MT(l)>());
        if constexpr (l + 1 < L)
            layer<l + 1>(lds, Bout, a, row0, lane);
    }

    // ---- the caller's rows -> layer-0 B fragments -------------------------------------------------
    //
    // Lane (g, n) of block kb needs features 64 kb + 32 g + j, j = 0..31, of row 32 t + n: four
    // 16-byte loads, issued one tile ahead with clamped addresses and no select (so the wave does
    // not wait for them at issue), masked and converted when the tile is used.

    template <int t>
    static __device__ __forceinline__ void load_tile(h8 (&R)[KB0][NT][4], const LaunchArgs &a, int64_t row0, int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const int64_t row = row0 + 32 * t + n;
        const int64_t rr = row < a.batch ? row : a.batch - 1;
        constexpr int w0 = N::w[0];
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = 64 * kb + 32 * g + 8 * c;
                const int cc = col < w0 ? col : w0 - 8;
                R[kb][t][c] = *(const h8 *)((const _Float16 *)a.x + rr * w0 + cc);
            }
    }

    template <int... T>
    static __device__ __forceinline__ void load_inputs(h8 (&R)[KB0][NT][4], const LaunchArgs &a, int64_t row0, int lane,
                                                       std::integer_sequence<int, T...>)
    {
        (load_tile<T>(R, a, row0, lane), ...);
    }

    template <int t>
    static __device__ __forceinline__ void convert_tile(i8 (&B)[KB0][NT], const h8 (&R)[KB0][NT][4], const LaunchArgs &a,
                                                        int64_t row0, int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const bool live = row0 + 32 * t + n < a.batch;
        constexpr int w0 = N::w[0];
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = 64 * kb + 32 * g + 8 * c;
                const h8 v = (live && col < w0) ? R[kb][t][c] : (h8)(_Float16)0;
                B[kb][t][2 * c] = to_e4m3x4(__builtin_shufflevector(v, v, 0, 1, 2, 3));
                B[kb][t][2 * c + 1] = to_e4m3x4(__builtin_shufflevector(v, v, 4, 5, 6, 7));
            }
    }

    template <int... T>
    static __device__ __forceinline__ void convert_inputs(i8 (&B)[KB0][NT], const h8 (&R)[KB0][NT][4],
                                                          const LaunchArgs &a, int64_t row0, int lane,
                                                          std::integer_sequence<int, T...>)
    {
        (convert_tile<T>(B, R, a, row0, lane), ...);
    }
};

// Copy the image into LDS with every load in flight before the first store, in two steps so that
// the first tile's input loads can be issued in between: the stores then wait for the image (from
// L2), not for the inputs (from HBM, requested by every wave of the chip at once).  The empty asm
// reads every loaded chunk before the first store, so the compiler cannot move the load of a
// partly used chunk into the branch around its store (a second round trip).
template <int C>
struct Chunks {
    uint4 v[C];
};

__device__ __forceinline__ void loaded(const uint4 &v) { asm volatile("" ::"v"(v.x)); }
__device__ __forceinline__ void store16(uint8_t *dst, const uint4 &v) { *(uint4 *)dst = make_uint4(v.x, v.y, v.z, v.w); }

template <int BYTES, int THREADS, int... K>
__device__ __forceinline__ Chunks<sizeof...(K)> stage_load(const uint8_t *image, std::integer_sequence<int, K...>)
{
    const int t16 = (int)threadIdx.x * 16;
    return {{*(const uint4 *)(image + (K * THREADS * 16 + t16 < BYTES ? K * THREADS * 16 + t16 : BYTES - 16))...}};
}

template <int BYTES, int THREADS, int... K>
__device__ __forceinline__ void stage_store(uint8_t *lds, const Chunks<sizeof...(K)> &c, std::integer_sequence<int, K...>)
{
    const int t16 = (int)threadIdx.x * 16;
    (loaded(c.v[K]), ...);
    ((K * THREADS * 16 + t16 < BYTES ? store16(lds + K * THREADS * 16 + t16, c.v[K]) : (void)0), ...);
}

// Scheduling as in the FP16 kernel: workgroup b owns tiles [lo, hi) of an even split; its waves take
// the first WAVES and then claim tiles from an LDS counter two ahead.
template <class N, int NT, int WAVES, int EU>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(EU, EU))) mlp_fused_fp8(LaunchArgs a)
{
    using B = Body<N, NT>;
    constexpr int bytes = (int)N::bytes();
    static_assert(bytes % 16 == 0, "image must be a multiple of 16 bytes");
    constexpr int kRows = NT * 32;
    constexpr int KB0 = B::KB0;
    __shared__ int next_tile;
    __shared__ __attribute__((aligned(16))) uint8_t lds[bytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tiles = (a.batch + kRows - 1) / kRows;
    const int64_t lo = (int64_t)blockIdx.x * tiles / gridDim.x;
    const int64_t hi = ((int64_t)blockIdx.x + 1) * tiles / gridDim.x;
    int64_t tile = lo + wave;
    int64_t next = lo + WAVES + wave;

    h8 Rnext[KB0][NT][4];
    constexpr int kChunks = (bytes + WAVES * 64 * 16 - 1) / (WAVES * 64 * 16);
    const auto chunks = stage_load<bytes, WAVES * 64>(a.image, std::make_integer_sequence<int, kChunks>());
    B::load_inputs(Rnext, a, (tile < hi ? tile : lo) * kRows, lane, std::make_integer_sequence<int, NT>());
    stage_store<bytes, WAVES * 64>(lds, chunks, std::make_integer_sequence<int, kChunks>());
    if (threadIdx.x == 0)
        next_tile = 2 * WAVES;
    __syncthreads();

    int claimed = 0;
    if (lane == 0)
        claimed = atomicAdd(&next_tile, 1);
    while (tile < hi) {
        // keeps the loop-invariant fragment reads inside the loop (see the FP16 kernel)
        asm volatile("" ::: "memory");
        i8 B0[KB0][NT];
        B::convert_inputs(B0, Rnext, a, tile * kRows, lane, std::make_integer_sequence<int, NT>());
        const int64_t after = lo + __builtin_amdgcn_readfirstlane(claimed);
        if (lane == 0)
            claimed = atomicAdd(&next_tile, 1);
        B::template layer<0>(lds, B0, a, tile * kRows, lane);
        if (next < hi)
            B::load_inputs(Rnext, a, next * kRows, lane, std::make_integer_sequence<int, NT>());
        tile = next;
        next = after;
    }
}

template <class N, int NT, int WAVES, int EU>
hipError_t launch(const LaunchArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((mlp_fused_fp8<N, NT, WAVES, EU>), dim3(grid), dim3(WAVES * 64), 0, s, a);
    return hipGetLastError();
}

template <class N, int NT, int WAVES, int EU>
KernelEntry entry(const char *name)
{
    KernelEntry e{};
    e.name = name;
    e.n_layers = N::L;
    for (int i = 0; i <= N::L; ++i)
        e.widths[i] = N::w[i];
    e.generic = false;
    e.layout = kPackedFp8;
    e.act = kVector;
    e.threads = WAVES * 64;
    e.rows_per_wave = NT * 32;
    e.weights_in_lds = true;
    e.launch = &launch<N, NT, WAVES, EU>;
    e.func = (const void *)&mlp_fused_fp8<N, NT, WAVES, EU>;
    return e;
}

using NetSmall = Net<16, 32, 32, 32, 32, 32, 32, 32, 4>;
using NetPage = Net<32, 64, 64, 64, 64, 64, 64, 64, 4>;
using NetHetero = Net<32, 64, 64, 64, 128, 64, 64, 32, 4>;
using NetWide = Net<64, 128, 128, 128, 128, 128, 128, 128, 4>;
using NetStream = Net<64, 64, 64, 64, 64, 64, 64, 64, 16>;

static const KernelEntry kEntries[] = {
    // (net, 32-row tiles per wave, waves per workgroup, waves per SIMD)
    entry<NetSmall, 2, 8, 2>("mlp_fused_fp8<16-32x7-4>"),
    entry<NetPage, 2, 12, 3>("mlp_fused_fp8<32-64x7-4>"),
    entry<NetHetero, 2, 8, 2>("mlp_fused_fp8<32-64-64-64-128-64-64-32-4>"),
    entry<NetWide, 2, 8, 2>("mlp_fused_fp8<64-128x7-4>"),
    entry<NetStream, 2, 12, 3>("mlp_fused_fp8<64-64x7-16>"),
};

}  // namespace f8

const KernelEntry *registry_fp8(int *count)
{
    *count = (int)(sizeof(f8::kEntries) / sizeof(f8::kEntries[0]));
    return f8::kEntries;
}

}  // namespace mlpk

// mlp_kernels.hip -- the fused eight-layer FP16 MLP inference kernel for gfx950 (CDNA4).
//
// One launch evaluates the whole network for every input row ("Profiling neural material inference",
// section "Experiment setup": the timed unit is the complete inference pass).  Design:
//   - persistent grid; each wave loops over tiles of NT x 16 rows;
//   - the weight image is staged once per workgroup into LDS (or, when it does not fit in LDS, read
//     through the caches), and every A fragment is one 16-byte read per lane reused across the
//     wave's NT sample tiles;
//   - each layer is v_mfma_f32_16x16x32_f16 with the bias as the C operand of the first K block
//     (FP16 x FP16 products, FP32 accumulation);
//   - the epilogue of layers 1..L-1 converts FP32 -> FP16 with round-to-nearest-even and applies the
//     leaky ReLU max(v, v * half(0.01)) as packed FP16 operations on whole registers, the vector form
//     of "Bad versus good activation"; by the slot order in mlp_layout.h the result already sits
//     where the next layer's B operand needs it, so activations never leave the registers;
//   - the last layer converts to FP16 (no activation) and stores the row's outputs.
// Variants for the page's two A/B comparisons: the row-major weight image (fragments assembled from
// the canonical [out][in] matrices with per-lane index arithmetic), and the scalarised activation
// (one component at a time, compare and branch, "if (v < 0) v *= half(0.01)").
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mlp_layout.h"
#include "mlp_registry.h"

namespace mlpk {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// half(0.01): 0.01 rounded to binary16 (0x211f = 0.01000213623046875).
__device__ __forceinline__ _Float16 slope() { return __builtin_bit_cast(_Float16, (unsigned short)0x211f); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Vector leaky ReLU on four FP16 values: two packed instructions for every two values.
__device__ __forceinline__ h4 leaky_vector(h4 v)
{
    const h4 s = (h4)slope();
    return __builtin_elementwise_max(v, v * s);
}

// Scalarised leaky ReLU: each component on its own, with a compare and a conditional multiply.
__device__ __forceinline__ h4 leaky_scalarised(h4 v)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        _Float16 e = v[c];
        // The empty asm pins each element as a separate scalar value so that the compiler cannot
        // re-vectorise the loop into the packed form.
        asm volatile("" : "+v"(e));
        if (e < (_Float16)0)
            e = e * slope();
        v[c] = e;
    }
    return v;
}

// Where the weight image is read from.  Offsets are split into a per-lane part (voff, a VGPR) and
// a wave-uniform constant part (soff) so that neither path needs a register per fragment address.
struct LdsSource {  // image staged in LDS: ds_read with the constant as an immediate offset
    const uint8_t *base;
    __device__ __forceinline__ h8 load16(int voff, int soff) const { return *(const h8 *)(base + voff + soff); }
    __device__ __forceinline__ h4 load8(int voff, int soff) const { return *(const h4 *)(base + voff + soff); }
};

struct BufferSource {  // image read through the caches with buffer loads (constant offset in an SGPR)
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ h8 load16(int voff, int soff) const
    {
        return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
    }
    __device__ __forceinline__ h4 load8(int voff, int soff) const
    {
        return __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 0));
    }
};

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Wave priority from progress: 3 for a wave on its first tile, then 2, 1, 0.
__device__ __forceinline__ void set_priority(int it)
{
    switch (it) {
    case 0: __builtin_amdgcn_s_setprio(3); break;
    case 1: __builtin_amdgcn_s_setprio(2); break;
    case 2: __builtin_amdgcn_s_setprio(1); break;
    case 3: __builtin_amdgcn_s_setprio(0); break;
    default: break;
    }
}

// Compile-time description of the network a kernel instance computes.
template <int... W>
struct Net {
    static constexpr int L = sizeof...(W) - 1;
    static constexpr int w[sizeof...(W)] = {W...};
    static constexpr int MT(int l) { return mlpl::m_tiles(w, l); }
    static constexpr int KB(int l) { return mlpl::k_blocks(w, l); }
    static constexpr size_t image_bytes(int layout) { return layout == kPacked ? mlpl::pk_bytes(w, L) : mlpl::rm_bytes(w, L); }
};

template <class N, int NT, int LAYOUT, int ACT, bool GENERIC, bool LDS_W, class Src>
struct Body {
    static constexpr int L = N::L;
    // Caller widths known at compile time (exact instances) allow vector loads and stores.
    static constexpr bool kVecIn = !GENERIC && N::w[0] % 8 == 0;
    static constexpr bool kVecOut = !GENERIC && N::w[L] % 4 == 0;

    // ---- weight delivery ------------------------------------------------------------------

    template <int l>
    static __device__ __forceinline__ h8 a_frag(const Src &src, int mt, int kb, int lane)
    {
        constexpr int KB = N::KB(l);
        if constexpr (LAYOUT == kPacked) {
            return src.load16(lane * 16, (int)mlpl::pk_a_off(N::w, l) + (mt * KB + kb) * mlpl::kFragBytes);
        } else {
            // Row-major [out][in]: lane (g, m) gathers row 16 mt + m at its slot features.
            constexpr int win = N::w[l], wout = N::w[l + 1];
            static_assert(l > 0 || win % 8 == 0, "row-major input layer needs w0 % 8 == 0");
            static_assert(l == 0 || win % 4 == 0, "row-major hidden layer needs w % 4 == 0");
            const int g = lane >> 4, m = lane & 15;
            const int r = 16 * mt + m;
            const int row = (int)mlpl::rm_w_off(N::w, l) + 16 * mt * win * 2;  // wave-uniform
            h8 a = (h8)(_Float16)0;
            if constexpr (l == 0) {
                const int f = 32 * kb + 8 * g;
                if (r < wout && f < win)
                    a = src.load16((m * win + 8 * g) * 2, row + 32 * kb * 2);
            } else {
                const int f0 = 32 * kb + 4 * g, f1 = f0 + 16;
                h4 lo = (h4)(_Float16)0, hi = (h4)(_Float16)0;
                if (r < wout && f0 < win)
                    lo = src.load8((m * win + 4 * g) * 2, row + 32 * kb * 2);
                if (r < wout && f1 < win)
                    hi = src.load8((m * win + 4 * g) * 2, row + (32 * kb + 16) * 2);
                a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return a;
        }
    }

    template <int l>
    static __device__ __forceinline__ f4 bias_tile(const Src &src, int mt, int lane)
    {
        const int g = lane >> 4;
        if constexpr (LAYOUT == kPacked) {
            return __builtin_bit_cast(f4, src.load16(g * 16, (int)mlpl::pk_b_off(N::w, l) + mt * mlpl::kBiasTileBytes));
        } else {
            constexpr int wout = N::w[l + 1];
            static_assert(wout % 4 == 0, "row-major layer needs w_out % 4 == 0");
            h4 b = (h4)(_Float16)0;
            if (16 * mt + 4 * g < wout)
                b = src.load8(g * 8, (int)mlpl::rm_b_off(N::w, l) + 16 * mt * 2);
            return __builtin_convertvector(b, f4);
        }
    }

    // ---- one layer: NT sample tiles x MT output tiles x KB input blocks --------------------

    template <int l>
    static __device__ __forceinline__ void layer(const Src &wb, const h8 (&Bin)[N::KB(l)][NT],
                                                 const LaunchArgs &a, int64_t row0, int lane)
    {
        constexpr int MT = N::MT(l), KB = N::KB(l);
        // Weights read through the caches: keep each layer's reads inside the layer, or the
        // scheduler front-loads the whole network's fragments and runs out of registers.
        if constexpr (!LDS_W)
            asm volatile("" ::: "memory");
        if constexpr (l + 1 < L) {
            h8 Bout[N::KB(l + 1)][NT];
            h4 pend[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 af[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    af[kb] = a_frag<l>(wb, mt, kb, lane);
                const f4 bias = bias_tile<l>(wb, mt, lane);
                f4 acc[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = mfma(af[0], Bin[0][t], bias);
#pragma unroll
                for (int kb = 1; kb < KB; ++kb)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = mfma(af[kb], Bin[kb][t], acc[t]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    h4 v = __builtin_convertvector(acc[t], h4);  // v_cvt_pk_f16_f32: round to nearest even
                    v = (ACT == kVector) ? leaky_vector(v) : leaky_scalarised(v);
                    if (mt % 2 == 0) {
                        pend[t] = v;
                        if (mt == MT - 1)
                            Bout[mt / 2][t] = __builtin_shufflevector(v, (h4)(_Float16)0, 0, 1, 2, 3, 4, 5, 6, 7);
                    } else {
                        Bout[mt / 2][t] = __builtin_shufflevector(pend[t], v, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                }
            }
            layer<l + 1>(wb, Bout, a, row0, lane);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 af[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    af[kb] = a_frag<l>(wb, mt, kb, lane);
                const f4 bias = bias_tile<l>(wb, mt, lane);
                f4 acc[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = mfma(af[0], Bin[0][t], bias);
#pragma unroll
                for (int kb = 1; kb < KB; ++kb)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = mfma(af[kb], Bin[kb][t], acc[t]);
                store_outputs(acc, mt, a, row0, lane, std::make_integer_sequence<int, NT>());
            }
        }
    }

    // ---- input rows -> layer-0 B fragments --------------------------------------------------
    //
    // Written as one straight-line body per sample tile (an index-sequence expansion, not a loop):
    // a loop over tiles with the "row < batch" test gets peeled by the compiler into a run-time loop
    // with dynamically indexed fragment registers.  Loads are branch-free: the address is clamped to
    // a valid row and the value replaced by zero for rows past the batch.

    template <int t>
    static __device__ __forceinline__ void load_tile(h8 (&B)[N::KB(0)][NT], const LaunchArgs &a, int64_t row0,
                                                     int lane)
    {
        const int g = lane >> 4, n = lane & 15;
        const int64_t row = row0 + 16 * t + n;
        const bool live = row < a.batch;
        const int64_t rr = live ? row : a.batch - 1;
        constexpr int KB0 = N::KB(0);  // a constant expression, so the loop below fully unrolls
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb) {
            const int c = 32 * kb + 8 * g;
            h8 v = (h8)(_Float16)0;  // padded slots are zero in registers, never loaded
            if constexpr (kVecIn) {
                constexpr int w0 = N::w[0];
                if (32 * kb + 32 <= w0) {  // whole block inside the row (folds after unrolling)
                    v = *(const h8 *)((const _Float16 *)a.x + rr * w0 + c);
                    v = live ? v : (h8)(_Float16)0;
                } else {
                    const int cc = c < w0 ? c : w0 - 8;
                    v = *(const h8 *)((const _Float16 *)a.x + rr * w0 + cc);
                    v = (live && c < w0) ? v : (h8)(_Float16)0;
                }
            } else {
                const _Float16 *xr = (const _Float16 *)a.x + rr * a.w0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int cj = c + j;
                    const _Float16 e = xr[cj < a.w0 ? cj : a.w0 - 1];
                    v[j] = (live && cj < a.w0) ? e : (_Float16)0;
                }
            }
            B[kb][t] = v;
        }
    }

    template <int... T>
    static __device__ __forceinline__ void load_inputs(h8 (&B)[N::KB(0)][NT], const LaunchArgs &a, int64_t row0,
                                                       int lane, std::integer_sequence<int, T...>)
    {
        (load_tile<T>(B, a, row0, lane), ...);
    }

    // ---- last layer: FP32 -> FP16 and store -------------------------------------------------

    template <int t>
    static __device__ __forceinline__ void store_tile(const f4 (&acc)[NT], int mt, const LaunchArgs &a,
                                                      int64_t row0, int lane)
    {
        const int g = lane >> 4, n = lane & 15;
        const int c = 16 * mt + 4 * g;  // first output feature this lane holds
        const h4 v = __builtin_convertvector(acc[t], h4);
        const int64_t row = row0 + 16 * t + n;
        if (row < a.batch) {
            if constexpr (kVecOut) {
                constexpr int wl = N::w[L];
                if (c < wl)
                    *(h4 *)((_Float16 *)a.y + row * wl + c) = v;
            } else {
                _Float16 *yr = (_Float16 *)a.y + row * a.wL;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (c + i < a.wL)
                        yr[c + i] = v[i];
            }
        }
    }

    template <int... T>
    static __device__ __forceinline__ void store_outputs(const f4 (&acc)[NT], int mt, const LaunchArgs &a,
                                                         int64_t row0, int lane, std::integer_sequence<int, T...>)
    {
        (store_tile<T>(acc, mt, a, row0, lane), ...);
    }
};

// EU: waves per SIMD the instance is built for (its register budget is 512 / EU per lane).
template <class N, int NT, int WAVES, int EU, bool LDS_W, int LAYOUT, int ACT, bool GENERIC>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(EU, EU))) mlp_fused(LaunchArgs a)
{
    using Src = typename std::conditional<LDS_W, LdsSource, BufferSource>::type;
    using B = Body<N, NT, LAYOUT, ACT, GENERIC, LDS_W, Src>;
    constexpr int bytes = (int)N::image_bytes(LAYOUT);
    static_assert(bytes % 16 == 0, "image must be a multiple of 16 bytes");
    constexpr int kRows = NT * 16;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tiles = (a.batch + kRows - 1) / kRows;
    const int64_t stride = (int64_t)gridDim.x * WAVES;
    int64_t tile = (int64_t)blockIdx.x * WAVES + wave;

    // The first tile's inputs are requested before the weights are staged, so the two latencies
    // overlap; every later tile's inputs are requested one tile ahead.
    h8 Bnext[N::KB(0)][NT];
    B::load_inputs(Bnext, a, (tile < tiles ? tile : 0) * kRows, lane, std::make_integer_sequence<int, NT>());

    Src src;
    if constexpr (LDS_W) {
        __shared__ __attribute__((aligned(16))) uint8_t lds[bytes];
        for (int i = threadIdx.x * 16; i < bytes; i += WAVES * 64 * 16)
            *(uint4 *)(lds + i) = *(const uint4 *)(a.image + i);
        __syncthreads();
        src.base = lds;
    } else {
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.image, 0, bytes, kBufferRsrcWord3);
    }

    for (int it = 0; tile < tiles; tile += stride, ++it) {
        // Waves of a SIMD start together and the oldest one is issued first; left alone, some
        // race ahead and the last ones finish with nothing to overlap.  Giving the waves that are
        // behind the higher priority keeps them in step.
        set_priority(it);
        // The weights are loop-invariant; without this barrier the compiler hoists every fragment
        // read out of the tile loop and the whole image (up to ~1 KB per lane) spills.  The barrier
        // keeps them as per-tile reads, each reused across the NT sample tiles.
        asm volatile("" ::: "memory");
        constexpr int KB0 = N::KB(0);  // a constant expression, so the copy below fully unrolls
        h8 B0[KB0][NT];
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                B0[kb][t] = Bnext[kb][t];
        const int64_t next = tile + stride;
        if (next < tiles)
            B::load_inputs(Bnext, a, next * kRows, lane, std::make_integer_sequence<int, NT>());
        B::template layer<0>(src, B0, a, tile * kRows, lane);
    }
    __builtin_amdgcn_s_setprio(0);
}

template <class N, int NT, int WAVES, int EU, bool LDS_W, int LAYOUT, int ACT, bool GENERIC>
hipError_t launch(const LaunchArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((mlp_fused<N, NT, WAVES, EU, LDS_W, LAYOUT, ACT, GENERIC>), dim3(grid), dim3(WAVES * 64), 0, s, a);
    return hipGetLastError();
}

template <class N, int NT, int WAVES, int EU, bool LDS_W, int LAYOUT, int ACT, bool GENERIC>
KernelEntry entry(const char *name)
{
    KernelEntry e{};
    e.name = name;
    e.n_layers = N::L;
    for (int i = 0; i <= N::L; ++i)
        e.widths[i] = N::w[i];
    e.generic = GENERIC;
    e.layout = LAYOUT;
    e.act = ACT;
    e.threads = WAVES * 64;
    e.rows_per_wave = NT * 16;
    e.weights_in_lds = LDS_W;
    e.launch = &launch<N, NT, WAVES, EU, LDS_W, LAYOUT, ACT, GENERIC>;
    e.func = (const void *)&mlp_fused<N, NT, WAVES, EU, LDS_W, LAYOUT, ACT, GENERIC>;
    return e;
}

// ---- instances ------------------------------------------------------------------------------

using NetSmall = Net<16, 32, 32, 32, 32, 32, 32, 32, 4>;
using NetPage = Net<32, 64, 64, 64, 64, 64, 64, 64, 4>;
using NetHetero = Net<32, 64, 64, 64, 128, 64, 64, 32, 4>;
using NetWide = Net<64, 128, 128, 128, 128, 128, 128, 128, 4>;
using NetStream = Net<64, 64, 64, 64, 64, 64, 64, 64, 16>;

#define MLP_VARIANTS(NET, NT, WAVES, EU, LDS, TAG)                                                             \
    entry<NET, NT, WAVES, EU, LDS, kPacked, kVector, false>("mlp_fused<" TAG ",packed,vector>"),                  \
        entry<NET, NT, WAVES, EU, LDS, kPacked, kScalarised, false>("mlp_fused<" TAG ",packed,scalarised>"),      \
        entry<NET, NT, WAVES, EU, LDS, kRowMajor, kVector, false>("mlp_fused<" TAG ",rowmajor,vector>"),          \
        entry<NET, NT, WAVES, EU, LDS, kRowMajor, kScalarised, false>("mlp_fused<" TAG ",rowmajor,scalarised>")

#define MLP_GENERIC(...) entry<Net<__VA_ARGS__>, 1, 4, 2, false, kPacked, kVector, true>

static const KernelEntry kEntries[] = {
    // (net, rows tiles per wave, waves per workgroup, waves per SIMD, image in LDS)
    MLP_VARIANTS(NetSmall, 4, 8, 4, true, "16-32x7-4"),
    MLP_VARIANTS(NetPage, 4, 8, 4, true, "32-64x7-4"),
    MLP_VARIANTS(NetHetero, 4, 8, 4, true, "32-64-64-64-128-64-64-32-4"),
    MLP_VARIANTS(NetWide, 4, 4, 1, false, "64-128x7-4"),
    MLP_VARIANTS(NetStream, 4, 8, 4, true, "64-64x7-16"),
    MLP_GENERIC(128, 128)("mlp_fused<generic128,L=1>"),
    MLP_GENERIC(128, 128, 128)("mlp_fused<generic128,L=2>"),
    MLP_GENERIC(128, 128, 128, 128)("mlp_fused<generic128,L=3>"),
    MLP_GENERIC(128, 128, 128, 128, 128)("mlp_fused<generic128,L=4>"),
    MLP_GENERIC(128, 128, 128, 128, 128, 128)("mlp_fused<generic128,L=5>"),
    MLP_GENERIC(128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128,L=6>"),
    MLP_GENERIC(128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128,L=7>"),
    MLP_GENERIC(128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128,L=8>"),
};

const KernelEntry *registry(int *count)
{
    *count = (int)(sizeof(kEntries) / sizeof(kEntries[0]));
    return kEntries;
}

}  // namespace mlpk

// mlp_kernels.hip -- the fused eight-layer FP16 MLP inference kernel for gfx950 (CDNA4).
//
// One launch evaluates the whole network for every input row ("Profiling neural material inference",
// section "Experiment setup": the timed unit is the complete inference pass).  Design:
//   - persistent grid; each wave loops over tiles of NT x 16 rows;
//   - the weight image is staged once per workgroup into LDS (or, when it does not fit in LDS, read
//     through the caches), and every A fragment is one 16-byte read per lane reused across the
//     wave's NT sample tiles;
//   - each layer is v_mfma_f32_32x32x16_f16 with the bias as the C operand of the first K block
//     (FP16 x FP16 products, FP32 accumulation).  The 32x32 shape does twice the work of the
//     16x16x32 one per issued instruction, which leaves the VALU room for the epilogue: measured on
//     MI355X, about six packed-FP16 VALU instructions fit under each 32x32x16 MFMA at no cost, while
//     more than two per 16x16x32 MFMA already slow the MFMA pipe;
//   - the epilogue of layers 1..L-1 converts FP32 -> FP16 with round-to-nearest-even and applies the
//     leaky ReLU max(v, v * half(0.01)) as packed FP16 operations on whole registers, the vector form
//     of "Bad versus good activation"; by the slot order in mlp_layout.h the result already sits
//     where the next layer's B operand needs it, so activations never leave the registers;
//   - the last layer converts to FP16 (no activation) and stores the row's outputs.
// Variants for the page's two A/B comparisons: the row-major weight image (fragments assembled from
// the canonical [out][in] matrices with per-lane index arithmetic; staged in LDS with padded rows),
// and the scalarised activation (one component at a time, compare and branch,
// "if (v < 0) v *= half(0.01)").
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mlp_layout.h"
#include "mlp_registry.h"

namespace mlpk {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));

// half(0.01): 0.01 rounded to binary16 (0x211f = 0.01000213623046875).
__device__ __forceinline__ _Float16 slope() { return __builtin_bit_cast(_Float16, (unsigned short)0x211f); }

__device__ __forceinline__ f16x mfma(h8 a, h8 b, f16x c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Vector leaky ReLU on eight FP16 values: two packed instructions for every two values.
__device__ __forceinline__ h8 leaky_vector(h8 v)
{
    const h8 s = (h8)slope();
    return __builtin_elementwise_max(v, v * s);
}

// Scalarised leaky ReLU: each component on its own, with a compare and a conditional multiply.
__device__ __forceinline__ h8 leaky_scalarised(h8 v)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
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

// An LDS address voff + soff with a constant soff: a ds_read's immediate offset has 16 bits, so an
// soff of 64 KB or more is split into a 64 KB-aligned part added to voff (one register for every read
// that shares voff and that part: the empty asm hides the sum from constant folding, so the compiler
// computes it once rather than a register per distinct offset) and the rest as the immediate.
__device__ __forceinline__ const uint8_t *lds_addr(const uint8_t *base, int voff, int soff)
{
    if (soff >= 65536) {
        int vb = voff + (soff & ~0xffff);
        asm("" : "+v"(vb));
        return base + vb + (soff & 0xffff);
    }
    return base + voff + soff;
}

// Where the weight image is read from.  Offsets are split into a per-lane part (voff, a VGPR) and
// a wave-uniform constant part (soff) so that neither path needs a register per fragment address.
struct LdsSource {  // image staged in LDS: ds_read with the constant as an immediate offset
    const uint8_t *base;
    __device__ __forceinline__ h8 load16(int voff, int soff) const { return *(const h8 *)lds_addr(base, voff, soff); }
    __device__ __forceinline__ h4 load8(int voff, int soff) const { return *(const h4 *)lds_addr(base, voff, soff); }
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

// Images larger than LDS: the leading LAYERS whole layers are staged into LDS (row-major rows padded
// as in a fully staged image) and read from there, the rest through the caches; which of the two a
// layer uses is decided at compile time (Body::in_lds), per layer, for either layout.
template <int LAYERS>
struct HybridSource {
    static constexpr int kLayers = LAYERS;
    const uint8_t *base;
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ h8 lds16(int voff, int soff) const { return *(const h8 *)lds_addr(base, voff, soff); }
    __device__ __forceinline__ h4 lds8(int voff, int soff) const { return *(const h4 *)lds_addr(base, voff, soff); }
    __device__ __forceinline__ h8 buf16(int voff, int soff) const
    {
        return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
    }
    __device__ __forceinline__ h4 buf8(int voff, int soff) const
    {
        return __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, soff, 0));
    }
};

template <class S>
struct is_hybrid : std::false_type {};
template <int LAYERS>
struct is_hybrid<HybridSource<LAYERS>> : std::true_type {};

// LDS the staged weight image may use (the CU has 160 KB; a little is left for the kernel's own).
constexpr int kLdsImageBudget = 159 * 1024;

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Compile-time description of the network a kernel instance computes.
template <int... W>
struct Net {
    static constexpr int L = sizeof...(W) - 1;
    static constexpr int w[sizeof...(W)] = {W...};
    static constexpr int MT(int l) { return mlpl::m_tiles(w, l); }
    static constexpr int KB(int l) { return mlpl::k_blocks(w, l); }
    static constexpr size_t image_bytes(int layout) { return layout == kPacked ? mlpl::pk_bytes(w, L) : mlpl::rm_bytes(w, L); }
    // Bytes of the image as staged in LDS (row-major rows are padded there).
    static constexpr size_t lds_bytes(int layout) { return layout == kPacked ? mlpl::pk_bytes(w, L) : mlpl::rml_bytes(w, L); }
    // The longest run of whole layers, from layer 0, whose LDS copy fits the budget, and the bytes of
    // that prefix in the image (as stored) and in LDS (as staged).
    static constexpr size_t lds_off(int layout, int l) { return layout == kPacked ? mlpl::pk_a_off(w, l) : mlpl::rml_w_off(w, l); }
    static constexpr int lds_layers(int layout)
    {
        int l = 0;
        while (l < L && lds_off(layout, l + 1) <= (size_t)kLdsImageBudget)
            ++l;
        return l;
    }
    static constexpr int prefix_image_bytes(int layout, int p)
    {
        return (int)(layout == kPacked ? mlpl::pk_a_off(w, p) : mlpl::rm_w_off(w, p));
    }
};

// A generic network whose caller widths are taken at run time but are known to allow vector input
// and output (input width a multiple of 8, output width a multiple of 4): the host selects it only
// for such shapes.
template <int... W>
struct VecNet : Net<W...> {};
template <class N>
struct runtime_vec_io : std::false_type {};
template <int... W>
struct runtime_vec_io<VecNet<W...>> : std::true_type {};

template <class N, int NT, int LAYOUT, int ACT, bool GENERIC, bool LDS_W, class Src, bool DEFER>
struct Body {
    static constexpr int L = N::L;
    // Vector loads and stores: caller widths known at compile time (exact instances) that allow
    // them, or a generic instance for vector-friendly widths (then the row strides are run time).
    static constexpr bool kRtVec = GENERIC && runtime_vec_io<N>::value;
    static constexpr bool kVecIn = (!GENERIC && N::w[0] % 8 == 0) || kRtVec;
    static constexpr bool kVecOut = (!GENERIC && N::w[L] % 4 == 0) || kRtVec;
    // The last layer's outputs are held in registers and stored at the top of the next tile, after
    // that tile's inputs have been waited for: a store issued at the end of a tile would otherwise
    // sit in front of the next tile's wait (the vector-memory counter counts stores too) and every
    // tile would wait for its own store's round trip.  That wait only shows where fewer than three
    // waves share a SIMD and the weights come from LDS (measured: -2.8 % on the net with a 128-wide
    // layer; +0.4 % on the page net; +5 % on the net whose weights are read with buffer loads, where
    // the held store would sit in front of every weight fetch instead), so the instance chooses.
    static constexpr bool kDefer = DEFER && !GENERIC && kVecOut && N::MT(L - 1) == 1;
    // A last layer of at most 4 outputs runs on the 16x16x32 MFMA (mlp_layout.h, narrow_last).
    static constexpr bool kNarrow = !GENERIC && mlpl::narrow_last(N::w, L);
    static constexpr int kQ = (N::w[L] + 7) / 8;  // 8-output groups holding real outputs
    struct Pending {
        h4 v[NT][kQ];
    };

    // ---- weight delivery ------------------------------------------------------------------

    // Whether layer l is read from LDS (then a row-major layer has padded rows) or through the caches.
    static constexpr bool in_lds(int l)
    {
        if constexpr (is_hybrid<Src>::value)
            return l < Src::kLayers;
        else
            return LDS_W;
    }

    // 16- and 8-byte reads of layer l's part of the image, from LDS or through the caches.
    template <int l>
    static __device__ __forceinline__ h8 ld16(const Src &src, int voff, int soff)
    {
        if constexpr (is_hybrid<Src>::value) {
            if constexpr (in_lds(l))
                return src.lds16(voff, soff);
            else
                return src.buf16(voff, soff);
        } else {
            return src.load16(voff, soff);
        }
    }
    template <int l>
    static __device__ __forceinline__ h4 ld8(const Src &src, int voff, int soff)
    {
        if constexpr (is_hybrid<Src>::value) {
            if constexpr (in_lds(l))
                return src.lds8(voff, soff);
            else
                return src.buf8(voff, soff);
        } else {
            return src.load8(voff, soff);
        }
    }

    template <int l>
    static __device__ __forceinline__ h8 a_frag(const Src &src, int mt, int kb, int lane)
    {
        constexpr int KB = N::KB(l);
        if constexpr (LAYOUT == kPacked) {
            constexpr int a_off = (int)mlpl::pk_a_off(N::w, l);  // constant-evaluated, not computed per wave
            return ld16<l>(src, lane * 16, a_off + (mt * KB + kb) * mlpl::kFragBytes);
        } else {
            // Row-major [out][in]: lane (g, m) gathers row 32 mt + m at its slot features.  In LDS
            // the rows are padded (mlp_layout.h), in global memory they are as given.
            constexpr int win = N::w[l], wout = N::w[l + 1];
            static_assert(win % 8 == 0, "row-major layers need w_in % 8 == 0");
            constexpr int stride = in_lds(l) ? mlpl::rml_stride(l, win) : win * 2;
            constexpr int w_off = in_lds(l) ? (int)mlpl::rml_w_off(N::w, l) : (int)mlpl::rm_w_off(N::w, l);
            const int g = lane >> 5, m = lane & 31;
            const int r = 32 * mt + m;
            const int row = w_off + 32 * mt * stride;  // wave-uniform
            h8 a = (h8)(_Float16)0;
            if constexpr (l == 0) {
                if (r < wout && 16 * kb + 8 * g < win)
                    a = ld16<l>(src, m * stride + 8 * g * 2, row + 16 * kb * 2);
            } else {
                const int f0 = 16 * kb + 4 * g, f1 = f0 + 8;
                h4 lo = (h4)(_Float16)0, hi = (h4)(_Float16)0;
                if (r < wout && f0 < win)
                    lo = ld8<l>(src, m * stride + 4 * g * 2, row + 16 * kb * 2);
                if (r < wout && f1 < win)
                    hi = ld8<l>(src, m * stride + 4 * g * 2, row + (16 * kb + 8) * 2);
                a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return a;
        }
    }

    template <int l>
    static __device__ __forceinline__ f16x bias_tile(const Src &src, int mt, int lane)
    {
        const int g = lane >> 5;
        if constexpr (LAYOUT == kPacked) {
            constexpr int b_off = (int)mlpl::pk_b_off(N::w, l);
            const int soff = b_off + mt * mlpl::kBiasTileBytes;
            const f4 b0 = __builtin_bit_cast(f4, ld16<l>(src, g * 64, soff));
            const f4 b1 = __builtin_bit_cast(f4, ld16<l>(src, g * 64 + 16, soff));
            const f4 b2 = __builtin_bit_cast(f4, ld16<l>(src, g * 64 + 32, soff));
            const f4 b3 = __builtin_bit_cast(f4, ld16<l>(src, g * 64 + 48, soff));
            const f8 lo = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
            const f8 hi = __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        } else {
            constexpr int wout = N::w[l + 1];
            static_assert(wout % 4 == 0, "row-major layer needs w_out % 4 == 0");
            constexpr int b_off = in_lds(l) ? (int)mlpl::rml_b_off(N::w, l) : (int)mlpl::rm_b_off(N::w, l);
            const int soff = b_off + 32 * mt * 2;
            h4 q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                q[k] = (h4)(_Float16)0;
                if (32 * mt + 8 * k + 4 * g < wout)
                    q[k] = ld8<l>(src, (8 * k + 4 * g) * 2, soff);
            }
            const h8 lo = __builtin_shufflevector(q[0], q[1], 0, 1, 2, 3, 4, 5, 6, 7);
            const h8 hi = __builtin_shufflevector(q[2], q[3], 0, 1, 2, 3, 4, 5, 6, 7);
            return __builtin_convertvector(
                __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15), f16x);
        }
    }

    // ---- narrow last layer: both 16-sample halves of each B fragment in one 16x16x32 MFMA ---------
    //
    // Lane (a, i) of the A fragment holds output narrow_row(lane) over the slots of group lane / 32
    // (zeros elsewhere), so rows 0..3 of the result are sample 32 t + c and rows 4..7 sample
    // 32 t + 16 + c, and lane s < 32 ends with the four outputs of sample 32 t + s (mlp_layout.h).

    template <int l>
    static __device__ __forceinline__ h8 narrow_frag(const Src &src, int kb, int lane)
    {
        if constexpr (LAYOUT == kPacked) {
            constexpr int a_off = (int)mlpl::pk_a_off(N::w, l);
            return ld16<l>(src, lane * 16, a_off + kb * mlpl::kFragBytes);
        } else {
            // gathered from the row-major matrix: row narrow_row(lane), the slot features of group g
            constexpr int win = N::w[l], wout = N::w[l + 1];
            static_assert(win % 8 == 0, "row-major layers need w_in % 8 == 0");
            constexpr int stride = in_lds(l) ? mlpl::rml_stride(l, win) : win * 2;
            constexpr int w_off = in_lds(l) ? (int)mlpl::rml_w_off(N::w, l) : (int)mlpl::rm_w_off(N::w, l);
            const int g = lane >> 5, r = mlpl::narrow_row(lane);
            const bool live = r >= 0 && r < wout;
            const int m = live ? r : 0;
            h8 a = (h8)(_Float16)0;
            if constexpr (l == 0) {
                if (live && 16 * kb + 8 * g < win)
                    a = ld16<l>(src, m * stride + 8 * g * 2, w_off + 16 * kb * 2);
            } else {
                const int f0 = 16 * kb + 4 * g, f1 = f0 + 8;
                h4 lo = (h4)(_Float16)0, hi = (h4)(_Float16)0;
                if (live && f0 < win)
                    lo = ld8<l>(src, m * stride + 4 * g * 2, w_off + 16 * kb * 2);
                if (live && f1 < win)
                    hi = ld8<l>(src, m * stride + 4 * g * 2, w_off + (16 * kb + 8) * 2);
                a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return a;
        }
    }

    // C operand: b[0..3] in the lanes of both sample halves (a = lane / 16 < 2), zero in the others.
    template <int l>
    static __device__ __forceinline__ f4 narrow_bias(const Src &src, int lane)
    {
        if constexpr (LAYOUT == kPacked) {
            constexpr int b_off = (int)mlpl::pk_b_off(N::w, l);
            return __builtin_bit_cast(f4, ld16<l>(src, (lane >> 4) * 16, b_off));
        } else {
            // b [w_out] FP16, its section zero-padded to 16 bytes
            constexpr int soff = in_lds(l) ? (int)mlpl::rml_b_off(N::w, l) : (int)mlpl::rm_b_off(N::w, l);
            h4 q = ld8<l>(src, 0, soff);
            if (lane >= 32)
                q = (h4)(_Float16)0;
            return __builtin_convertvector(q, f4);
        }
    }

    template <int l>
    static __device__ __forceinline__ void narrow_layer(const Src &src, const h8 (&Bin)[N::KB(l)][NT],
                                                        const LaunchArgs &a, int64_t row0, int lane, Pending &pend)
    {
        constexpr int KB = N::KB(l);
        h8 af[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            af[kb] = narrow_frag<l>(src, kb, lane);
        const f4 bias = narrow_bias<l>(src, lane);
        f4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = mfma16(af[0], Bin[0][t], bias);
#pragma unroll
        for (int kb = 1; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = mfma16(af[kb], Bin[kb][t], acc[t]);
        if constexpr (kDefer) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                pend.v[t][0] = __builtin_convertvector(acc[t], h4);  // lanes < 32 hold real rows
        } else {
            constexpr int wl = N::w[L];
            if (lane < 32) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int64_t row = row0 + 32 * t + lane;
                    if (row < a.batch) {
                        const h4 v = __builtin_convertvector(acc[t], h4);
                        if constexpr (kVecOut) {
                            *(h4 *)((char *)((_Float16 *)a.y + row0 * wl) + (unsigned)((32 * t + lane) * wl * 2)) = v;
                        } else {
                            _Float16 *yr = (_Float16 *)a.y + row * wl;
#pragma unroll
                            for (int i = 0; i < wl; ++i)
                                yr[i] = v[i];
                        }
                    }
                }
            }
        }
    }

    // ---- one layer: NT sample tiles x MT output tiles x KB input blocks --------------------
    //
    // Software-pipelined over the output tiles mt: the fragments of tile mt+1 are requested first,
    // then tile mt's MFMAs are issued, then tile mt-1's epilogue runs.  The epilogue does not depend
    // on the MFMAs in flight, so the MFMA pipe and the VALU work side by side.

    template <int l>
    static __device__ __forceinline__ void fetch(const Src &src, int mt, h8 (&af)[N::KB(l)], f16x &bias, int lane)
    {
        constexpr int KB = N::KB(l);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            af[kb] = a_frag<l>(src, mt, kb, lane);
        bias = bias_tile<l>(src, mt, lane);
    }

    template <int l>
    static __device__ __forceinline__ void mfmas(const h8 (&af)[N::KB(l)], const h8 (&Bin)[N::KB(l)][NT],
                                                 const f16x &bias, f16x (&acc)[NT])
    {
        constexpr int KB = N::KB(l);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = mfma(af[0], Bin[0][t], bias);
#pragma unroll
        for (int kb = 1; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = mfma(af[kb], Bin[kb][t], acc[t]);
    }

    // FP32 -> FP16 (round to nearest even) and leaky ReLU of output tile mt; accumulator half h of
    // each lane is exactly block 2 mt + h of the next layer's B operand (see mlp_layout.h).
    template <int KBN>
    static __device__ __forceinline__ void epilogue(int mt, const f16x (&acc)[NT], h8 (&Bout)[KBN][NT])
    {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (2 * mt + h < KBN) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const f8 half = h == 0 ? __builtin_shufflevector(acc[t], acc[t], 0, 1, 2, 3, 4, 5, 6, 7)
                                           : __builtin_shufflevector(acc[t], acc[t], 8, 9, 10, 11, 12, 13, 14, 15);
                    const h8 v = __builtin_convertvector(half, h8);  // v_cvt_pk_f16_f32: nearest even
                    Bout[2 * mt + h][t] = (ACT == kVector) ? leaky_vector(v) : leaky_scalarised(v);
                }
            }
        }
    }

    template <int l>
    static __device__ __forceinline__ void layer(const Src &wb, const h8 (&Bin)[N::KB(l)][NT],
                                                 const LaunchArgs &a, int64_t row0, int lane, Pending &pend)
    {
        constexpr int MT = N::MT(l), KB = N::KB(l);
        // Weights read through the caches: keep each layer's reads inside the layer, or the
        // scheduler front-loads the whole network's fragments and runs out of registers.
        if constexpr (!LDS_W)
            asm volatile("" ::: "memory");
        if constexpr (kNarrow && l == L - 1) {
            narrow_layer<l>(wb, Bin, a, row0, lane, pend);
            return;
        }
        h8 af[KB];
        f16x bias;
        fetch<l>(wb, 0, af, bias, lane);
        if constexpr (l + 1 < L) {
            constexpr int KBN = N::KB(l + 1);
            h8 Bout[KBN][NT];
            f16x prev[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 afn[KB];
                f16x biasn;
                if (mt + 1 < MT)
                    fetch<l>(wb, mt + 1, afn, biasn, lane);
                f16x acc[NT];
                mfmas<l>(af, Bin, bias, acc);
                if (mt > 0)
                    epilogue<KBN>(mt - 1, prev, Bout);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    prev[t] = acc[t];
                if (mt + 1 < MT) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        af[kb] = afn[kb];
                    bias = biasn;
                }
            }
            epilogue<KBN>(MT - 1, prev, Bout);
            layer<l + 1>(wb, Bout, a, row0, lane, pend);
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                h8 afn[KB];
                f16x biasn;
                if (mt + 1 < MT)
                    fetch<l>(wb, mt + 1, afn, biasn, lane);
                f16x acc[NT];
                mfmas<l>(af, Bin, bias, acc);
                if constexpr (kDefer)
                    hold_outputs(acc, pend);
                else
                    store_outputs(acc, mt, a, row0, lane, std::make_integer_sequence<int, NT>());
                if (mt + 1 < MT) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        af[kb] = afn[kb];
                    bias = biasn;
                }
            }
        }
    }

    // ---- input rows -> layer-0 B fragments --------------------------------------------------
    //
    // Loads are issued one tile ahead and must not be waited for until the tile is used, so they
    // are raw (address clamped to a valid row and column, no select on the value: a select right
    // after the load would make the wave wait for it).  Rows past the batch and columns past w0 are
    // zeroed when the fragments are consumed.  Everything is written as one straight-line body per
    // sample tile (an index-sequence expansion) with constant-expression loop bounds, so the
    // fragment arrays stay in registers.

    template <int t>
    static __device__ __forceinline__ void load_tile(h8 (&R)[N::KB(0)][NT], const LaunchArgs &a, int64_t row0,
                                                     int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const int64_t row = row0 + 32 * t + n;
        const int64_t rr = row < a.batch ? row : a.batch - 1;
        constexpr int KB0 = N::KB(0);
        // The tile's first row is the same for the whole wave: the address is a uniform base plus
        // a 32-bit lane offset (row within the tile clamped to the batch), which the loads take as
        // a scalar base and a vector offset, with no 64-bit address arithmetic per lane.
        const int in_tile = 32 * t + n;
        const int last = (int)(a.batch - 1 - row0 < NT * 32 - 1 ? a.batch - 1 - row0 : NT * 32 - 1);
        const int r32 = in_tile < last ? in_tile : last;
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb) {
            const int c = 16 * kb + 8 * g;
            if constexpr (kVecIn) {
                const int w0 = kRtVec ? a.w0 : N::w[0];  // a constant for exact instances
                const int cc = (16 * kb + 16 <= w0 || c < w0) ? c : w0 - 8;  // folds for whole blocks
                const char *base = (const char *)((const _Float16 *)a.x + row0 * w0);
                R[kb][t] = *(const h8 *)(base + (unsigned)((r32 * w0 + cc) * 2));
            } else {
                const _Float16 *xr = (const _Float16 *)a.x + rr * a.w0;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    R[kb][t][j] = xr[c + j < a.w0 ? c + j : a.w0 - 1];
            }
        }
    }

    template <int... T>
    static __device__ __forceinline__ void load_inputs(h8 (&R)[N::KB(0)][NT], const LaunchArgs &a, int64_t row0,
                                                       int lane, std::integer_sequence<int, T...>)
    {
        (load_tile<T>(R, a, row0, lane), ...);
    }

    // B = R with the padded slots (columns >= w0) and the rows past the batch set to zero.
    template <int t>
    static __device__ __forceinline__ void mask_tile(h8 (&B)[N::KB(0)][NT], const h8 (&R)[N::KB(0)][NT],
                                                     const LaunchArgs &a, int64_t row0, int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const bool live = row0 + 32 * t + n < a.batch;
        constexpr int KB0 = N::KB(0);
#pragma unroll
        for (int kb = 0; kb < KB0; ++kb) {
            const int c = 16 * kb + 8 * g;
            if constexpr (kVecIn) {
                const int w0 = kRtVec ? a.w0 : N::w[0];
                const bool in = 16 * kb + 16 <= w0 || c < w0;  // folds for whole blocks
                B[kb][t] = (live && in) ? R[kb][t] : (h8)(_Float16)0;
            } else {
                h8 v = R[kb][t];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[j] = (live && c + j < a.w0) ? v[j] : (_Float16)0;
                B[kb][t] = v;
            }
        }
    }

    template <int... T>
    static __device__ __forceinline__ void mask_inputs(h8 (&B)[N::KB(0)][NT], const h8 (&R)[N::KB(0)][NT],
                                                       const LaunchArgs &a, int64_t row0, int lane,
                                                       std::integer_sequence<int, T...>)
    {
        (mask_tile<T>(B, R, a, row0, lane), ...);
    }

    // ---- last layer: FP32 -> FP16 and store -------------------------------------------------

    template <int t>
    static __device__ __forceinline__ void store_tile(const f16x (&acc)[NT], int mt, const LaunchArgs &a,
                                                      int64_t row0, int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        const int64_t row = row0 + 32 * t + n;
        if (row < a.batch) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 32 * mt + 8 * q + 4 * g;  // first of the 4 outputs held by this lane
                const f4 part = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
                if constexpr (kVecOut) {
                    const int wl = kRtVec ? a.wL : N::w[L];
                    if (32 * mt + 8 * q < wl && c < wl)
                        *(h4 *)((char *)((_Float16 *)a.y + row0 * wl) + (unsigned)(((32 * t + n) * wl + c) * 2)) =
                            __builtin_convertvector(part, h4);
                } else {
                    _Float16 *yr = (_Float16 *)a.y + row * a.wL;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c + i < a.wL)
                            yr[c + i] = (_Float16)part[i];
                }
            }
        }
    }

    template <int... T>
    static __device__ __forceinline__ void store_outputs(const f16x (&acc)[NT], int mt, const LaunchArgs &a,
                                                         int64_t row0, int lane, std::integer_sequence<int, T...>)
    {
        (store_tile<T>(acc, mt, a, row0, lane), ...);
    }

    // Deferred form (one output tile, vector stores): convert now, store at the next tile's top.
    static __device__ __forceinline__ void hold_outputs(const f16x (&acc)[NT], Pending &pend)
    {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                const f4 part = {acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
                pend.v[t][q] = __builtin_convertvector(part, h4);
            }
    }

    static __device__ __forceinline__ void store_pending(const Pending &pend, const LaunchArgs &a, int64_t row0,
                                                         int lane)
    {
        const int g = lane >> 5, n = lane & 31;
        constexpr int wl = N::w[L];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t row = row0 + 32 * t + n;
            if (row < a.batch) {
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    const int c = 8 * q + 4 * g;
                    if (c < wl)
                        *(h4 *)((char *)((_Float16 *)a.y + row0 * wl) + (unsigned)(((32 * t + n) * wl + c) * 2)) = pend.v[t][q];
                }
            }
        }
    }
};

// Copy the weight image into LDS with every load in flight before the first store (the copy is a
// handful of 16-byte loads per thread, so its cost is one round trip rather than one per load).
// Written as index-sequence expansions with constant indices: a loop-indexed staging array would
// be placed in LDS by the compiler.  Load addresses are clamped into the image; only in-range
// chunks are stored.
//
// The loads and the stores are separate steps: the kernel issues the first tile's input loads in
// between, behind the image loads, so the stores wait for the image (from L2) and not for the
// inputs (every wave of the chip requests its first tile's inputs from HBM at the same moment).
// The empty asm reads every loaded chunk before the first store: without it the compiler moves the
// load of a chunk that only some threads store into the branch around that store, which turns the
// copy into two round trips, the second behind the input loads.
template <int C>
struct Chunks {
    uint4 v[C];
};

// An empty use of a loaded value: the load must have been issued (and waited for) before this point.
__device__ __forceinline__ void loaded(const uint4 &v) { asm volatile("" ::"v"(v.x)); }

// A 16-byte LDS store written component by component (a whole-struct copy kept the chunk array in
// memory, which the compiler then placed in LDS).
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

// LDS offset of the 16-byte chunk at byte offset g of a row-major image (all widths multiples of 8,
// so every row is a whole number of chunks): its row moves to the padded row stride.
template <class N, int... L>
__device__ __forceinline__ int rowmajor_lds_offset(int g, std::integer_sequence<int, L...>)
{
    int o = 0;
    const auto one = [&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int w0 = (int)mlpl::rm_w_off(N::w, l), b0 = (int)mlpl::rm_b_off(N::w, l);
        constexpr int end = (int)mlpl::rm_w_off(N::w, l + 1), row = N::w[l] * 2;
        if (g >= w0 && g < end)
            o = g < b0 ? (int)mlpl::rml_w_off(N::w, l) + (g - w0) / row * mlpl::rml_stride(l, N::w[l]) + (g - w0) % row
                       : (int)mlpl::rml_b_off(N::w, l) + (g - b0);
    };
    (one(std::integral_constant<int, L>()), ...);
    return o;
}

// Stage a row-major image into LDS with padded rows (same load pattern as stage_image).  Padded rows
// are only 8-byte aligned, so each 16-byte chunk is stored as two 8-byte halves.
__device__ __forceinline__ void store_chunk8(uint8_t *dst, const uint4 &v)
{
    ((uint2 *)dst)[0] = make_uint2(v.x, v.y);
    ((uint2 *)dst)[1] = make_uint2(v.z, v.w);
}

template <class N, int BYTES, int THREADS, int... K>
__device__ __forceinline__ void stage_store_rowmajor(uint8_t *lds, const Chunks<sizeof...(K)> &c,
                                                     std::integer_sequence<int, K...>)
{
    const int t16 = (int)threadIdx.x * 16;
    (loaded(c.v[K]), ...);
    ((K * THREADS * 16 + t16 < BYTES
          ? store_chunk8(lds + rowmajor_lds_offset<N>(K * THREADS * 16 + t16, std::make_integer_sequence<int, N::L>()), c.v[K])
          : (void)0),
     ...);
}

// EU: waves per SIMD the instance is built for (its register budget is 512 / EU per lane).
//
// Work distribution: workgroup b owns the contiguous tiles [lo, hi) of an even split; its waves take
// the first WAVES of them and then claim the next unclaimed tile from a counter in LDS.  The waves
// sharing a SIMD are not issued fairly (the oldest goes first), so with a fixed share per wave one of
// them finishes well before the other and the SIMD runs the rest half-empty; claiming tiles keeps
// every wave busy until the range is exhausted.
template <class N, int NT, int WAVES, int EU, bool LDS_W, int LAYOUT, int ACT, bool GENERIC>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(EU, EU))) mlp_fused(LaunchArgs a)
{
    // Weights: the whole image in LDS (LDS_W), else the layers that fit in LDS and the rest through
    // the caches (packed layout), else everything through the caches.
    constexpr int kLdsLayers = !LDS_W ? N::lds_layers(LAYOUT) : 0;
    using Src = typename std::conditional<
        LDS_W, LdsSource, typename std::conditional<(kLdsLayers > 0), HybridSource<kLdsLayers>, BufferSource>::type>::type;
    using B = Body<N, NT, LAYOUT, ACT, GENERIC, LDS_W, Src, (EU < 3 && LDS_W)>;
    constexpr int bytes = (int)N::image_bytes(LAYOUT);
    constexpr int lbytes = (int)N::lds_bytes(LAYOUT);
    static_assert(bytes % 16 == 0, "image must be a multiple of 16 bytes");
    constexpr int kRows = NT * 32;
    __shared__ int next_tile;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tiles = (a.batch + kRows - 1) / kRows;
    const int64_t lo = (int64_t)blockIdx.x * tiles / gridDim.x;
    const int64_t hi = ((int64_t)blockIdx.x + 1) * tiles / gridDim.x;
    // Each wave starts with two tiles of its own; later tiles are claimed two ahead, so neither the
    // claim's result nor a tile's inputs are waited for in the iteration that requests them.
    int64_t tile = lo + wave;
    int64_t next = lo + WAVES + wave;

    // The first tile's inputs are requested right behind the weight image's loads, so the two
    // latencies overlap; every later tile's inputs are requested at the end of the tile before it,
    // straight into the layer-0 fragments (no prefetch buffer and no copy: 16 fewer registers; the
    // other waves of the SIMD cover the wait).
    constexpr int KB0 = N::KB(0);  // a constant expression, so the loops below fully unroll
    h8 B0[KB0][NT];  // this tile's inputs, loaded at the end of the previous tile
    Src src;
    if constexpr (LDS_W) {
        __shared__ __attribute__((aligned(16))) uint8_t lds[lbytes];
        constexpr int kChunks = (bytes + WAVES * 64 * 16 - 1) / (WAVES * 64 * 16);
        const auto chunks = stage_load<bytes, WAVES * 64>(a.image, std::make_integer_sequence<int, kChunks>());
        B::load_inputs(B0, a, (tile < hi ? tile : lo) * kRows, lane, std::make_integer_sequence<int, NT>());
        if constexpr (LAYOUT == kPacked)
            stage_store<bytes, WAVES * 64>(lds, chunks, std::make_integer_sequence<int, kChunks>());
        else
            stage_store_rowmajor<N, bytes, WAVES * 64>(lds, chunks, std::make_integer_sequence<int, kChunks>());
        src.base = lds;
    } else if constexpr (kLdsLayers > 0) {
        // the leading kLdsLayers layers: kPrefix bytes of the image, kLdsPrefix bytes in LDS
        constexpr int kPrefix = N::prefix_image_bytes(LAYOUT, kLdsLayers);
        constexpr int kLdsPrefix = (int)N::lds_off(LAYOUT, kLdsLayers);
        __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsPrefix];
        constexpr int kChunks = (kPrefix + WAVES * 64 * 16 - 1) / (WAVES * 64 * 16);
        const auto chunks = stage_load<kPrefix, WAVES * 64>(a.image, std::make_integer_sequence<int, kChunks>());
        B::load_inputs(B0, a, (tile < hi ? tile : lo) * kRows, lane, std::make_integer_sequence<int, NT>());
        if constexpr (LAYOUT == kPacked)
            stage_store<kPrefix, WAVES * 64>(lds, chunks, std::make_integer_sequence<int, kChunks>());
        else
            stage_store_rowmajor<N, kPrefix, WAVES * 64>(lds, chunks, std::make_integer_sequence<int, kChunks>());
        src.base = lds;
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.image, 0, bytes, kBufferRsrcWord3);
    } else {
        B::load_inputs(B0, a, (tile < hi ? tile : lo) * kRows, lane, std::make_integer_sequence<int, NT>());
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a.image, 0, bytes, kBufferRsrcWord3);
    }
    if (threadIdx.x == 0)
        next_tile = 2 * WAVES;  // tiles are counted from lo
    __syncthreads();

    int claimed = 0;
    if (lane == 0)
        claimed = atomicAdd(&next_tile, 1);
    typename B::Pending pend;
    int64_t held_row0 = -1;  // first row of the tile whose outputs are held in pend
    while (tile < hi) {
        // The weights are loop-invariant; without this barrier the compiler hoists every fragment
        // read out of the tile loop and the whole image (up to ~1 KB per lane) spills.  The barrier
        // keeps them as per-tile reads, each reused across the NT sample tiles.
        asm volatile("" ::: "memory");
        constexpr bool kWholeBlocks = B::kVecIn && !B::kRtVec && N::w[0] % 16 == 0;
        if (!(kWholeBlocks && (tile + 1) * kRows <= a.batch))
            B::mask_inputs(B0, B0, a, tile * kRows, lane, std::make_integer_sequence<int, NT>());
        if constexpr (B::kDefer)
            if (held_row0 >= 0)
                B::store_pending(pend, a, held_row0, lane);
        const int64_t after = lo + __builtin_amdgcn_readfirstlane(claimed);  // claimed one tile ago
        if (lane == 0)
            claimed = atomicAdd(&next_tile, 1);
        B::template layer<0>(src, B0, a, tile * kRows, lane, pend);
        if (next < hi)
            B::load_inputs(B0, a, next * kRows, lane, std::make_integer_sequence<int, NT>());
        held_row0 = tile * kRows;
        tile = next;
        next = after;
    }
    if constexpr (B::kDefer)
        if (held_row0 >= 0)
            B::store_pending(pend, a, held_row0, lane);
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
    e.rows_per_wave = NT * 32;
    e.weights_in_lds = LDS_W;
    e.launch = &launch<N, NT, WAVES, EU, LDS_W, LAYOUT, ACT, GENERIC>;
    e.func = (const void *)&mlp_fused<N, NT, WAVES, EU, LDS_W, LAYOUT, ACT, GENERIC>;
    e.vec_io = GENERIC && runtime_vec_io<N>::value;
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

#define MLP_GENERIC64V3(...) entry<VecNet<__VA_ARGS__>, 2, 12, 3, true, kPacked, kVector, true>
#define MLP_GENERIC64V(...) entry<VecNet<__VA_ARGS__>, 2, 8, 2, true, kPacked, kVector, true>
#define MLP_GENERIC64(...) entry<Net<__VA_ARGS__>, 2, 8, 2, true, kPacked, kVector, true>
#define MLP_GENERIC128V(...) entry<VecNet<__VA_ARGS__>, 1, 8, 2, false, kPacked, kVector, true>
#define MLP_GENERIC(...) entry<Net<__VA_ARGS__>, 1, 4, 1, false, kPacked, kVector, true>

// Launch shapes, measured on MI355X: three waves per SIMD (12 per workgroup, one workgroup per compute
// unit) beat two by 2-3 % on the 64-wide nets, whose kernels fit the 168-register budget without
// spills; the net with a 128-wide layer needs more registers and stays at two (at three it spills and
// runs ~15 % slower).  Tiles of 96 rows (NT = 3) were 1 % slower than 64 on the page-shaped net.
// The generic kernels pad every width to 64 (the image in LDS, two waves per SIMD: at three the
// per-element input and output code spills 228-284 bytes) or to 128, each with vector input and
// output for input widths that are multiples of 8 and output widths that are multiples of 4, or
// element by element for the others; a shape takes the first family that serves it.  The 64-wide
// vector kernels run at three waves per SIMD up to six layers (1-5 % faster than two; seven and eight
// layers spill there and stay at two); the 128-wide vector kernels fit two waves per SIMD (169-218
// registers; 4-23 % faster than one), the 128-wide element-by-element ones spill there and stay at
// one.
static const KernelEntry kEntries[] = {
    // (net, 32-row tiles per wave, waves per workgroup, waves per SIMD, image in LDS)
    MLP_VARIANTS(NetSmall, 2, 8, 4, true, "16-32x7-4"),
    MLP_VARIANTS(NetPage, 2, 12, 3, true, "32-64x7-4"),
    MLP_VARIANTS(NetHetero, 2, 8, 2, true, "32-64-64-64-128-64-64-32-4"),
    MLP_VARIANTS(NetWide, 2, 8, 2, false, "64-128x7-4"),
    MLP_VARIANTS(NetStream, 2, 12, 3, true, "64-64x7-16"),
    MLP_GENERIC64V3(64, 64)("mlp_fused<generic64v,L=1>"),
    MLP_GENERIC64V3(64, 64, 64)("mlp_fused<generic64v,L=2>"),
    MLP_GENERIC64V3(64, 64, 64, 64)("mlp_fused<generic64v,L=3>"),
    MLP_GENERIC64V3(64, 64, 64, 64, 64)("mlp_fused<generic64v,L=4>"),
    MLP_GENERIC64V3(64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=5>"),
    MLP_GENERIC64V3(64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=6>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=7>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=8>"),
    // deeper narrow nets (all widths at most 64), vector I/O only: the image of 16 layers takes
    // ~140 KB of LDS (one workgroup of two waves per SIMD per CU)
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=9>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=10>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=11>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=12>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=13>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=14>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=15>"),
    MLP_GENERIC64V(64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64v,L=16>"),
    MLP_GENERIC64(64, 64)("mlp_fused<generic64,L=1>"),
    MLP_GENERIC64(64, 64, 64)("mlp_fused<generic64,L=2>"),
    MLP_GENERIC64(64, 64, 64, 64)("mlp_fused<generic64,L=3>"),
    MLP_GENERIC64(64, 64, 64, 64, 64)("mlp_fused<generic64,L=4>"),
    MLP_GENERIC64(64, 64, 64, 64, 64, 64)("mlp_fused<generic64,L=5>"),
    MLP_GENERIC64(64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64,L=6>"),
    MLP_GENERIC64(64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64,L=7>"),
    MLP_GENERIC64(64, 64, 64, 64, 64, 64, 64, 64, 64)("mlp_fused<generic64,L=8>"),
    MLP_GENERIC128V(128, 128)("mlp_fused<generic128v,L=1>"),
    MLP_GENERIC128V(128, 128, 128)("mlp_fused<generic128v,L=2>"),
    MLP_GENERIC128V(128, 128, 128, 128)("mlp_fused<generic128v,L=3>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128)("mlp_fused<generic128v,L=4>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=5>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=6>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=7>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=8>"),
    // deeper nets with a width above 64 (layers 0-3 in LDS, the rest through the caches), taken only
    // where the layer-by-layer path would not run the whole network as one chain (which is faster)
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=9>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=10>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=11>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=12>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=13>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=14>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=15>"),
    MLP_GENERIC128V(128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128, 128)("mlp_fused<generic128v,L=16>"),
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

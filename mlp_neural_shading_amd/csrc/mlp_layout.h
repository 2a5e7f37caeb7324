// mlp_layout.h -- geometry of the device weight images, shared by the host packer and the kernels.
//
// Tiling.  Every layer runs as v_mfma_f32_32x32x16_f16 with the weights in the A operand (32 output
// features x 16 input features per fragment), the samples in the B operand (16 input features x 32
// samples) and the 32x32 FP32 result in D.  Lane l of a wave is (g, n) = (l / 32, l % 32):
//   A fragment: lane (g, m) holds row m and the 8 input-feature "slots" of group g,
//   B fragment: lane (g, n) holds sample n and the same 8 slots,
//   D fragment: lane (g, n) holds, for sample n, the 16 output features 8 q + 4 g + i (q, i in 0..3),
//               as accumulator element j = 4 q + i.
// Only the pairing of A's and B's slots matters to the product, so the slot -> feature map is ours
// to choose, per layer; block kb always covers input features 16 kb .. 16 kb + 15:
//   layer 0 (reads the caller's row-major input): slot (kb, g, j) = feature 16 kb + 8 g + j, so one
//     16-byte load per lane fills a B fragment;
//   layer l >= 1: slot (kb, g, j) = feature 16 kb + 8 (j / 4) + 4 g + j % 4.  Output tile mt of the
//     previous layer feeds blocks 2 mt and 2 mt + 1, and accumulator elements 8 h .. 8 h + 7 of lane
//     (g, n) are exactly slots 0..7 of block 2 mt + h in the same lane: the hand-off between layers
//     is an in-lane FP32 -> FP16 convert of each half of the accumulator, with no data movement.
// The packer applies this permutation to the weight columns once ("Row-major versus
// InferencingOptimal weights": the optimal layout is a one-time reordering of the same matrices).
//
// Packed image, per layer l (MT = output tiles of 32, KB = input blocks of 16):
//   A fragments  [mt][kb][lane][8 halves]   1024 bytes per fragment, one ds_read_b128 per lane
//   bias tiles   [mt][g][16 floats]         FP32, lane (g, n) reads b[32 mt + 8 q + 4 g + i]
// (a last layer of at most 4 outputs is laid out for a smaller MFMA, see narrow_last below).
// Row-major image, per layer l: W_l [w_out][w_in] FP16 as given, then b_l [w_out] FP16, each
// section padded to a multiple of 16 bytes.
#pragma once

#include <stddef.h>

namespace mlpl {

constexpr int kTileM = 32;  // output features per A fragment (and samples per B fragment)
constexpr int kTileK = 16;  // input features per A fragment
constexpr int kFragBytes = 64 * 8 * 2;
constexpr int kBiasTileBytes = 32 * 4;

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
constexpr int k0_pad(int w0) { return round_up(w0, kTileK); }

// w: the kernel's widths w[0..L]
constexpr int m_tiles(const int *w, int l) { return (w[l + 1] + kTileM - 1) / kTileM; }
constexpr int k_blocks(const int *w, int l) { return (w[l] + kTileK - 1) / kTileK; }

// Input feature carried by slot (kb, g, j) of layer l.
constexpr int slot_feature(int l, int kb, int g, int j)
{
    return l == 0 ? kTileK * kb + 8 * g + j : kTileK * kb + 8 * (j / 4) + 4 * g + (j % 4);
}

// Output feature held in accumulator element j of lane group g for output tile mt.
constexpr int acc_feature(int mt, int g, int j) { return kTileM * mt + 8 * (j / 4) + 4 * g + (j % 4); }

// Narrow last layer (at most 4 outputs, e.g. the page network's 4-wide output).  A 32x32 tile would
// spend 28 of its 32 rows on padding, so this layer runs as v_mfma_f32_16x16x32_f16 instead (half the
// MFMA time per input block), which reads a lane of the 32-sample B fragment as it stands: lane
// l = 16 a + c of that MFMA is column c and K group a, which here carries sample 32 t + 16 (a % 2) + c
// and the slots of group a / 2.  The A fragment therefore holds every output twice, once per sample
// half: lane (a, i) holds output i % 4 over the slots of group a / 2 when i / 4 == a % 2 and i < 8,
// else zeros, so D rows 0..3 are the outputs of samples 32 t + c and rows 4..7 those of samples
// 32 t + 16 + c.  By the MFMA's output layout (lane 16 a + c holds rows 4 a .. 4 a + 3 of column c),
// lane s < 32 ends with the four outputs of sample 32 t + s.
//   A fragments  [kb][lane][8 halves]     one per input block, slots as for any other layer
//   bias         [a][4 floats]            b[0..3] for a = 0, 1 (the C operand of both halves), 0 for
//                                         a = 2, 3; the rest of the layer's bias tile is zero
constexpr int kNarrowOut = 4;
constexpr bool narrow_last(const int *w, int L) { return w[L] <= kNarrowOut; }
// Output (0..3) that lane `lane` of a narrow A fragment holds, or -1 for a zero lane.
constexpr int narrow_row(int lane)
{
    return (lane % 16) < 2 * kNarrowOut && (lane % 16) / kNarrowOut == (lane / 16) % 2 ? (lane % 16) % kNarrowOut : -1;
}

constexpr size_t pk_a_bytes(const int *w, int l) { return (size_t)m_tiles(w, l) * k_blocks(w, l) * kFragBytes; }
constexpr size_t pk_layer_bytes(const int *w, int l) { return pk_a_bytes(w, l) + (size_t)m_tiles(w, l) * kBiasTileBytes; }
constexpr size_t pk_a_off(const int *w, int l)
{
    size_t o = 0;
    for (int i = 0; i < l; ++i)
        o += pk_layer_bytes(w, i);
    return o;
}
constexpr size_t pk_b_off(const int *w, int l) { return pk_a_off(w, l) + pk_a_bytes(w, l); }
constexpr size_t pk_bytes(const int *w, int L) { return pk_a_off(w, L); }

constexpr size_t rm_w_bytes(const int *w, int l) { return (size_t)round_up(w[l + 1] * w[l] * 2, 16); }
constexpr size_t rm_b_bytes(const int *w, int l) { return (size_t)round_up(w[l + 1] * 2, 16); }
constexpr size_t rm_w_off(const int *w, int l)
{
    size_t o = 0;
    for (int i = 0; i < l; ++i)
        o += rm_w_bytes(w, i) + rm_b_bytes(w, i);
    return o;
}
constexpr size_t rm_b_off(const int *w, int l) { return rm_w_off(w, l) + rm_w_bytes(w, l); }
constexpr size_t rm_bytes(const int *w, int L) { return rm_w_off(w, L); }

// Row-major image as staged in LDS: the same matrices with padded rows ("Optimization Techniques",
// "Avoiding Bank Conflicts": pad the row stride), so that the 32 rows one fragment read touches
// fall in distinct LDS banks (64 banks of 4 bytes).  Unpadded, a 64-wide layer's 128-byte rows all
// start in the same bank.  Widths are multiples of 8.
//   layer 0: each lane reads 16 bytes (ds_read_b128, 16-byte aligned); stride w_in * 2 + 16 bytes
//            puts consecutive rows 4 banks apart (mod 64), so every 16 rows cover the 64 banks once;
//   layers >= 1: each lane reads 8 bytes twice (ds_read_b64); stride w_in * 2 + 8 bytes is 2 x an
//            odd number of banks, so the 32 rows start on 32 distinct even banks and cover all 64.
// Every section starts on a 16-byte boundary; rows of layers >= 1 are 8-byte aligned.
constexpr int rml_stride(int l, int win) { return win * 2 + (l == 0 ? 16 : 8); }
constexpr size_t rml_w_bytes(const int *w, int l) { return (size_t)round_up(w[l + 1] * rml_stride(l, w[l]), 16); }
constexpr size_t rml_w_off(const int *w, int l)
{
    size_t o = 0;
    for (int i = 0; i < l; ++i)
        o += rml_w_bytes(w, i) + rm_b_bytes(w, i);
    return o;
}
constexpr size_t rml_b_off(const int *w, int l) { return rml_w_off(w, l) + rml_w_bytes(w, l); }
constexpr size_t rml_bytes(const int *w, int L) { return rml_w_off(w, L); }

// ---- FP8 image (v_mfma_f32_32x32x64_f8f6f4, OCP E4M3 operands) ------------------------------
//
// The FP8 MFMA takes 64 input features per block: lane (g, m) of the A operand holds 32 bytes, slots
// j = 0..31 of group g for row m, and pairs slot (g, j) with the same slot of the B operand (lane
// (g, n), sample n); the 32x32 FP32 result has the same lane layout as the FP16 MFMA's.  Slots:
//   layer 0 (reads the caller's rows): slot (kb, g, j) = feature 64 kb + 32 g + j;
//   layer l >= 1: output tiles 2 kb and 2 kb + 1 of the previous layer fill block kb, the first in
//     slots 0..15 and the second in 16..31, each as its accumulator elements in order:
//     slot (kb, g, j) = feature 32 (2 kb + j / 16) + 8 ((j % 16) / 4) + 4 g + j % 4.
// Per layer: A fragments [mt][kb][lane][32 bytes] (2 KB each), then the row scales
// [ceil(MT / 4)][lane][4 bytes] (byte i of lane (g, m)'s word: the E8M0 code of row
// 32 (4 q + i) + m, selected by the MFMA's op_sel), then FP32 bias tiles as in the FP16 image.
constexpr int kF8FragBytes = 64 * 32;
constexpr int f8_k_blocks(const int *w, int l) { return (w[l] + 63) / 64; }
constexpr int f8_slot_feature(int l, int kb, int g, int j)
{
    return l == 0 ? 64 * kb + 32 * g + j : 32 * (2 * kb + j / 16) + 8 * ((j % 16) / 4) + 4 * g + j % 4;
}
constexpr size_t f8_a_bytes(const int *w, int l) { return (size_t)m_tiles(w, l) * f8_k_blocks(w, l) * kF8FragBytes; }
constexpr size_t f8_s_bytes(const int *w, int l) { return (size_t)((m_tiles(w, l) + 3) / 4) * 256; }
constexpr size_t f8_layer_bytes(const int *w, int l)
{
    return f8_a_bytes(w, l) + f8_s_bytes(w, l) + (size_t)m_tiles(w, l) * kBiasTileBytes;
}
constexpr size_t f8_a_off(const int *w, int l)
{
    size_t o = 0;
    for (int i = 0; i < l; ++i)
        o += f8_layer_bytes(w, i);
    return o;
}
constexpr size_t f8_s_off(const int *w, int l) { return f8_a_off(w, l) + f8_a_bytes(w, l); }
constexpr size_t f8_b_off(const int *w, int l) { return f8_s_off(w, l) + f8_s_bytes(w, l); }
constexpr size_t f8_bytes(const int *w, int L) { return f8_a_off(w, L); }

}  // namespace mlpl

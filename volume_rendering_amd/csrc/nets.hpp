// Network layouts shared by the host packer and the device kernels.
//
// A network is a list of dense layers.  Each layer reads one or two input
// segments (the previous hidden state, a frequency encoding, or a feature
// vector such as grid features or harmonics) and has n_out outputs.
//
// Matrix-engine mapping (gfx950, wave64).  A layer is computed transposed,
// D[out, sample] = W[out, k] * X[k, sample], so that the output
// accumulators of one layer are already, register for register, the B
// operand of the next layer:
//   bf16: v_mfma_f32_32x32x16_bf16.  A tile is 32 outputs x 16 k; lane l
//         holds row l%32, k = 8*(l/32) .. +7.  B holds sample l%32, the same
//         k.  D lane l holds sample l%32, rows 8*(r/4) + 4*(l/32) + r%4 for
//         accumulator r = 0..15.
//   f32:  v_mfma_f32_32x32x2_f32.  A tile is 32 outputs x 2 k; lane l holds
//         row l%32, k = l/32; B and D as above.
// Output block ob of a layer (32 outputs) therefore becomes 2 k-blocks
// (bf16) or 16 k-steps (f32) of the next layer, in a permuted k order that
// the packer applies to the next layer's weight columns.  The permutation
// changes only the order of the terms of each dot product.
//
// Frequency-encoding inputs are supplied in (sin, cos) pairs of one
// argument so each lane evaluates one sincospi per pair: pair P < 3L is
// (sin, cos)(pi 2^(P/3) x[P%3]); pair 3L is (x, y); pair 3L+1 is (z, 0).
// In float32 an encoding segment is zero-padded to a whole number of
// 16-step groups (the unit in which the looped float32 network streams its
// weight tiles).
//
// Packed buffer: all A tiles (layer order; within a layer output block
// major, k-step minor; 64 operands per tile), zero padding to a 16 KB boundary,
// then all biases (layer order; [ob][half][16] float32 in accumulator
// order).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __HIPCC__
#define NERF_HD __host__ __device__
#else
#define NERF_HD
#endif

namespace nerf {

enum SegKind : int { SEG_NONE = 0, SEG_HIDDEN = 1, SEG_ENC = 2, SEG_FEAT = 3 };

struct Seg {
    int kind;
    int width;  // logical inputs: hidden width, 3 + 6L for encodings, feature count
    int L;      // frequencies (SEG_ENC)
};

struct Layer {
    int n_out;
    int relu;
    Seg s0, s1;
};

enum Prec : int { PREC_F32 = 0, PREC_BF16 = 1 };

NERF_HD constexpr int enc_pairs(int L) { return 3 * L + 2; }
NERF_HD constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
NERF_HD constexpr int out_blocks(int n_out) { return ceil_div(n_out, 32); }

// k-steps (bf16: k-blocks of 16; f32: k-steps of 2) of an input segment
NERF_HD constexpr int seg_steps(Seg s, int prec) {
    return s.kind == SEG_NONE     ? 0
           : s.kind == SEG_HIDDEN ? (prec == PREC_BF16 ? 2 : 16) * out_blocks(s.width)
           : s.kind == SEG_ENC    ? (prec == PREC_BF16 ? ceil_div(enc_pairs(s.L), 8) : 16 * ceil_div(enc_pairs(s.L), 16))
                                  : (prec == PREC_BF16 ? ceil_div(s.width, 16) : ceil_div(s.width, 2));
}

NERF_HD constexpr int layer_steps(Layer l, int prec) { return seg_steps(l.s0, prec) + seg_steps(l.s1, prec); }
NERF_HD constexpr int layer_tiles(Layer l, int prec) { return out_blocks(l.n_out) * layer_steps(l, prec); }
NERF_HD constexpr int tile_bytes(int prec) { return prec == PREC_BF16 ? 1024 : 256; }

// ---------------------------------------------------------------------------
// The four networks
// ---------------------------------------------------------------------------
constexpr Seg H(int w) { return Seg{SEG_HIDDEN, w, 0}; }
constexpr Seg E(int L) { return Seg{SEG_ENC, 3 + 6 * L, L}; }
constexpr Seg F(int w) { return Seg{SEG_FEAT, w, 0}; }
constexpr Seg NONE{SEG_NONE, 0, 0};

// NeRF 8x256, skip after layer index 4 ("4. The NeRF network")
constexpr Layer kNet8x256[] = {
    {256, 1, E(10), NONE}, {256, 1, H(256), NONE}, {256, 1, H(256), NONE}, {256, 1, H(256), NONE},
    {256, 1, H(256), NONE}, {256, 1, H(256), E(10)}, {256, 1, H(256), NONE}, {256, 1, H(256), NONE},
    {1, 0, H(256), NONE},     // density head
    {256, 0, H(256), NONE},   // feature (no activation)
    {128, 1, H(256), E(4)},   // direction layer
    {3, 0, H(128), NONE},     // rgb head
};
constexpr Layer kNet4x64[] = {
    {64, 1, E(6), NONE}, {64, 1, H(64), NONE}, {64, 1, H(64), NONE}, {64, 1, H(64), NONE},
    {1, 0, H(64), NONE}, {64, 0, H(64), NONE}, {32, 1, H(64), E(4)}, {3, 0, H(32), NONE},
};
constexpr Layer kNetCell2x32[] = {
    {32, 1, E(10), NONE}, {32, 1, H(32), NONE}, {1, 0, H(32), NONE},
    {32, 0, H(32), NONE}, {16, 1, H(32), E(4)}, {3, 0, H(16), NONE},
};
constexpr Layer kNetHashField[] = {
    {64, 1, F(32), NONE}, {64, 1, H(64), NONE}, {1, 0, H(64), NONE}, {64, 0, H(64), NONE},
    {64, 1, H(64), F(16)}, {64, 1, H(64), NONE}, {3, 0, H(64), NONE},
};

enum NetKind : int { NET_8x256 = 1, NET_4x64 = 2, NET_CELL_2x32 = 3, NET_HASH_FIELD = 4 };

NERF_HD constexpr const Layer* net_layers(int kind) {
    return kind == NET_8x256 ? kNet8x256 : kind == NET_4x64 ? kNet4x64 : kind == NET_CELL_2x32 ? kNetCell2x32
                                                                                                 : kNetHashField;
}
NERF_HD constexpr int net_n_layers(int kind) {
    return kind == NET_8x256 ? 12 : kind == NET_4x64 ? 8 : kind == NET_CELL_2x32 ? 6 : kind == NET_HASH_FIELD ? 7 : 0;
}

NERF_HD constexpr size_t net_tile_offset(int kind, int prec, int layer) {
    size_t off = 0;
    for (int i = 0; i < layer; ++i) off += (size_t)layer_tiles(net_layers(kind)[i], prec) * tile_bytes(prec);
    return off;
}
NERF_HD constexpr size_t net_tiles_bytes(int kind, int prec) {
    return net_tile_offset(kind, prec, net_n_layers(kind));
}
// The tile region is padded to a whole number of 16 KB chunks (the unit in
// which kernels copy weights into LDS), so chunk copies never run past it.
constexpr size_t kTileRegionAlign = 16384;
NERF_HD constexpr size_t net_tiles_padded(int kind, int prec) {
    return (net_tiles_bytes(kind, prec) + kTileRegionAlign - 1) / kTileRegionAlign * kTileRegionAlign;
}
NERF_HD constexpr size_t net_bias_offset(int kind, int prec, int layer) {
    size_t off = net_tiles_padded(kind, prec);
    for (int i = 0; i < layer; ++i) off += (size_t)out_blocks(net_layers(kind)[i].n_out) * 32 * sizeof(float);
    return off;
}
NERF_HD constexpr size_t net_packed_bytes(int kind, int prec) {
    return net_bias_offset(kind, prec, net_n_layers(kind));
}

// Algorithmic multiply-adds per sample of the network's definition (logical
// widths, no padding).
NERF_HD constexpr long net_macs(int kind) {
    long m = 0;
    for (int i = 0; i < net_n_layers(kind); ++i) {
        const Layer l = net_layers(kind)[i];
        m += (long)l.n_out * (l.s0.width + l.s1.width);
    }
    return m;
}

// ---------------------------------------------------------------------------
// Slot -> logical input column.  Returns -1 for padding.
// ---------------------------------------------------------------------------
NERF_HD constexpr int pair_col(int P, int comp, int L) {
    return P < 3 * L ? 3 + 6 * (P / 3) + 3 * comp + (P % 3) : P == 3 * L ? comp : (P == 3 * L + 1 && comp == 0) ? 2 : -1;
}

// Logical column within segment `s` of k-step `step`, lane half `h`,
// element `j` (bf16: j = 0..7; f32: j = 0).
NERF_HD constexpr int seg_col(Seg s, int prec, int step, int h, int j) {
    if (s.kind == SEG_HIDDEN) {
        int n = 0;
        if (prec == PREC_BF16) {
            n = 32 * (step / 2) + 8 * (2 * (step % 2) + j / 4) + 4 * h + (j % 4);
        } else {
            const int ob = step / 16, r = step % 16;
            n = 32 * ob + 8 * (r / 4) + 4 * h + (r % 4);
        }
        return n < s.width ? n : -1;
    }
    if (s.kind == SEG_ENC) {
        if (prec == PREC_BF16) return pair_col(8 * step + 4 * h + j / 2, j % 2, s.L);
        return pair_col(2 * (step / 2) + h, step % 2, s.L);
    }
    if (s.kind == SEG_FEAT) {
        const int f = prec == PREC_BF16 ? 16 * step + 8 * h + j : 2 * step + h;
        return f < s.width ? f : -1;
    }
    return -1;
}

// Output neuron held in accumulator r by lane half h of output block ob.
NERF_HD constexpr int acc_row(int ob, int h, int r) { return 32 * ob + 8 * (r / 4) + 4 * h + (r % 4); }

}  // namespace nerf

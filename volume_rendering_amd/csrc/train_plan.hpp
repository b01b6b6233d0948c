// Plan and workspace of a training step (host side): per-layer offsets of
// the flat parameter vector, padded activation widths, and the buffers of a
// step.  Shared by the step's launcher and the workspace layout.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "nets.hpp"

namespace nerf {

inline int pad32(int n) { return (n + 31) / 32 * 32; }

// Buffers of a step (ids into TrainBufs::ptr).
enum : int { BZ = 0, BE, BV, BF, BG, BRAW, BDRGB, BDSIG, BDG, BDF, BDH0, BDH1, BSQ, BGRAD, BPART, BBPART, BH0 };

struct NetPlan {
    int D, W, skip, Lpos, Ldir, DW;
    int pe, de, ldE, ldV, ldG;
    // flat offsets of each layer's weights and biases, and its input width
    int64_t w_off[16], b_off[16];
    int in_total[16];
    int64_t P;  // parameters
};

inline NetPlan make_plan(int kind) {
    NetPlan p{};
    const Layer* L = net_layers(kind);
    const int nl = net_n_layers(kind);
    p.D = nl - 4;
    p.W = L[0].n_out;
    p.skip = -1;
    for (int l = 1; l < p.D; ++l)
        if (L[l].s1.kind == SEG_ENC) p.skip = l - 1;
    p.Lpos = L[0].s0.L;
    p.Ldir = L[p.D + 2].s1.L;
    p.DW = L[p.D + 2].n_out;
    p.pe = 3 + 6 * p.Lpos;
    p.de = 3 + 6 * p.Ldir;
    p.ldE = pad32(p.pe);
    p.ldV = pad32(p.de);
    p.ldG = pad32(p.DW);
    int64_t off = 0;
    for (int l = 0; l < nl; ++l) {
        p.in_total[l] = L[l].s0.width + L[l].s1.width;
        p.w_off[l] = off;
        off += (int64_t)L[l].n_out * p.in_total[l];
        p.b_off[l] = off;
        off += L[l].n_out;
    }
    p.P = off;
    return p;
}

struct TrainBufs {
    void* ptr[BH0 + 16];
    int splits, k_chunk;
    // weights: forward matrices, transposed matrices, biases (per layer), the
    // combined feature+density transpose
    void* wf[16];
    void* wt[16];
    float* bias[16];
    void* wt_head;
    // bfloat16 steps: one bit per hidden activation (and per direction-layer
    // output), set where the stored value is > 0: the ReLU masks of the
    // input-gradient products, 1/16 of the activations' bytes
    unsigned char* hbits[16];
    unsigned char* gbits;
};


}  // namespace nerf

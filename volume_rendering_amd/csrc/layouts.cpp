// Workspace layouts of the many-network render and of the training steps:
// host arithmetic only, shared by the launchers and the C ABI's size queries.
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "inr_plan.hpp"
#include "launch.hpp"
#include "nets.hpp"
#include "train_plan.hpp"

namespace nerf {

size_t kilo_workspace_layout(int64_t n_rays, int n_samples, int n_cells, char* base, KiloArgs* k) {
    const uint64_t max_live = (uint64_t)n_rays * (uint64_t)n_samples;
    const uint64_t nb = (uint64_t)((n_rays + kKiloScanBlock - 1) / kKiloScanBlock);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    const int words = (n_samples + 63) / 64;  // 64-bit live masks, one bit per sample
    const size_t o_mask = take(8 * (size_t)n_rays * words);
    const size_t o_live = take(4 * (size_t)n_rays), o_start = take(4 * ((size_t)n_rays + 1)),
                 o_bs = take(4 * (nb + 1)), o_er = take(4 * max_live), o_em = take(4 * max_live),
                 o_cc = take(4 * (size_t)n_cells), o_cs = take(4 * ((size_t)n_cells + 1)),
                 o_sl = take(4 * max_live), o_bk = take(32 * max_live), o_raw = take(16 * max_live);
    if (base && k) {
        k->live_mask = (unsigned long long*)(base + o_mask);
        k->mask_words = words;
        k->live_count = (uint32_t*)(base + o_live);
        k->ray_start = (uint32_t*)(base + o_start);
        k->block_sums = (uint32_t*)(base + o_bs);
        k->ent_ray = (uint32_t*)(base + o_er);
        k->ent_meta = (uint32_t*)(base + o_em);
        k->cell_count = (uint32_t*)(base + o_cc);
        k->cell_start = (uint32_t*)(base + o_cs);
        k->ent_slot = (uint32_t*)(base + o_sl);
        k->bucket = (float*)(base + o_bk);
        k->raw_live = (float*)(base + o_raw);
    }
    return off;
}

// Workspace of one step (bytes), laid out into b when base is given.
size_t train_workspace_layout(int kind, int bf16, int64_t R, int N, char* base, void* bufs_out) {
    const NetPlan p = make_plan(kind);
    const int64_t S = R * N;
    const size_t es = bf16 ? 2 : 4;
    TrainBufs b{};
    size_t off = 0;
    auto take = [&](size_t bytes) -> void* {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? base + at : nullptr;
    };
    // about 128 splits of the samples for the weight gradients (whole
    // multiples of 64, at least 512 samples each), and few enough samples
    // per split that a split of the widest operand spans under 2^31 bytes
    // (the weight-gradient products address a split with 32-bit offsets)
    const int64_t per = ((S + 127) / 128 + 63) / 64 * 64;
    int maxld = p.W;
    for (int ld : {p.ldE, p.ldG, p.ldV}) maxld = ld > maxld ? ld : maxld;
    const int64_t cap = (((int64_t)1 << 31) - 1) / ((int64_t)es * maxld) / 64 * 64;
    b.k_chunk = (int)(per > 512 ? (per < cap ? per : cap) : 512);
    b.splits = (int)((S + b.k_chunk - 1) / b.k_chunk);
    b.ptr[BZ] = take(4 * (size_t)S);
    b.ptr[BE] = take(es * (size_t)S * p.ldE);
    b.ptr[BV] = take(es * (size_t)R * p.ldV);
    for (int l = 0; l < p.D; ++l) b.ptr[BH0 + l] = take(es * (size_t)S * p.W);
    b.ptr[BF] = take(es * (size_t)S * p.W);
    b.ptr[BG] = take(es * (size_t)S * p.ldG);
    b.ptr[BRAW] = take(16 * (size_t)S);
    b.ptr[BDRGB] = take(es * (size_t)S * 32);
    b.ptr[BDSIG] = take(es * (size_t)S * 32);
    b.ptr[BDG] = take(es * (size_t)S * p.ldG);
    b.ptr[BDF] = take(es * (size_t)S * p.W);
    b.ptr[BDH0] = take(es * (size_t)S * p.W);
    b.ptr[BDH1] = take(es * (size_t)S * p.W);
    b.ptr[BSQ] = take(4 * (size_t)R);
    b.ptr[BGRAD] = take(4 * (size_t)p.P);
    const int maxk = p.ldE > p.W ? p.ldE : p.W;
    b.ptr[BPART] = take(4 * (size_t)b.splits * pad32(p.W + 32) * pad32(maxk + 32));
    b.ptr[BBPART] = take(4 * (size_t)b.splits * pad32(p.W + 32));
    const int nl = p.D + 4;
    const Layer* L = net_layers(kind);
    for (int l = 0; l < nl; ++l) {
        const int no = pad32(L[l].n_out);
        const int k1 = L[l].s0.kind == SEG_HIDDEN ? pad32(L[l].s0.width) : p.ldE;
        const int k2 = L[l].s1.kind == SEG_NONE ? 0 : (l == p.D + 2 ? p.ldV : p.ldE);
        b.wf[l] = take(es * (size_t)no * (k1 + k2));
        b.wt[l] = take(es * (size_t)k1 * no);
        b.bias[l] = (float*)take(4 * (size_t)no);
    }
    b.wt_head = take(es * (size_t)p.W * (p.W + 32));
    if (bf16) {
        for (int l = 0; l < p.D; ++l) b.hbits[l] = (unsigned char*)take((size_t)S * p.W / 8);
        b.gbits = (unsigned char*)take((size_t)S * p.ldG / 8);
    }
    if (bufs_out) *static_cast<TrainBufs*>(bufs_out) = b;
    return off;
}

int64_t train_param_count(int kind) { return make_plan(kind).P; }

int64_t hash_inr_param_count(const GridArgs& g, int hidden, int n_out) {
    return inr_table_floats(g) + inr_decoder_params(g, hidden, n_out);
}

size_t hash_inr_workspace_layout(const GridArgs& g, int hidden, int n_out, int64_t n, char* base, void* out) {
    size_t off = 0;
    auto take = [&](size_t bytes) -> float* {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? reinterpret_cast<float*>(base + at) : nullptr;
    };
    const InrShape sh = inr_shape(g, hidden, n_out, n);
    InrWs w{};
    w.dfeat = take(4 * (size_t)sh.dstride * 2 * g.n_levels);
    w.part_dec = take(4 * (size_t)sh.groups * (size_t)sh.part_w);
    w.part_tab = take(4 * (size_t)sh.scat_chunks * (size_t)sh.lds_tab_floats);
    w.grad = take(4 * (size_t)hash_inr_param_count(g, hidden, n_out));
    w.wpad = take(4 * (size_t)sh.weight_floats);
    if (out) *static_cast<InrWs*>(out) = w;
    return off;
}

}  // namespace nerf

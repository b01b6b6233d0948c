// Host helpers of the C ABI: hash-grid level layout and weight packing.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "abi_util.hpp"
#include "nerf_mi355x.h"
#include "nets.hpp"

using namespace nerf;

namespace {

uint16_t bf16_bits_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

bool supported_kind(int kind) {
    return kind == NET_8x256 || kind == NET_4x64 || kind == NET_CELL_2x32 || kind == NET_HASH_FIELD;
}

}  // namespace

extern "C" {

nerf_status nerf_hashgrid_init(nerf_hashgrid* g, int dim, int n_levels, uint32_t table_size, int n_min, int n_max) {
    if (!g) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_hashgrid_init: g is NULL");
    if (dim != 2 && dim != 3) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_hashgrid_init: dim %d", dim);
    if (n_levels < 2 || n_levels > NERF_HASH_MAX_LEVELS)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_hashgrid_init: n_levels %d outside 2..16", n_levels);
    if (table_size == 0 || (table_size & (table_size - 1)))
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_hashgrid_init: table size %u is not a power of two",
                         table_size);
    if (n_min < 1 || n_max < n_min)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_hashgrid_init: bad resolutions %d..%d", n_min, n_max);
    std::memset(g, 0, sizeof(*g));
    g->dim = dim;
    for (int l = 0; l < NERF_HASH_MAX_LEVELS; ++l) g->level_mask[l] = 1.0f;
    g->n_levels = n_levels;
    g->n_feat = 2;
    g->table_size = table_size;
    // N_l = round(N_min * b^l), b = exp((ln N_max - ln N_min)/(L-1)), ties to even
    const double b = std::exp((std::log((double)n_max) - std::log((double)n_min)) / (double)(n_levels - 1));
    uint64_t off = 0;
    for (int l = 0; l < n_levels; ++l) {
        const int N = (int)std::nearbyint((double)n_min * std::pow(b, (double)l));
        const uint64_t verts = (uint64_t)(N + 1) * (uint64_t)(N + 1) * (dim == 3 ? (uint64_t)(N + 1) : 1u);
        g->res[l] = N;
        g->direct[l] = verts <= table_size ? 1 : 0;
        g->size[l] = (uint32_t)(verts <= table_size ? verts : table_size);
        g->offset[l] = off;
        off += g->size[l];
    }
    g->total_entries = off;
    g->tables = nullptr;
    return NERF_OK;
}

size_t nerf_mlp_packed_bytes(const nerf_mlp_desc* net) {
    if (!net || !supported_kind(net->kind) || (net->dtype != NERF_F32 && net->dtype != NERF_BF16)) return 0;
    return net_packed_bytes(net->kind, net->dtype == NERF_BF16 ? PREC_BF16 : PREC_F32);
}

nerf_status nerf_pack_mlp(const nerf_mlp_desc* net, const float* const* tensors, int n_tensors, void* dst,
                          size_t dst_bytes) {
    if (!net || !tensors || !dst) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_pack_mlp: NULL argument");
    if (!supported_kind(net->kind)) return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_pack_mlp: kind %d", net->kind);
    if (net->dtype != NERF_F32 && net->dtype != NERF_BF16)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_pack_mlp: dtype %d", net->dtype);
    const int kind = net->kind;
    const int prec = net->dtype == NERF_BF16 ? PREC_BF16 : PREC_F32;
    const int nl = net_n_layers(kind);
    if (n_tensors != 2 * nl)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_pack_mlp: expected %d tensors, got %d", 2 * nl, n_tensors);
    for (int i = 0; i < n_tensors; ++i)
        if (!tensors[i]) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_pack_mlp: tensor %d is NULL", i);
    const size_t need = net_packed_bytes(kind, prec);
    if (dst_bytes < need)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_pack_mlp: dst has %zu bytes, needs %zu", dst_bytes, need);
    char* out = static_cast<char*>(dst);
    std::memset(out, 0, need);
    for (int li = 0; li < nl; ++li) {
        const Layer L = net_layers(kind)[li];
        const float* W = tensors[2 * li];
        const float* bias = tensors[2 * li + 1];
        const int in_total = L.s0.width + L.s1.width;
        const int S1 = seg_steps(L.s0, prec), S2 = seg_steps(L.s1, prec);
        const int OB = out_blocks(L.n_out);
        char* tiles = out + net_tile_offset(kind, prec, li);
        size_t t = 0;
        for (int ob = 0; ob < OB; ++ob)
            for (int st = 0; st < S1 + S2; ++st, ++t) {
                const Seg seg = st < S1 ? L.s0 : L.s1;
                const int sst = st < S1 ? st : st - S1;
                const int cbase = st < S1 ? 0 : L.s0.width;
                for (int lane = 0; lane < 64; ++lane) {
                    const int row = 32 * ob + (lane % 32), h = lane / 32;
                    if (prec == PREC_BF16) {
                        uint16_t* dstp = reinterpret_cast<uint16_t*>(tiles + t * 1024 + lane * 16);
                        for (int j = 0; j < 8; ++j) {
                            const int c = seg_col(seg, prec, sst, h, j);
                            const float v = (row < L.n_out && c >= 0) ? W[(size_t)row * in_total + cbase + c] : 0.0f;
                            dstp[j] = bf16_bits_rne(v);
                        }
                    } else {
                        float* dstp = reinterpret_cast<float*>(tiles + t * 256 + lane * 4);
                        const int c = seg_col(seg, prec, sst, h, 0);
                        *dstp = (row < L.n_out && c >= 0) ? W[(size_t)row * in_total + cbase + c] : 0.0f;
                    }
                }
            }
        float* bdst = reinterpret_cast<float*>(out + net_bias_offset(kind, prec, li));
        for (int ob = 0; ob < OB; ++ob)
            for (int h = 0; h < 2; ++h)
                for (int r = 0; r < 16; ++r) {
                    const int row = acc_row(ob, h, r);
                    bdst[(ob * 2 + h) * 16 + r] = row < L.n_out ? bias[row] : 0.0f;
                }
    }
    return NERF_OK;
}

}  // extern "C"

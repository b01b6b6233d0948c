// Sizes, launch shape and workspace of a hash-grid INR training step (host
// side), shared by the step's launcher and the workspace layout.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "launch.hpp"

namespace nerf {

constexpr int kInrMaxLevels = 16;
constexpr int kInrMaxHidden = 64;
constexpr int kInrMaxOut = 4;
constexpr int64_t kInrMaxPoints = (int64_t)1 << 27;  // points per step
constexpr int kInrThreads = 256;                     // threads per workgroup
constexpr int kInrWaves = kInrThreads / 64;
constexpr int kInrStageRows = 16;                    // points per staging round of a wave
constexpr int kInrDecodeGroups = 1024;               // decoder workgroups (at most, before points per thread grow)
constexpr int kInrScatEntries = 4096;                // table entries per scatter workgroup (64 KB of 64-bit sums)
constexpr int kInrMaxRanges = 8;                     // ranges per level before a level scatters by global atomics
constexpr int kInrScatGroups = 2048;                 // scatter workgroups aimed at
constexpr int64_t kInrMaxChunk = (int64_t)1 << 17;   // points per scatter chunk (fixed-point headroom)

// Floats of the tables: 2 per entry over all levels.
inline int64_t inr_table_floats(const GridArgs& g) {
    return 2 * (int64_t)(g.offset[g.n_levels - 1] + g.size[g.n_levels - 1]);
}

inline int inr_decoder_params(const GridArgs& g, int hidden, int n_out) {
    return hidden * 2 * g.n_levels + hidden + n_out * hidden + n_out;
}

// Floats per staged point of the decoder kernel: dpre | h | feat | 16, padded
// to 20 mod 32 (LDS banks).
constexpr int inr_stage_width(int hm, int fm) {
    return (2 * hm + fm + 16) + ((20 - (2 * hm + fm + 16) % 32) + 32) % 32;
}

// Launch shape of one step.  The decoder is padded to hm hidden units and fm
// features (multiples of 16, the MFMA tile).  The table gradients of the
// first lds_levels levels (sizes grow with the level: a prefix) are
// scattered through LDS in ranges of kInrScatEntries entries; larger levels
// by global atomics.
struct InrShape {
    int hm, fm;               // padded hidden width (32, 64) and feature width (16, 32)
    int stage_w;              // floats per staged point: dpre | h | feat | dy (16), padded
    int weight_floats;        // padded decoder: hm rows of fm + 8 (W1 row, b1, W2 column, 0s), b2 [8], W1^T, W2
    int pm;                   // decoder parameters
    int part_w;               // floats per decoder partial: decoder gradient, then the squared-error sum
    int groups;               // decoder workgroups
    int iters;                // points per decoder thread
    size_t lds_bytes;         // decoder LDS per workgroup
    int lds_levels;           // levels scattered through LDS
    int64_t lds_tab_floats;   // their table floats
    int64_t tab_floats;       // all table floats
    int scat_jobs;            // (level, range) pairs, plus one per global-atomic level
    int64_t scat_chunk;       // points per scatter chunk: a multiple of 4 points per thread
    int scat_chunks;
    int64_t dstride;          // points per level slice of the feature gradients (even)
};

inline InrShape inr_shape(const GridArgs& g, int hidden, int n_out, int64_t n) {
    InrShape s{};
    s.hm = hidden <= 32 ? 32 : 64;
    s.fm = 2 * g.n_levels <= 16 ? 16 : 32;
    s.stage_w = inr_stage_width(s.hm, s.fm);
    s.weight_floats = s.hm * (s.fm + 8) + 8 + s.fm * s.hm + 4 * s.hm;
    s.tab_floats = inr_table_floats(g);
    s.pm = inr_decoder_params(g, hidden, n_out);
    s.part_w = (s.pm + 1 + 3) / 4 * 4;
    const int64_t tiles = (n + kInrThreads - 1) / kInrThreads;
    s.iters = (int)((tiles + kInrDecodeGroups - 1) / kInrDecodeGroups);
    if (s.iters < 1) s.iters = 1;
    s.groups = (int)((tiles + s.iters - 1) / s.iters);
    if (s.groups < 1) s.groups = 1;
    s.lds_bytes = 4 * (size_t)kInrWaves * kInrStageRows * s.stage_w;
    int k = 0;
    int64_t ltf = 0;
    int jobs = 0;
    while (k < g.n_levels && (g.size[k] + kInrScatEntries - 1) / kInrScatEntries <= kInrMaxRanges) {
        jobs += (g.size[k] + kInrScatEntries - 1) / kInrScatEntries;
        ltf += 2 * (int64_t)g.size[k];
        ++k;
    }
    s.lds_levels = k;
    s.lds_tab_floats = ltf;
    s.scat_jobs = jobs + (g.n_levels - k);
    int64_t chunk = (n * s.scat_jobs + kInrScatGroups - 1) / kInrScatGroups;
    chunk = (chunk + 4 * kInrThreads - 1) / (4 * kInrThreads) * (4 * kInrThreads);
    if (chunk < 4 * kInrThreads) chunk = 4 * kInrThreads;
    if (chunk > kInrMaxChunk) chunk = kInrMaxChunk;
    s.scat_chunk = chunk;
    s.scat_chunks = (int)((n + chunk - 1) / chunk);
    if (s.scat_chunks < 1) s.scat_chunks = 1;
    s.dstride = (n + 1) / 2 * 2;
    return s;
}

struct InrWs {
    float* dfeat;     // [levels][dstride][2]: feature gradients
    float* part_dec;  // [groups][part_w]: decoder-gradient and loss partials
    float* part_tab;  // [scat_chunks][lds_tab_floats]: table-gradient partials of the LDS levels
    float* grad;      // [parameters] when the caller gives none
    float* wpad;      // [weight_floats]: the padded decoder
};

}  // namespace nerf

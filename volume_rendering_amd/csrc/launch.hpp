// Host-side launchers of the gfx950 kernels and the plain argument structs
// they take.  Shapes and pointers are validated by the C ABI layer before
// any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nerf {

struct GridArgs {
    int n_levels;
    int dim;         // 2 or 3
    float mask[16];  // per-level multiplier; 0: level not looked up
    uint32_t tmask;  // T - 1 (T a power of two)
    int res[16];
    int direct[16];
    uint32_t size[16];  // entries of each level
    uint64_t offset[16];
    const void* tables;  // float16 pairs, levels back to back
    int bytes;           // bytes readable from tables: entries rounded up to whole 8-byte words
};

struct RenderArgs {
    const float* ro;
    const float* rd;
    const float* tn;
    const float* tf;
    int64_t n_rays;
    const void* coarse;
    const void* fine;
    int n_coarse, n_fine;
    int use_pi, white, jitter;
    uint64_t seed, ray_offset;
    float box_lo, box_hi;
    float* rgb;
    float* depth;
    float* acc;
    float* dbg_z;
    float* dbg_w;
    // empty-space skipping and early termination (NeRF and hash modes)
    const uint32_t* occ;  // occupancy bitset over the box, or NULL (every sample live)
    int occ_res;
    float vscale;         // occ_res / (hi - lo), rounded to float32 once
    float term_T;         // drop sample i and later once T_i < term_T (0: never)
    int64_t* n_live;      // optional: live samples evaluated, added
};

// Many-tiny-networks render: scene box, occupancy grid, cell networks and
// the device workspace carved by the ABI layer.
struct KiloArgs {
    float lo, hi;       // scene box
    float vscale;       // occ_res / (hi - lo), rounded to float32 once
    float cscale;       // cell_res / (hi - lo), rounded to float32 once
    int occ_res, cell_res;
    float term_T;
    const uint32_t* occ;
    const void* cells;  // packed cell networks back to back
    size_t cell_stride; // bytes per packed network
    int64_t* dbg_n_live;
    // workspace
    unsigned long long* live_mask;  // [n_rays, mask_words]: bit i of word w = sample 64w+i live
    int mask_words;
    uint32_t* live_count;  // [n_rays]
    uint32_t* ray_start;   // [n_rays + 1]
    uint32_t* block_sums;  // [scan blocks + 1]
    uint32_t* ent_ray;     // [max_live]
    uint32_t* ent_meta;    // [max_live]: sample << 16 | cell
    uint32_t* ent_slot;    // [max_live]: place in the cell's bucket
    uint32_t* cell_count;  // [n_cells]
    uint32_t* cell_start;  // [n_cells + 1]
    float* bucket;         // [max_live][8]: per bucket slot, the sample's point, its entry index
                           // (bits of a float) and its unit view direction
    float* raw_live;       // [max_live, 4]
};

// One training step of a NeRF-family network (frequency encodings): samples,
// network, compositing, mean squared error, gradients, Adam.
struct TrainArgs {
    const float* ro;
    const float* rd;
    const float* tn;
    const float* tf;
    const float* target;  // [n_rays, 3]
    int64_t n_rays;
    int n_samples;
    int use_pi, white, jitter;
    uint64_t seed, ray_offset;
    float* params;  // flat float32 weights and biases, updated in place by Adam
    float* adam_m;  // NULL: no Adam step
    float* adam_v;
    float* grad;    // flat gradient out, or NULL (kept in the workspace)
    int64_t step;   // Adam step t >= 1
    float lr, beta1, beta2, eps;
    float* loss;     // [1]
    float* rgb_out;  // [n_rays, 3] or NULL
    const float* z_in;  // [n_rays, n_samples] sample depths, or NULL (stratified)
    float* w_out;       // [n_rays, n_samples] compositing weights, or NULL
    void* workspace;
};

size_t train_workspace_layout(int kind, int bf16, int64_t n_rays, int n_samples, char* base, void* bufs_out);
int64_t train_param_count(int kind);
void launch_train_step(int kind, int bf16, const TrainArgs& t, hipStream_t s);

// One training step of the hash-grid INR (learnable float32 tables and a
// decoder with one hidden ReLU layer).
struct HashInrArgs {
    const float* x;       // [n, dim] points in [0,1]^dim
    const float* target;  // [n, n_out]
    int64_t n;
    int hidden, n_out;
    float* params;  // flat: tables (2 floats per entry, levels back to back), W1, b1, W2, b2
    float* adam_m;  // NULL: no Adam step
    float* adam_v;
    float* grad;  // flat gradient out, or NULL (kept in the workspace)
    int64_t step;
    float lr, beta1, beta2, eps;
    float* loss;  // [1]
    float* pred;  // [n, n_out] or NULL
    void* workspace;
};

int64_t hash_inr_param_count(const GridArgs& g, int hidden, int n_out);
size_t hash_inr_workspace_layout(const GridArgs& g, int hidden, int n_out, int64_t n, char* base, void* out);
void launch_hash_inr_step(const GridArgs& g, const HashInrArgs& a, hipStream_t s);

// Rays per local-scan block of the many-network render's prefix sums (256 threads x 4).
constexpr int kKiloScanBlock = 1024;

// Workspace layout of the many-tiny-networks render for n_rays x n_samples.
size_t kilo_workspace_layout(int64_t n_rays, int n_samples, int n_cells, char* base, KiloArgs* k);

void launch_render_kilo(int bf16, const RenderArgs& a, const KiloArgs& k, int add_n_live, hipStream_t s);

void launch_gen_rays(const float* pose, int W, int H, float fx, float fy, float cx, float cy, float* ro, float* rd,
                     hipStream_t s);
void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
void launch_stratified(const float* tn, const float* tf, int64_t n_rays, int n, uint64_t seed, uint64_t ray_offset,
                       int jitter, float* z, hipStream_t s);
void launch_encode_freq(const float* x, int64_t n, int d, int L, int inc, int use_pi, int bf16, void* out,
                        hipStream_t s);
void launch_sh16(const float* dirs, int64_t n, float* out, hipStream_t s);
void launch_encode_hash(const float* x, int64_t n, const GridArgs& g, float* out, uint32_t* idx, hipStream_t s);
void launch_composite(const float* raw, const float* z, const float* rd, int64_t n_rays, int n, int white, float* rgb,
                      float* depth, float* acc, float* w, hipStream_t s);
void launch_sample_pdf(const float* zc, const float* wc, int64_t n_rays, int nc, int nf, uint64_t seed,
                       uint64_t ray_offset, float* zf, int32_t* bins, float* z2, hipStream_t s);
void launch_render_nerf(int kind, int bf16, const RenderArgs& a, hipStream_t s);
void launch_render_nerf_bf16(int kind, const RenderArgs& a, hipStream_t s);
void launch_render_nerf_f32(int kind, const RenderArgs& a, hipStream_t s);
void launch_mlp_bf16(int kind, const void* packed, const float* ex, const float* ev, int64_t n, int spr, float* raw,
                     hipStream_t s);
void launch_mlp_f32(int kind, const void* packed, const float* ex, const float* ev, int64_t n, int spr, float* raw,
                    hipStream_t s);
void launch_render_hash(int bf16, const RenderArgs& a, const GridArgs& g, hipStream_t s);

}  // namespace nerf

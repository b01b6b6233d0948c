// C ABI of libnerf_mi355x.so: argument validation, error reporting and
// dispatch to the gfx950 launchers.  Nothing is enqueued unless every
// argument checks out.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include <vector>

#include "abi_util.hpp"
#include "launch.hpp"
#include "nerf_mi355x.h"
#include "nets.hpp"

using namespace nerf;

namespace nerf {
// Readers of the index-check words of every translation unit of a checked
// build, registered while the library loads (none without NERF_CHECK).
std::vector<unsigned (*)()>& check_readers() {
    static std::vector<unsigned (*)()> readers;
    return readers;
}
int check_register(unsigned (*take)()) {
    check_readers().push_back(take);
    return 0;
}
}  // namespace nerf

namespace {

thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Clears an unrelated pending error, so the check after a launch reports
// only this call's failure.
void clear_pending() { (void)hipGetLastError(); }

nerf_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return nerf_fail(NERF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return NERF_OK;
}

#define NERF_REQUIRE(cond, ...)                                  \
    do {                                                         \
        if (!(cond)) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
    } while (0)

bool net_is_nerf_family(int kind) { return kind == NET_8x256 || kind == NET_4x64 || kind == NET_CELL_2x32; }

GridArgs grid_args(const nerf_hashgrid* g) {
    GridArgs a{};
    a.n_levels = g->n_levels;
    a.dim = g->dim;
    a.tmask = g->table_size - 1;
    for (int l = 0; l < g->n_levels; ++l) {
        const uint64_t n1 = (uint64_t)g->res[l] + 1;
        a.res[l] = g->res[l];
        a.direct[l] = g->direct[l];
        a.size[l] = g->direct[l] ? (uint32_t)(n1 * n1 * (g->dim == 3 ? n1 : 1u)) : g->table_size;
        a.offset[l] = g->offset[l];
        a.mask[l] = g->level_mask[l];
    }
    a.tables = g->tables;
    a.bytes = (int)((g->total_entries + 1) / 2 * 8);
    return a;
}

nerf_status check_grid_layout(const nerf_hashgrid* g, const char* who);

nerf_status check_grid(const nerf_hashgrid* g, const char* who) {
    if (!g) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: grid is NULL", who);
    if (!g->tables) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: grid tables are NULL", who);
    if ((reinterpret_cast<uintptr_t>(g->tables) & 7u) != 0)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: tables not 8-byte aligned", who);
    return check_grid_layout(g, who);
}

// The grid's levels, resolutions and table layout (not its tables).
nerf_status check_grid_layout(const nerf_hashgrid* g, const char* who) {
    if (!g) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: grid is NULL", who);
    if (g->n_levels < 1 || g->n_levels > NERF_HASH_MAX_LEVELS || g->n_feat != 2)
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: grid not initialised (levels %d, features %d)", who,
                         g->n_levels, g->n_feat);
    if (g->table_size == 0 || (g->table_size & (g->table_size - 1)))
        return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: table size %u not a power of two", who, g->table_size);
    if (g->dim != 2 && g->dim != 3) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: grid dim %d", who, g->dim);
    for (int l = 0; l < g->n_levels; ++l) {
        const int N = g->res[l];
        if (N < 1 || N > 65535) return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: level %d resolution %d", who, l, N);
        const uint64_t verts = (uint64_t)(N + 1) * (N + 1) * (g->dim == 3 ? (uint64_t)(N + 1) : 1u);
        const uint64_t need = g->direct[l] ? verts : g->table_size;
        if (g->direct[l] && verts > g->table_size)
            return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: level %d marked direct but has %llu vertices", who, l,
                             (unsigned long long)verts);
        if (g->offset[l] + need > g->total_entries)
            return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "%s: level %d overruns the tables", who, l);
    }
    if (g->total_entries > ((uint64_t)1 << 28))
        return nerf_fail(NERF_ERR_UNSUPPORTED, "%s: %llu table entries (at most 2^28)", who,
                         (unsigned long long)g->total_entries);
    return NERF_OK;
}

// Rays per launch of the many-network mode: the caller's chunk, capped so
// that every per-chunk sample index fits 32 bits.
int64_t kilo_chunk(const nerf_render_cfg* cfg, int64_t n_rays) {
    int64_t c = cfg->chunk > 0 ? cfg->chunk : n_rays;
    const int64_t cap = ((int64_t)1 << 31) / (cfg->n_coarse > 0 ? cfg->n_coarse : 1);
    if (c > cap) c = cap;
    return c < n_rays ? c : n_rays;
}

}  // namespace

nerf_status nerf_fail(nerf_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

extern "C" {

int nerf_abi_version(void) { return NERF_ABI_VERSION; }

int64_t nerf_check_flags(void) {
#ifdef NERF_CHECK
    if (hipDeviceSynchronize() != hipSuccess) return (int64_t)0xFFFFFFFFu;
    unsigned v = 0u;
    for (unsigned (*take)() : nerf::check_readers()) v |= take();
    return (int64_t)v;
#else
    return -1;
#endif
}

const char* nerf_status_str(nerf_status s) {
    switch (s) {
        case NERF_OK:
            return "NERF_OK";
        case NERF_ERR_INVALID_ARGUMENT:
            return "NERF_ERR_INVALID_ARGUMENT";
        case NERF_ERR_UNSUPPORTED:
            return "NERF_ERR_UNSUPPORTED";
        case NERF_ERR_WORKSPACE:
            return "NERF_ERR_WORKSPACE";
        case NERF_ERR_HIP:
            return "NERF_ERR_HIP";
    }
    return "NERF_ERR_UNKNOWN";
}

const char* nerf_last_error(void) { return g_last_error.c_str(); }

nerf_status nerf_gen_rays(const float* pose, const nerf_intrinsics* K, float* rays_o, float* rays_d, void* stream) {
    NERF_REQUIRE(pose && K && rays_o && rays_d, "nerf_gen_rays: NULL argument");
    NERF_REQUIRE(K->W >= 1 && K->H >= 1, "nerf_gen_rays: image %dx%d", K->W, K->H);
    NERF_REQUIRE((int64_t)K->W * K->H <= (int64_t)1 << 31, "nerf_gen_rays: image too large");
    NERF_REQUIRE(K->fx != 0.0f && K->fy != 0.0f, "nerf_gen_rays: zero focal length");
    NERF_REQUIRE(aligned4(rays_o) && aligned4(rays_d), "nerf_gen_rays: misaligned output");
    clear_pending();
    launch_gen_rays(pose, K->W, K->H, K->fx, K->fy, K->cx, K->cy, rays_o, rays_d, as_stream(stream));
    return check_launch("nerf_gen_rays");
}

nerf_status nerf_sample_stratified(const float* t_near, const float* t_far, int64_t n_rays, int n, uint64_t seed,
                                   uint64_t ray_offset, int jitter, float* z, void* stream) {
    NERF_REQUIRE(n_rays >= 0, "nerf_sample_stratified: n_rays %lld", (long long)n_rays);
    NERF_REQUIRE(n >= 1 && n <= 256, "nerf_sample_stratified: %d samples outside 1..256", n);
    if (n_rays == 0) return NERF_OK;
    NERF_REQUIRE(t_near && t_far && z, "nerf_sample_stratified: NULL argument");
    clear_pending();
    launch_stratified(t_near, t_far, n_rays, n, seed, ray_offset, jitter, z, as_stream(stream));
    return check_launch("nerf_sample_stratified");
}

nerf_status nerf_encode_freq(const float* x, int64_t n, int in_dim, int n_freq, int include_input, int use_pi,
                             int out_dtype, void* out, void* stream) {
    NERF_REQUIRE(n >= 0, "nerf_encode_freq: n %lld", (long long)n);
    NERF_REQUIRE(in_dim >= 1 && in_dim <= 4, "nerf_encode_freq: in_dim %d outside 1..4", in_dim);
    NERF_REQUIRE(n_freq >= 0 && n_freq <= 16, "nerf_encode_freq: n_freq %d outside 0..16", n_freq);
    NERF_REQUIRE(out_dtype == NERF_F32 || out_dtype == NERF_BF16, "nerf_encode_freq: dtype %d", out_dtype);
    NERF_REQUIRE(include_input || n_freq > 0, "nerf_encode_freq: empty encoding");
    if (n == 0) return NERF_OK;
    NERF_REQUIRE(x && out, "nerf_encode_freq: NULL argument");
    clear_pending();
    launch_encode_freq(x, n, in_dim, n_freq, include_input ? 1 : 0, use_pi ? 1 : 0, out_dtype == NERF_BF16, out,
                       as_stream(stream));
    return check_launch("nerf_encode_freq");
}

nerf_status nerf_encode_sh16(const float* dirs, int64_t n, float* out, void* stream) {
    NERF_REQUIRE(n >= 0, "nerf_encode_sh16: n %lld", (long long)n);
    if (n == 0) return NERF_OK;
    NERF_REQUIRE(dirs && out, "nerf_encode_sh16: NULL argument");
    clear_pending();
    launch_sh16(dirs, n, out, as_stream(stream));
    return check_launch("nerf_encode_sh16");
}

nerf_status nerf_encode_hashgrid(const float* x, int64_t n, const nerf_hashgrid* g, float* out, uint32_t* idx_dbg,
                                 void* stream) {
    NERF_REQUIRE(n >= 0, "nerf_encode_hashgrid: n %lld", (long long)n);
    const nerf_status gs = check_grid(g, "nerf_encode_hashgrid");
    if (gs != NERF_OK) return gs;
    if (n == 0) return NERF_OK;
    NERF_REQUIRE(x && out, "nerf_encode_hashgrid: NULL argument");
    NERF_REQUIRE(aligned16(out) || ((reinterpret_cast<uintptr_t>(out) & 7u) == 0),
                 "nerf_encode_hashgrid: out not 8-byte aligned");
    clear_pending();
    const GridArgs a = grid_args(g);
    launch_encode_hash(x, n, a, out, idx_dbg, as_stream(stream));
    return check_launch("nerf_encode_hashgrid");
}

nerf_status nerf_mlp(const nerf_mlp_desc* net, const void* packed, const float* enc_x, const float* enc_v, int64_t n,
                     int samples_per_ray, float* raw, void* stream) {
    NERF_REQUIRE(net, "nerf_mlp: net is NULL");
    if (nerf_mlp_packed_bytes(net) == 0)
        return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_mlp: unsupported network kind %d / dtype %d", net->kind,
                         net->dtype);
    NERF_REQUIRE(n >= 0, "nerf_mlp: n %lld", (long long)n);
    NERF_REQUIRE(samples_per_ray >= 1, "nerf_mlp: samples_per_ray %d", samples_per_ray);
    if (n == 0) return NERF_OK;
    NERF_REQUIRE(packed && enc_x && enc_v && raw, "nerf_mlp: NULL argument");
    NERF_REQUIRE(aligned16(packed) && aligned16(raw), "nerf_mlp: packed weights and raw must be 16-byte aligned");
    clear_pending();
    if (net->dtype == NERF_BF16)
        launch_mlp_bf16(net->kind, packed, enc_x, enc_v, n, samples_per_ray, raw, as_stream(stream));
    else
        launch_mlp_f32(net->kind, packed, enc_x, enc_v, n, samples_per_ray, raw, as_stream(stream));
    return check_launch("nerf_mlp");
}

nerf_status nerf_composite(const float* raw, const float* z, const float* rays_d, int64_t n_rays, int n,
                           int white_bkgd, float* rgb, float* depth, float* acc, float* weights, void* stream) {
    NERF_REQUIRE(n_rays >= 0, "nerf_composite: n_rays %lld", (long long)n_rays);
    NERF_REQUIRE(n >= 1 && n <= 4096, "nerf_composite: %d samples outside 1..4096", n);
    if (n_rays == 0) return NERF_OK;
    NERF_REQUIRE(raw && z && rays_d && rgb && depth && acc, "nerf_composite: NULL argument");
    NERF_REQUIRE(aligned16(raw), "nerf_composite: raw must be 16-byte aligned");
    clear_pending();
    launch_composite(raw, z, rays_d, n_rays, n, white_bkgd ? 1 : 0, rgb, depth, acc, weights, as_stream(stream));
    return check_launch("nerf_composite");
}

nerf_status nerf_sample_pdf(const float* z_coarse, const float* w_coarse, int64_t n_rays, int n_coarse, int n_fine,
                            uint64_t seed, uint64_t ray_offset, float* z_fine, int32_t* bin_idx, float* z_merged,
                            void* stream) {
    NERF_REQUIRE(n_rays >= 0, "nerf_sample_pdf: n_rays %lld", (long long)n_rays);
    NERF_REQUIRE(n_coarse >= 3, "nerf_sample_pdf: n_coarse %d < 3", n_coarse);
    NERF_REQUIRE(n_fine >= 1, "nerf_sample_pdf: n_fine %d < 1", n_fine);
    NERF_REQUIRE(n_coarse + n_fine <= 256, "nerf_sample_pdf: n_coarse + n_fine = %d > 256", n_coarse + n_fine);
    if (n_rays == 0) return NERF_OK;
    NERF_REQUIRE(z_coarse && w_coarse, "nerf_sample_pdf: NULL input");
    clear_pending();
    launch_sample_pdf(z_coarse, w_coarse, n_rays, n_coarse, n_fine, seed, ray_offset, z_fine, bin_idx, z_merged,
                      as_stream(stream));
    return check_launch("nerf_sample_pdf");
}

size_t nerf_render_workspace_size(const nerf_render_cfg* cfg, int64_t n_rays) {
    if (!cfg || cfg->mode != NERF_MODE_KILO || n_rays <= 0 || cfg->n_coarse < 1 || cfg->cell_res < 1) return 0;
    const int64_t chunk = kilo_chunk(cfg, n_rays);
    const int n_cells = cfg->cell_res * cfg->cell_res * cfg->cell_res;
    return kilo_workspace_layout(chunk, cfg->n_coarse, n_cells, nullptr, nullptr);
}

nerf_status nerf_render(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                        int64_t n_rays, const nerf_weights* w, const nerf_render_cfg* cfg, float* rgb, float* depth,
                        float* acc, void* stream) {
    return nerf::render_entry(rays_o, rays_d, t_near, t_far, n_rays, w, cfg, rgb, depth, acc, stream, nullptr, 0);
}

nerf_status nerf_render_poses(const float* poses, int n_poses, const nerf_intrinsics* K, float t_near, float t_far,
                              const nerf_weights* w, const nerf_render_cfg* cfg, void* workspace,
                              size_t workspace_bytes, float* rgb, float* depth, float* acc, void* stream) {
    NERF_REQUIRE(n_poses >= 0, "nerf_render_poses: n_poses %d", n_poses);
    NERF_REQUIRE(K && w && cfg, "nerf_render_poses: NULL camera, weights or cfg");
    NERF_REQUIRE(K->W >= 1 && K->H >= 1 && (int64_t)K->W * K->H <= (int64_t)1 << 31,
                 "nerf_render_poses: image %dx%d", K->W, K->H);
    NERF_REQUIRE(K->fx != 0.0f && K->fy != 0.0f, "nerf_render_poses: zero focal length");
    NERF_REQUIRE(!cfg->dbg_z && !cfg->dbg_w_coarse && !cfg->dbg_n_live,
                 "nerf_render_poses: debug outputs are per render; use nerf_render");
    if (n_poses == 0) return NERF_OK;
    NERF_REQUIRE(poses && rgb && depth && acc, "nerf_render_poses: NULL poses or output");
    const int64_t R = (int64_t)K->W * K->H;
    const size_t need = (size_t)32 * R;  // rays_o, rays_d, t_near, t_far of one frame
    char* ws = static_cast<char*>(workspace);
    void* own = nullptr;
    if (ws) {
        if (workspace_bytes < need)
            return nerf_fail(NERF_ERR_WORKSPACE, "nerf_render_poses: workspace has %zu bytes, needs %zu",
                             workspace_bytes, need);
        NERF_REQUIRE(aligned16(ws), "nerf_render_poses: workspace must be 16-byte aligned");
    } else {
        clear_pending();
        const hipError_t e = hipMallocAsync(&own, need, as_stream(stream));
        if (e != hipSuccess)
            return nerf_fail(NERF_ERR_WORKSPACE, "nerf_render_poses: cannot allocate %zu workspace bytes: %s", need,
                             hipGetErrorString(e));
        ws = static_cast<char*>(own);
    }
    float* ro = reinterpret_cast<float*>(ws);
    float* rd = ro + 3 * R;
    float* tn = rd + 3 * R;
    float* tf = tn + R;
    clear_pending();
    launch_fill_f32(tn, R, t_near, as_stream(stream));
    launch_fill_f32(tf, R, t_far, as_stream(stream));
    nerf_status st = check_launch("nerf_render_poses");
    for (int f = 0; f < n_poses && st == NERF_OK; ++f) {
        launch_gen_rays(poses + 12 * (int64_t)f, K->W, K->H, K->fx, K->fy, K->cx, K->cy, ro, rd, as_stream(stream));
        st = check_launch("nerf_render_poses");
        if (st != NERF_OK) break;
        nerf_render_cfg c = *cfg;
        c.ray_offset = cfg->ray_offset + (uint64_t)f * (uint64_t)R;
        st = nerf::render_entry(ro, rd, tn, tf, R, w, &c, rgb + 3 * R * f, depth + R * f, acc + R * f, stream,
                                nullptr, 0);
    }
    if (own) {
        const hipError_t e = hipFreeAsync(own, as_stream(stream));
        if (st == NERF_OK && e != hipSuccess)
            return nerf_fail(NERF_ERR_HIP, "nerf_render_poses: workspace free: %s", hipGetErrorString(e));
    }
    return st;
}

int64_t nerf_train_param_count(int kind) { return net_is_nerf_family(kind) ? train_param_count(kind) : 0; }

size_t nerf_train_workspace_size(const nerf_train_cfg* cfg, int64_t n_rays) {
    if (!cfg || !net_is_nerf_family(cfg->net.kind) || (cfg->net.dtype != NERF_F32 && cfg->net.dtype != NERF_BF16))
        return 0;
    if (cfg->n_samples < 1 || cfg->n_samples > 256 || n_rays < 0) return 0;
    return train_workspace_layout(cfg->net.kind, cfg->net.dtype == NERF_BF16, n_rays, cfg->n_samples, nullptr,
                                  nullptr);
}

nerf_status nerf_train_step(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                            const float* target_rgb, int64_t n_rays, const nerf_train_cfg* cfg, float* params,
                            float* adam_m, float* adam_v, int64_t step, float* grad, float* loss, float* rgb,
                            void* workspace, size_t workspace_bytes, void* stream) {
    NERF_REQUIRE(cfg, "nerf_train_step: cfg is NULL");
    NERF_REQUIRE(n_rays >= 0, "nerf_train_step: n_rays %lld", (long long)n_rays);
    if (!net_is_nerf_family(cfg->net.kind))
        return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_train_step: network kind %d is not a NeRF-family network",
                         cfg->net.kind);
    NERF_REQUIRE(cfg->net.dtype == NERF_F32 || cfg->net.dtype == NERF_BF16, "nerf_train_step: dtype %d",
                 cfg->net.dtype);
    NERF_REQUIRE(cfg->n_samples >= 1 && cfg->n_samples <= 256, "nerf_train_step: n_samples %d outside 1..256",
                 cfg->n_samples);
    if (n_rays * (int64_t)cfg->n_samples > ((int64_t)1 << 28))
        return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_train_step: %lld samples (at most 2^28)",
                         (long long)(n_rays * cfg->n_samples));
    NERF_REQUIRE(!adam_m == !adam_v, "nerf_train_step: give both Adam moments or neither");
    NERF_REQUIRE(!adam_m || step >= 1, "nerf_train_step: Adam step %lld < 1", (long long)step);
    if (n_rays == 0) return NERF_OK;
    NERF_REQUIRE(rays_o && rays_d && t_near && t_far && target_rgb && params && loss,
                 "nerf_train_step: NULL input or output");
    NERF_REQUIRE(aligned4(rays_o) && aligned4(rays_d) && aligned4(t_near) && aligned4(t_far) &&
                     aligned4(target_rgb) && aligned4(params) && aligned4(loss) && (!grad || aligned4(grad)) &&
                     (!rgb || aligned4(rgb)) && (!adam_m || (aligned4(adam_m) && aligned4(adam_v))) &&
                     (!cfg->z || aligned4(cfg->z)) && (!cfg->weights || aligned4(cfg->weights)),
                 "nerf_train_step: misaligned pointer");
    const int bf16 = cfg->net.dtype == NERF_BF16;
    const size_t need = train_workspace_layout(cfg->net.kind, bf16, n_rays, cfg->n_samples, nullptr, nullptr);
    void* own = nullptr;
    if (workspace) {
        if (workspace_bytes < need)
            return nerf_fail(NERF_ERR_WORKSPACE, "nerf_train_step: workspace has %zu bytes, needs %zu",
                             workspace_bytes, need);
        NERF_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
                     "nerf_train_step: workspace must be 256-byte aligned");
    } else {
        clear_pending();
        const hipError_t e = hipMallocAsync(&own, need, as_stream(stream));
        if (e != hipSuccess)
            return nerf_fail(NERF_ERR_WORKSPACE, "nerf_train_step: cannot allocate %zu workspace bytes: %s", need,
                             hipGetErrorString(e));
        workspace = own;
    }
    TrainArgs t{};
    t.ro = rays_o;
    t.rd = rays_d;
    t.tn = t_near;
    t.tf = t_far;
    t.target = target_rgb;
    t.n_rays = n_rays;
    t.n_samples = cfg->n_samples;
    t.use_pi = cfg->use_pi;
    t.white = cfg->white_bkgd;
    t.jitter = cfg->jitter;
    t.seed = cfg->seed;
    t.ray_offset = cfg->ray_offset;
    t.params = params;
    t.adam_m = adam_m;
    t.adam_v = adam_v;
    t.grad = grad;
    t.step = step;
    t.lr = cfg->lr;
    t.beta1 = cfg->beta1;
    t.beta2 = cfg->beta2;
    t.eps = cfg->eps;
    t.loss = loss;
    t.rgb_out = rgb;
    t.z_in = cfg->z;
    t.w_out = cfg->weights;
    t.workspace = workspace;
    clear_pending();
    launch_train_step(cfg->net.kind, bf16, t, as_stream(stream));
    nerf_status st = check_launch("nerf_train_step");
    if (own) {
        const hipError_t e = hipFreeAsync(own, as_stream(stream));
        if (st == NERF_OK && e != hipSuccess)
            st = nerf_fail(NERF_ERR_HIP, "nerf_train_step: workspace free: %s", hipGetErrorString(e));
    }
    return st;
}

static bool inr_cfg_ok(const nerf_hash_inr_cfg* c) {
    return c && c->hidden >= 1 && c->hidden <= 64 && c->n_out >= 1 && c->n_out <= 4;
}

int64_t nerf_hash_inr_param_count(const nerf_hashgrid* g, const nerf_hash_inr_cfg* cfg) {
    if (!inr_cfg_ok(cfg) || check_grid_layout(g, "nerf_hash_inr_param_count") != NERF_OK) return 0;
    return hash_inr_param_count(grid_args(g), cfg->hidden, cfg->n_out);
}

size_t nerf_hash_inr_workspace_size(const nerf_hashgrid* g, const nerf_hash_inr_cfg* cfg, int64_t n) {
    if (!inr_cfg_ok(cfg) || n < 0 || check_grid_layout(g, "nerf_hash_inr_workspace_size") != NERF_OK) return 0;
    return hash_inr_workspace_layout(grid_args(g), cfg->hidden, cfg->n_out, n, nullptr, nullptr);
}

nerf_status nerf_hash_inr_train_step(const float* x, const float* target, int64_t n, const nerf_hashgrid* g,
                                     const nerf_hash_inr_cfg* cfg, float* params, float* adam_m, float* adam_v,
                                     int64_t step, float* grad, float* loss, float* pred, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    const char* who = "nerf_hash_inr_train_step";
    NERF_REQUIRE(inr_cfg_ok(cfg), "%s: cfg NULL or hidden/n_out outside 1..64 / 1..4", who);
    const nerf_status gs = check_grid_layout(g, who);
    if (gs != NERF_OK) return gs;
    NERF_REQUIRE(n >= 0 && n <= ((int64_t)1 << 27), "%s: n %lld above 2^27", who, (long long)n);
    NERF_REQUIRE(!adam_m == !adam_v, "%s: give both Adam moments or neither", who);
    NERF_REQUIRE(!adam_m || step >= 1, "%s: Adam step %lld < 1", who, (long long)step);
    if (n == 0) return NERF_OK;
    NERF_REQUIRE(x && target && params && loss, "%s: NULL input or output", who);
    NERF_REQUIRE(aligned16(x) && aligned4(target) && aligned16(params) && aligned4(loss) &&
                     (!grad || aligned4(grad)) && (!pred || aligned4(pred)) &&
                     (!adam_m || (aligned4(adam_m) && aligned4(adam_v))),
                 "%s: misaligned pointer (x and params 16-byte aligned, the rest 4)", who);
    const GridArgs ga = grid_args(g);
    const size_t need = hash_inr_workspace_layout(ga, cfg->hidden, cfg->n_out, n, nullptr, nullptr);
    void* own = nullptr;
    if (workspace) {
        if (workspace_bytes < need)
            return nerf_fail(NERF_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", who, workspace_bytes, need);
        NERF_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, "%s: workspace must be 256-byte aligned",
                     who);
    } else {
        clear_pending();
        const hipError_t e = hipMallocAsync(&own, need, as_stream(stream));
        if (e != hipSuccess)
            return nerf_fail(NERF_ERR_WORKSPACE, "%s: cannot allocate %zu workspace bytes: %s", who, need,
                             hipGetErrorString(e));
        workspace = own;
    }
    HashInrArgs a{};
    a.x = x;
    a.target = target;
    a.n = n;
    a.hidden = cfg->hidden;
    a.n_out = cfg->n_out;
    a.params = params;
    a.adam_m = adam_m;
    a.adam_v = adam_v;
    a.grad = grad;
    a.step = step;
    a.lr = cfg->lr;
    a.beta1 = cfg->beta1;
    a.beta2 = cfg->beta2;
    a.eps = cfg->eps;
    a.loss = loss;
    a.pred = pred;
    a.workspace = workspace;
    clear_pending();
    launch_hash_inr_step(ga, a, as_stream(stream));
    nerf_status st = check_launch(who);
    if (own) {
        const hipError_t e = hipFreeAsync(own, as_stream(stream));
        if (st == NERF_OK && e != hipSuccess) st = nerf_fail(NERF_ERR_HIP, "%s: workspace free: %s", who, hipGetErrorString(e));
    }
    return st;
}

}  // extern "C"

namespace nerf {

// Rays per launch of the many-network mode that fit `bytes` of workspace
// (0 if not even one ray does).
static int64_t kilo_chunk_fitting(const nerf_render_cfg* cfg, int64_t n_rays, size_t bytes) {
    const int n_cells = cfg->cell_res * cfg->cell_res * cfg->cell_res;
    int64_t lo = 0, hi = n_rays;  // largest chunk whose layout fits
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (kilo_workspace_layout(mid, cfg->n_coarse, n_cells, nullptr, nullptr) <= bytes)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

nerf_status render_entry(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                         int64_t n_rays, const nerf_weights* w, const nerf_render_cfg* cfg, float* rgb, float* depth,
                         float* acc, void* stream, void* fixed_ws, size_t fixed_bytes) {
    NERF_REQUIRE(w && cfg, "nerf_render: NULL weights or cfg");
    NERF_REQUIRE(n_rays >= 0, "nerf_render: n_rays %lld", (long long)n_rays);
    NERF_REQUIRE(cfg->n_coarse >= 1 && cfg->n_coarse <= 256, "nerf_render: n_coarse %d outside 1..256",
                 cfg->n_coarse);
    NERF_REQUIRE(cfg->n_fine >= 0, "nerf_render: n_fine %d", cfg->n_fine);
    NERF_REQUIRE(cfg->chunk >= 0, "nerf_render: chunk %lld", (long long)cfg->chunk);
    if (nerf_mlp_packed_bytes(&w->net) == 0)
        return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_render: unsupported network kind %d / dtype %d", w->net.kind,
                         w->net.dtype);
    const int bf16 = w->net.dtype == NERF_BF16;
    RenderArgs a{};
    a.n_coarse = cfg->n_coarse;
    a.n_fine = cfg->n_fine;
    a.use_pi = cfg->use_pi;
    a.white = cfg->white_bkgd;
    a.jitter = cfg->jitter;
    a.seed = cfg->seed;
    a.box_lo = cfg->box_lo;
    a.box_hi = cfg->box_hi;
    if (cfg->mode != NERF_MODE_KILO) {
        // empty-space skipping (occupancy grid over the box) and early termination
        NERF_REQUIRE(cfg->term_T >= 0.0f, "nerf_render: term_T %g < 0", (double)cfg->term_T);
        a.term_T = cfg->term_T;
        a.n_live = cfg->dbg_n_live;
        if (cfg->occ) {
            NERF_REQUIRE(cfg->occ_res >= 1 && cfg->occ_res <= 2048, "nerf_render: occ_res %d outside 1..2048",
                         cfg->occ_res);
            NERF_REQUIRE(cfg->box_hi > cfg->box_lo, "nerf_render: empty scene box");
            a.occ = cfg->occ;
            a.occ_res = cfg->occ_res;
            a.vscale = (float)((double)cfg->occ_res / ((double)cfg->box_hi - (double)cfg->box_lo));
        }
    }
    GridArgs ga{};
    switch (cfg->mode) {
        case NERF_MODE_NERF:
            if (w->net.kind != NET_8x256 && w->net.kind != NET_4x64)
                return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_render: NeRF mode needs the 8x256 or 4x64 network");
            NERF_REQUIRE(w->coarse, "nerf_render: coarse network is NULL");
            if (cfg->n_fine > 0) {
                NERF_REQUIRE(w->fine, "nerf_render: fine network is NULL");
                NERF_REQUIRE(cfg->n_coarse >= 3, "nerf_render: resampling needs n_coarse >= 3");
                NERF_REQUIRE(cfg->n_coarse + cfg->n_fine <= 256, "nerf_render: n_coarse + n_fine > 256");
            }
            NERF_REQUIRE(aligned16(w->coarse) && (!w->fine || aligned16(w->fine)),
                         "nerf_render: packed networks must be 16-byte aligned");
            break;
        case NERF_MODE_HASH: {
            if (w->net.kind != NET_HASH_FIELD)
                return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_render: hash mode needs the hash-field network");
            NERF_REQUIRE(w->coarse, "nerf_render: field network is NULL");
            NERF_REQUIRE(aligned16(w->coarse), "nerf_render: packed network must be 16-byte aligned");
            NERF_REQUIRE(cfg->n_fine == 0, "nerf_render: hash mode has no resampling pass");
            const nerf_status gs = check_grid(w->grid, "nerf_render");
            if (gs != NERF_OK) return gs;
            if (w->grid->n_levels != 16 || w->grid->dim != 3)
                return nerf_fail(NERF_ERR_UNSUPPORTED,
                                 "nerf_render: the field network takes a 3D grid of 16 levels x 2 features");
            NERF_REQUIRE(cfg->box_hi > cfg->box_lo, "nerf_render: empty scene box");
            ga = grid_args(w->grid);
            break;
        }
        case NERF_MODE_KILO: {
            if (w->net.kind != NET_CELL_2x32)
                return nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_render: many-network mode needs the 2x32 cell network");
            NERF_REQUIRE(cfg->n_fine == 0, "nerf_render: many-network mode has no resampling pass");
            NERF_REQUIRE(cfg->cell_res >= 1 && cfg->cell_res <= 40, "nerf_render: cell_res %d outside 1..40",
                         cfg->cell_res);
            NERF_REQUIRE(cfg->occ_res >= 1 && cfg->occ_res <= 2048, "nerf_render: occ_res %d outside 1..2048",
                         cfg->occ_res);
            NERF_REQUIRE(w->n_cells == cfg->cell_res * cfg->cell_res * cfg->cell_res,
                         "nerf_render: n_cells %d != cell_res^3", w->n_cells);
            NERF_REQUIRE(w->cells && cfg->occ, "nerf_render: cell networks or occupancy grid is NULL");
            NERF_REQUIRE(aligned16(w->cells), "nerf_render: packed cell networks must be 16-byte aligned");
            NERF_REQUIRE(cfg->box_hi > cfg->box_lo, "nerf_render: empty scene box");
            NERF_REQUIRE(cfg->term_T >= 0.0f, "nerf_render: term_T %g < 0", (double)cfg->term_T);
            break;
        }
        default:
            return nerf_fail(NERF_ERR_INVALID_ARGUMENT, "nerf_render: mode %d", cfg->mode);
    }
    if (n_rays == 0) return NERF_OK;
    NERF_REQUIRE(rays_o && rays_d && t_near && t_far && rgb && depth && acc, "nerf_render: NULL ray or output");
    const int n_total = cfg->mode == NERF_MODE_NERF ? cfg->n_coarse + cfg->n_fine : cfg->n_coarse;
    int64_t chunk = cfg->chunk > 0 ? cfg->chunk : n_rays;
    KiloArgs ka{};
    void* own_ws = nullptr;
    if (cfg->mode == NERF_MODE_KILO) {
        chunk = kilo_chunk(cfg, n_rays);
        const int n_cells = cfg->cell_res * cfg->cell_res * cfg->cell_res;
        if (fixed_ws) {
            // the library's fixed scratch: the caller's chunk must fit it;
            // without one, the largest chunk that fits is used
            NERF_REQUIRE(!cfg->workspace, "nerf_render_noalloc: cfg.workspace must be NULL (the call uses the "
                                          "library's fixed scratch)");
            const int64_t fit = kilo_chunk_fitting(cfg, chunk, fixed_bytes);
            if (fit < 1 || (cfg->chunk > 0 && fit < chunk))
                return nerf_fail(NERF_ERR_WORKSPACE,
                                 "nerf_render_noalloc: a chunk of %lld rays x %d samples needs %zu workspace bytes, "
                                 "the fixed scratch holds %zu",
                                 (long long)chunk, cfg->n_coarse,
                                 kilo_workspace_layout(cfg->chunk > 0 ? chunk : 1, cfg->n_coarse, n_cells, nullptr,
                                                       nullptr),
                                 fixed_bytes);
            chunk = fit;
        }
        const size_t need = kilo_workspace_layout(chunk, cfg->n_coarse, n_cells, nullptr, nullptr);
        char* ws = fixed_ws ? static_cast<char*>(fixed_ws) : static_cast<char*>(cfg->workspace);
        if (!fixed_ws) {  // (the fixed scratch fits by the choice of chunk above)
            if (ws) {
                if (cfg->workspace_bytes < need)
                    return nerf_fail(NERF_ERR_WORKSPACE, "nerf_render: workspace has %zu bytes, needs %zu",
                                     cfg->workspace_bytes, need);
                NERF_REQUIRE(aligned16(ws), "nerf_render: workspace must be 16-byte aligned");
            } else {
                clear_pending();
                const hipError_t e = hipMallocAsync(&own_ws, need, as_stream(stream));
                if (e != hipSuccess)
                    return nerf_fail(NERF_ERR_WORKSPACE, "nerf_render: cannot allocate %zu workspace bytes: %s",
                                     need, hipGetErrorString(e));
                ws = static_cast<char*>(own_ws);
            }
        }
        kilo_workspace_layout(chunk, cfg->n_coarse, n_cells, ws, &ka);
        ka.lo = cfg->box_lo;
        ka.hi = cfg->box_hi;
        const double span = (double)cfg->box_hi - (double)cfg->box_lo;
        ka.vscale = (float)((double)cfg->occ_res / span);
        ka.cscale = (float)((double)cfg->cell_res / span);
        ka.occ_res = cfg->occ_res;
        ka.cell_res = cfg->cell_res;
        ka.term_T = cfg->term_T;
        ka.occ = cfg->occ;
        ka.cells = w->cells;
        ka.cell_stride = nerf_mlp_packed_bytes(&w->net);
        ka.dbg_n_live = cfg->dbg_n_live;
    }
    clear_pending();
    if (cfg->mode != NERF_MODE_KILO && cfg->dbg_n_live)  // (added to by every ray of every chunk)
        launch_fill_f32(reinterpret_cast<float*>(cfg->dbg_n_live), 2, 0.0f, as_stream(stream));
    for (int64_t r0 = 0; r0 < n_rays; r0 += chunk) {
        const int64_t nr = (n_rays - r0) < chunk ? (n_rays - r0) : chunk;
        RenderArgs c = a;
        c.ro = rays_o + 3 * r0;
        c.rd = rays_d + 3 * r0;
        c.tn = t_near + r0;
        c.tf = t_far + r0;
        c.n_rays = nr;
        c.ray_offset = cfg->ray_offset + (uint64_t)r0;
        c.coarse = w->coarse;
        c.fine = w->fine;
        c.rgb = rgb + 3 * r0;
        c.depth = depth + r0;
        c.acc = acc + r0;
        c.dbg_z = cfg->dbg_z ? cfg->dbg_z + r0 * n_total : nullptr;
        c.dbg_w = cfg->dbg_w_coarse ? cfg->dbg_w_coarse + r0 * cfg->n_coarse : nullptr;
        if (cfg->mode == NERF_MODE_NERF)
            launch_render_nerf(w->net.kind, bf16, c, as_stream(stream));
        else if (cfg->mode == NERF_MODE_HASH)
            launch_render_hash(bf16, c, ga, as_stream(stream));
        else
            launch_render_kilo(bf16, c, ka, r0 > 0, as_stream(stream));
        const nerf_status st = check_launch("nerf_render");
        if (st != NERF_OK) {
            if (own_ws) (void)hipFreeAsync(own_ws, as_stream(stream));
            return st;
        }
    }
    if (own_ws) {
        const hipError_t e = hipFreeAsync(own_ws, as_stream(stream));
        if (e != hipSuccess) return nerf_fail(NERF_ERR_HIP, "nerf_render: workspace free: %s", hipGetErrorString(e));
    }
    return NERF_OK;
}

}  // namespace nerf

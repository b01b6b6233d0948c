// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU.
//
// The library's host sources (argument validation, packing, workspace
// layouts, chunk and frame loops) are linked against stand-ins for the
// device launchers, which only count calls, and for the four HIP runtime
// calls the ABI makes, whose failures can be forced.  "Device" buffers are
// host allocations that the stand-ins never touch.  Every check prints a
// line; the program exits non-zero at the first failed check.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "launch.hpp"
#include "nerf_mi355x.h"

// ---------------------------------------------------------------------------
// Stand-ins
// ---------------------------------------------------------------------------
static int g_launches = 0;
static bool g_fail_malloc = false;
static bool g_fail_launch = false;  // the next launch leaves an error for hipGetLastError
static bool g_pending = false;
static int g_live_allocs = 0;

static void launched() {
    ++g_launches;
    if (g_fail_launch) {
        g_pending = true;
        g_fail_launch = false;
    }
}

extern "C" {
hipError_t hipMallocAsync(void** p, size_t bytes, hipStream_t) {
    if (g_fail_malloc) return hipErrorOutOfMemory;
    *p = std::malloc(bytes ? bytes : 1);
    ++g_live_allocs;
    return hipSuccess;
}
hipError_t hipFreeAsync(void* p, hipStream_t) {
    std::free(p);
    --g_live_allocs;
    return hipSuccess;
}
hipError_t hipGetLastError(void) {
    const hipError_t e = g_pending ? hipErrorLaunchFailure : hipSuccess;
    g_pending = false;
    return e;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "forced error"; }
}

namespace nerf {
void launch_gen_rays(const float*, int, int, float, float, float, float, float*, float*, hipStream_t) { launched(); }
void launch_fill_f32(float*, int64_t, float, hipStream_t) { launched(); }
void launch_stratified(const float*, const float*, int64_t, int, uint64_t, uint64_t, int, float*, hipStream_t) {
    launched();
}
void launch_encode_freq(const float*, int64_t, int, int, int, int, int, void*, hipStream_t) { launched(); }
void launch_sh16(const float*, int64_t, float*, hipStream_t) { launched(); }
void launch_encode_hash(const float*, int64_t, const GridArgs&, float*, uint32_t*, hipStream_t) { launched(); }
void launch_composite(const float*, const float*, const float*, int64_t, int, int, float*, float*, float*, float*,
                      hipStream_t) {
    launched();
}
void launch_sample_pdf(const float*, const float*, int64_t, int, int, uint64_t, uint64_t, float*, int32_t*, float*,
                       hipStream_t) {
    launched();
}
void launch_render_nerf(int, int, const RenderArgs&, hipStream_t) { launched(); }
void launch_mlp_bf16(int, const void*, const float*, const float*, int64_t, int, float*, hipStream_t) { launched(); }
void launch_mlp_f32(int, const void*, const float*, const float*, int64_t, int, float*, hipStream_t) { launched(); }
void launch_render_hash(int, const RenderArgs&, const GridArgs&, hipStream_t) { launched(); }
void launch_render_kilo(int, const RenderArgs&, const KiloArgs& k, int, hipStream_t) {
    // the workspace pointers carved by the ABI lie inside the allocation it made
    if (!k.live_mask || !k.raw_live || k.mask_words < 1) std::abort();
    launched();
}
void launch_train_step(int, int, const TrainArgs& t, hipStream_t) {
    if (!t.workspace || !t.loss) std::abort();
    launched();
}
void launch_hash_inr_step(const GridArgs&, const HashInrArgs& a, hipStream_t) {
    if (!a.workspace || !a.loss || a.hidden < 1) std::abort();
    launched();
}
}  // namespace nerf

// ---------------------------------------------------------------------------
// Checks
// ---------------------------------------------------------------------------
static int g_checks = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        ++g_checks;                                                                   \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                         nerf_last_error());                                          \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

struct Buf {
    std::vector<float> v;
    explicit Buf(size_t n) : v(n ? n : 1, 0.0f) {}
    float* p() { return v.data(); }
};

static std::vector<std::vector<float>> random_net(int kind, std::mt19937& g) {
    // shapes of the four networks in nerf_pack_mlp's order (out, in)
    std::vector<std::pair<int, int>> shp;
    if (kind == NERF_NET_8x256) {
        for (int l = 0; l < 8; ++l) shp.push_back({256, l == 0 ? 63 : (l == 5 ? 319 : 256)});
        shp.insert(shp.end(), {{1, 256}, {256, 256}, {128, 283}, {3, 128}});
    } else if (kind == NERF_NET_4x64) {
        for (int l = 0; l < 4; ++l) shp.push_back({64, l == 0 ? 39 : 64});
        shp.insert(shp.end(), {{1, 64}, {64, 64}, {32, 91}, {3, 32}});
    } else if (kind == NERF_NET_CELL_2x32) {
        shp = {{32, 63}, {32, 32}, {1, 32}, {32, 32}, {16, 59}, {3, 16}};
    } else {
        shp = {{64, 32}, {64, 64}, {1, 64}, {64, 64}, {64, 80}, {64, 64}, {3, 64}};
    }
    std::uniform_real_distribution<float> u(-1.0f, 1.0f);
    std::vector<std::vector<float>> t;
    for (auto [o, i] : shp) {
        std::vector<float> W((size_t)o * i), b(o);
        for (auto& x : W) x = u(g);
        for (auto& x : b) x = u(g);
        t.push_back(W);
        t.push_back(b);
    }
    return t;
}

static void check_packing() {
    std::mt19937 g(1);
    for (int kind = 1; kind <= 4; ++kind)
        for (int dt = 0; dt <= 1; ++dt) {
            nerf_mlp_desc d{kind, dt};
            const size_t n = nerf_mlp_packed_bytes(&d);
            CHECK(n > 0);
            auto t = random_net(kind, g);
            std::vector<const float*> ptrs;
            for (auto& x : t) ptrs.push_back(x.data());
            std::vector<unsigned char> dst(n);
            CHECK(nerf_pack_mlp(&d, ptrs.data(), (int)ptrs.size(), dst.data(), n) == NERF_OK);
            CHECK(nerf_pack_mlp(&d, ptrs.data(), (int)ptrs.size(), dst.data(), n - 1) != NERF_OK);
            CHECK(nerf_pack_mlp(&d, ptrs.data(), (int)ptrs.size() - 1, dst.data(), n) != NERF_OK);
        }
    nerf_mlp_desc bad{9, 0};
    CHECK(nerf_mlp_packed_bytes(&bad) == 0);
    std::printf("packing: ok\n");
}

static void check_hashgrid() {
    nerf_hashgrid h;
    CHECK(nerf_hashgrid_init(&h, 3, 16, 1u << 19, 16, 2048) == NERF_OK);
    CHECK(h.total_entries > 0 && h.dim == 3);
    CHECK(nerf_hashgrid_init(&h, 2, 8, 1u << 12, 4, 256) == NERF_OK);
    CHECK(nerf_hashgrid_init(&h, 4, 8, 1u << 12, 4, 256) != NERF_OK);
    CHECK(nerf_hashgrid_init(&h, 3, 17, 1u << 12, 4, 256) != NERF_OK);
    CHECK(nerf_hashgrid_init(&h, 3, 8, 3000, 4, 256) != NERF_OK);
    std::printf("hash grid init: ok\n");
}

static void check_steps() {
    const int64_t R = 1000;
    Buf ro(3 * R), rd(3 * R), tn(R), tf(R), z(R * 64), raw(R * 64 * 4), rgb(3 * R), dep(R), acc(R), w(R * 64);
    float pose[12] = {1, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1, 4};
    nerf_intrinsics K{32, 32, 40.f, 40.f, 16.f, 16.f};
    int before = g_launches;
    CHECK(nerf_gen_rays(pose, &K, ro.p(), rd.p(), nullptr) == NERF_OK && g_launches == before + 1);
    nerf_intrinsics bad{0, 32, 40.f, 40.f, 16.f, 16.f};
    before = g_launches;
    CHECK(nerf_gen_rays(pose, &bad, ro.p(), rd.p(), nullptr) == NERF_ERR_INVALID_ARGUMENT && g_launches == before);
    CHECK(nerf_sample_stratified(tn.p(), tf.p(), R, 64, 0, 0, 1, z.p(), nullptr) == NERF_OK);
    CHECK(nerf_sample_stratified(tn.p(), tf.p(), R, 257, 0, 0, 1, z.p(), nullptr) == NERF_ERR_INVALID_ARGUMENT);
    CHECK(nerf_encode_freq(ro.p(), R, 3, 10, 1, 1, NERF_F32, raw.p(), nullptr) == NERF_OK);
    CHECK(nerf_encode_freq(ro.p(), R, 5, 10, 1, 1, NERF_F32, raw.p(), nullptr) == NERF_ERR_INVALID_ARGUMENT);
    CHECK(nerf_composite(raw.p(), z.p(), rd.p(), R, 64, 0, rgb.p(), dep.p(), acc.p(), w.p(), nullptr) == NERF_OK);
    CHECK(nerf_composite(raw.p(), z.p(), rd.p(), -1, 64, 0, rgb.p(), dep.p(), acc.p(), w.p(), nullptr) ==
          NERF_ERR_INVALID_ARGUMENT);
    CHECK(nerf_sample_pdf(z.p(), w.p(), R, 64, 128, 0, 0, nullptr, nullptr, raw.p(), nullptr) == NERF_OK);
    // a launch failure reported by the runtime maps to NERF_ERR_HIP
    g_fail_launch = true;
    CHECK(nerf_composite(raw.p(), z.p(), rd.p(), R, 64, 0, rgb.p(), dep.p(), acc.p(), w.p(), nullptr) == NERF_ERR_HIP);
    std::printf("single steps: ok\n");
}

static void check_renders() {
    const int64_t R = 5000;
    Buf ro(3 * R), rd(3 * R), tn(R), tf(R), rgb(3 * R), dep(R), acc(R);
    std::vector<unsigned char> packed(2 << 20), cells(64 * 40000);
    std::vector<uint32_t> occ(128 * 128 * 128 / 32);
    nerf_weights w{};
    w.net = {NERF_NET_8x256, NERF_BF16};
    w.coarse = packed.data();
    w.fine = packed.data();
    nerf_render_cfg c{};
    c.mode = NERF_MODE_NERF;
    c.n_coarse = 64;
    c.n_fine = 128;
    c.chunk = 777;  // several launches, the last one ragged
    int before = g_launches;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &w, &c, rgb.p(), dep.p(), acc.p(), nullptr) == NERF_OK);
    CHECK(g_launches - before == (int)((R + 776) / 777));
    c.n_fine = 200;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &w, &c, rgb.p(), dep.p(), acc.p(), nullptr) ==
          NERF_ERR_INVALID_ARGUMENT);
    // many networks: a caller workspace that is too small, then the library's own, then a failed allocation
    nerf_weights wk{};
    wk.net = {NERF_NET_CELL_2x32, NERF_BF16};
    wk.cells = cells.data();
    wk.n_cells = 4096;
    nerf_render_cfg k{};
    k.mode = NERF_MODE_KILO;
    k.n_coarse = 192;
    k.occ_res = 128;
    k.cell_res = 16;
    k.box_lo = -1.5f;
    k.box_hi = 1.5f;
    k.term_T = 1e-2f;
    k.occ = occ.data();
    const size_t need = nerf_render_workspace_size(&k, R);
    CHECK(need > 0);
    std::vector<unsigned char> ws(need);
    k.workspace = ws.data();
    k.workspace_bytes = need - 1;
    before = g_launches;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &wk, &k, rgb.p(), dep.p(), acc.p(), nullptr) ==
          NERF_ERR_WORKSPACE);
    CHECK(g_launches == before);
    k.workspace_bytes = need;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &wk, &k, rgb.p(), dep.p(), acc.p(), nullptr) == NERF_OK);
    k.workspace = nullptr;
    k.workspace_bytes = 0;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &wk, &k, rgb.p(), dep.p(), acc.p(), nullptr) == NERF_OK);
    CHECK(g_live_allocs == 0);
    g_fail_malloc = true;
    before = g_launches;
    CHECK(nerf_render(ro.p(), rd.p(), tn.p(), tf.p(), R, &wk, &k, rgb.p(), dep.p(), acc.p(), nullptr) ==
          NERF_ERR_WORKSPACE);
    CHECK(g_launches == before);
    // a pose sweep that cannot allocate its frame buffers
    nerf_intrinsics K{40, 30, 50.f, 50.f, 20.f, 15.f};
    std::vector<float> poses(3 * 12, 0.0f);
    Buf frgb(3 * 3 * 1200), fdep(3 * 1200), facc(3 * 1200);
    CHECK(nerf_render_poses(poses.data(), 3, &K, 2.f, 6.f, &w, &c, nullptr, 0, frgb.p(), fdep.p(), facc.p(),
                            nullptr) != NERF_OK);  // n_fine 200 is refused before any allocation
    c.n_fine = 128;
    CHECK(nerf_render_poses(poses.data(), 3, &K, 2.f, 6.f, &w, &c, nullptr, 0, frgb.p(), fdep.p(), facc.p(),
                            nullptr) == NERF_ERR_WORKSPACE);
    g_fail_malloc = false;
    before = g_launches;
    CHECK(nerf_render_poses(poses.data(), 3, &K, 2.f, 6.f, &w, &c, nullptr, 0, frgb.p(), fdep.p(), facc.p(),
                            nullptr) == NERF_OK);
    CHECK(g_launches - before == 2 + 3 * (1 + 2));  // near/far fills; per frame its rays and 2 chunks of 777 rays
    CHECK(g_live_allocs == 0);
    std::printf("renders: ok\n");
}

static void check_training() {
    for (int kind = 1; kind <= 3; ++kind) {
        const int64_t P = nerf_train_param_count(kind);
        CHECK(P > 0);
        nerf_train_cfg c{};
        c.net = {kind, NERF_BF16};
        c.n_samples = 64;
        c.lr = 1e-3f;
        c.beta1 = 0.9f;
        c.beta2 = 0.999f;
        c.eps = 1e-8f;
        const int64_t R = 300;
        const size_t need = nerf_train_workspace_size(&c, R);
        CHECK(need > (size_t)R * 64 * 4);
        Buf ro(3 * R), rd(3 * R), tn(R), tf(R), tg(3 * R), p(P), m(P), v(P), gr(P), loss(1), rgb(3 * R);
        std::vector<unsigned char> ws(need + 256);
        void* ws_al = (void*)(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
        int before = g_launches;
        CHECK(nerf_train_step(ro.p(), rd.p(), tn.p(), tf.p(), tg.p(), R, &c, p.p(), m.p(), v.p(), 1, gr.p(), loss.p(),
                              rgb.p(), ws_al, need, nullptr) == NERF_OK);
        CHECK(g_launches == before + 1);
        CHECK(nerf_train_step(ro.p(), rd.p(), tn.p(), tf.p(), tg.p(), R, &c, p.p(), m.p(), v.p(), 1, gr.p(), loss.p(),
                              rgb.p(), ws_al, need - 1, nullptr) == NERF_ERR_WORKSPACE);
        CHECK(nerf_train_step(ro.p(), rd.p(), tn.p(), tf.p(), tg.p(), R, &c, p.p(), m.p(), v.p(), 1, gr.p(), loss.p(),
                              rgb.p(), nullptr, 0, nullptr) == NERF_OK);
        CHECK(g_live_allocs == 0);
        g_fail_malloc = true;
        CHECK(nerf_train_step(ro.p(), rd.p(), tn.p(), tf.p(), tg.p(), R, &c, p.p(), m.p(), v.p(), 1, gr.p(), loss.p(),
                              rgb.p(), nullptr, 0, nullptr) == NERF_ERR_WORKSPACE);
        g_fail_malloc = false;
        CHECK(nerf_train_step(ro.p(), rd.p(), tn.p(), tf.p(), tg.p(), R, &c, p.p(), m.p(), nullptr, 1, gr.p(),
                              loss.p(), rgb.p(), ws_al, need, nullptr) == NERF_ERR_INVALID_ARGUMENT);
    }
    std::printf("training: ok\n");
}

int main() {
    check_packing();
    check_hashgrid();
    check_steps();
    check_renders();
    check_training();
    std::printf("all %d checks passed\n", g_checks);
    return 0;
}

// Kernels of the NeRF forward-render path for gfx950 and their launchers.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "mlp.hpp"
#include "raysteps.hpp"

namespace nerf {

// ===========================================================================
// Rays ("Spatial Intelligence - Part 1: NeRF", Section 2 Code, 2. Ray
// generation).  One thread per pixel, rounded float32 operations only.
// ===========================================================================
struct Pose {
    float m[12];
};

__global__ void __launch_bounds__(256) k_gen_rays(Pose P, int W, int H, float fx, float fy, float cx, float cy,
                                                  float* __restrict__ ro, float* __restrict__ rd) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= (int64_t)W * H) return;
    const int i = (int)(r % W), j = (int)(r / W);
    const float dx = __fdiv_rn(__fsub_rn((float)i, cx), fx);
    const float dy = -__fdiv_rn(__fsub_rn((float)j, cy), fy);
    const float dz = -1.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float* R = P.m + 4 * k;
        rd[3 * r + k] = __fadd_rn(__fadd_rn(__fmul_rn(R[0], dx), __fmul_rn(R[1], dy)), __fmul_rn(R[2], dz));
        ro[3 * r + k] = R[3];
    }
}

void launch_gen_rays(const float* pose, int W, int H, float fx, float fy, float cx, float cy, float* ro, float* rd,
                     hipStream_t s) {
    Pose P;
    for (int i = 0; i < 12; ++i) P.m[i] = pose[i];
    const int64_t n = (int64_t)W * H;
    hipLaunchKernelGGL(k_gen_rays, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P, W, H, fx, fy, cx, cy, ro,
                       rd);
}

__global__ void __launch_bounds__(256) k_fill_f32(float* __restrict__ p, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
}

// ===========================================================================
// Stratified samples: one thread per (ray, sample).
// ===========================================================================
__global__ void __launch_bounds__(256) k_stratified(const float* __restrict__ tn, const float* __restrict__ tf,
                                                    int64_t n_rays, int n, uint64_t seed, uint64_t ray_offset,
                                                    int jitter, float* __restrict__ z) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_rays * n) return;
    const int64_t r = t / n;
    const int i = (int)(t - r * n);
    const float u = jitter ? philox_uniform(seed, ray_offset + (uint64_t)r, (uint32_t)i, kStreamJitter) : 0.5f;
    z[t] = stratified_z(tn[r], tf[r], i, n, u);
}

void launch_stratified(const float* tn, const float* tf, int64_t n_rays, int n, uint64_t seed, uint64_t ray_offset,
                       int jitter, float* z, hipStream_t s) {
    const int64_t tot = n_rays * n;
    hipLaunchKernelGGL(k_stratified, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, tn, tf, n_rays, n, seed,
                       ray_offset, jitter, z);
}

// ===========================================================================
// Frequency encoding.  A workgroup encodes pw consecutive points, one thread
// per point, into a float32 stage in LDS (row stride = width, odd for the
// usual widths, so a wave's rows fall in distinct banks); the workgroup then
// streams the points' rows, which are contiguous in the output, with
// aligned 16-byte stores.
// ===========================================================================
constexpr int kEncStageBytes = 65536;

// Points per workgroup: a multiple of 8 (16-byte aligned rows of the block
// for any width and either output type) whose stage fits kEncStageBytes.
__host__ __device__ inline int enc_points_per_block(int width) {
    const int pw = kEncStageBytes / (4 * width);
    return (pw >= 256 ? 256 : pw) / 8 * 8;
}

__device__ __forceinline__ void enc_store16(float* dst, const float* src) {
    *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
}
__device__ __forceinline__ void enc_store16(__bf16* dst, const float* src) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_bf16(src[j]);
    *reinterpret_cast<bf16x8*>(dst) = v;
}
__device__ __forceinline__ void enc_store1(float* dst, float v) { *dst = v; }
__device__ __forceinline__ void enc_store1(__bf16* dst, float v) { *dst = to_bf16(v); }

// One point's row: [x (inc)] then for k < L: sin(2^k x_a) for a < D, then
// cos(2^k x_a) for a < D (times pi with use_pi).
template <int D>
__device__ __forceinline__ void enc_row(const float* xp, int d, int L, int inc, int use_pi, float* o) {
    constexpr int DD = D > 0 ? D : 4;
    const int dn = D > 0 ? D : d;
    float xv[DD];
#pragma unroll
    for (int a = 0; a < DD; ++a) xv[a] = a < dn ? xp[a] : 0.0f;
    if (inc) {
#pragma unroll
        for (int a = 0; a < DD; ++a)
            if (a < dn) o[a] = xv[a];
        o += dn;
    }
    for (int k = 0; k < L; ++k, o += 2 * dn) {
#pragma unroll
        for (int a = 0; a < DD; ++a) {
            if (a < dn) {
                const float arg = ldexpf(xv[a], k);  // exact
                float sn, cs;
                if (use_pi)
                    sincospi_taylor(arg, sn, cs);
                else
                    sincosf(arg, &sn, &cs);
                o[a] = sn;
                o[dn + a] = cs;
            }
        }
    }
}

template <typename OutT>
__global__ void __launch_bounds__(256) k_encode_freq(const float* __restrict__ x, int64_t n, int d, int L, int inc,
                                                     int use_pi, int pw, int vec, OutT* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) float enc_stage[];
    const int width = d * ((inc ? 1 : 0) + 2 * L);
    const int64_t p0 = (int64_t)blockIdx.x * pw;
    const int np = (int)((n - p0) < pw ? (n - p0) : pw);
    for (int pl = threadIdx.x; pl < np; pl += blockDim.x) {
        const float* xp = x + (p0 + pl) * d;
        float* o = enc_stage + pl * width;
        if (d == 3)
            enc_row<3>(xp, d, L, inc, use_pi, o);
        else
            enc_row<0>(xp, d, L, inc, use_pi, o);
    }
    __syncthreads();
    constexpr int VEC = 16 / (int)sizeof(OutT);
    OutT* dst = out + p0 * width;  // 16-byte aligned when out is (vec): pw is a multiple of 8
    const int total = np * width, nv = vec ? total / VEC : 0;
    for (int i = threadIdx.x; i < nv; i += blockDim.x) enc_store16(dst + i * VEC, enc_stage + i * VEC);
    for (int i = nv * VEC + threadIdx.x; i < total; i += blockDim.x) enc_store1(dst + i, enc_stage[i]);
}

void launch_encode_freq(const float* x, int64_t n, int d, int L, int inc, int use_pi, int bf16, void* out,
                        hipStream_t s) {
    const int width = d * ((inc ? 1 : 0) + 2 * L);
    const int pw = enc_points_per_block(width);
    const int threads = (pw + 63) / 64 * 64;  // one thread per point
    const dim3 g((unsigned)((n + pw - 1) / pw));
    const size_t lds = (size_t)pw * width * sizeof(float);
    const int vec = (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
    if (bf16)
        hipLaunchKernelGGL(k_encode_freq<__bf16>, g, dim3(threads), lds, s, x, n, d, L, inc, use_pi, pw, vec,
                           (__bf16*)out);
    else
        hipLaunchKernelGGL(k_encode_freq<float>, g, dim3(threads), lds, s, x, n, d, L, inc, use_pi, pw, vec,
                           (float*)out);
}

// ===========================================================================
// Spherical harmonics of directions
// ===========================================================================
__global__ void __launch_bounds__(256) k_sh16(const float* __restrict__ dirs, int64_t n, float* __restrict__ out) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n) return;
    float x = dirs[3 * p], y = dirs[3 * p + 1], z = dirs[3 * p + 2];
    const float inv = 1.0f / sqrtf(x * x + y * y + z * z);
    float o[16];
    sh16_eval(x * inv, y * inv, z * inv, o);
#pragma unroll
    for (int i = 0; i < 16; ++i) out[16 * p + i] = o[i];
}

void launch_sh16(const float* dirs, int64_t n, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_sh16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dirs, n, out);
}

// ===========================================================================
// Hash-grid encoding ("Instant-NGP - Visual Experiments", shared toolkit,
// extended to 3D), level-major.  The coarsest direct levels whose tables fit
// LDS together are staged there by workgroups that each take a large tile of
// points.  The other levels run as work items (level pair, tile of points)
// ordered by level, so the workgroups in flight at any moment gather from
// one pair's tables, which then stay in the L2 of every die instead of all
// 24 MB of tables competing for it; each point's two levels are written as
// one 16-byte store.
// ===========================================================================
constexpr int kHashLdsMax = 160 * 1024;  // LDS of one workgroup
constexpr int kHashLdsTile = 16384;      // points per staged workgroup
#ifndef NERF_HASH_LPI
#define NERF_HASH_LPI 2
#endif
constexpr int kHashLpi = NERF_HASH_LPI;  // levels per work item
constexpr int kHashPts = 2;              // points per thread of a work item

// Writes the features of levels l .. l+nl-1 (nl <= 2) of point p.
__device__ __forceinline__ void store_levels(float* out, int64_t p, int L, int l, int nl, const float (&f)[4]) {
    float2* o = reinterpret_cast<float2*>(out) + p * L + l;
    if (nl == 2 && ((reinterpret_cast<uintptr_t>(o) & 15u) == 0)) {
        *reinterpret_cast<f32x4*>(o) = f32x4{f[0], f[1], f[2], f[3]};
    } else {
        o[0] = make_float2(f[0], f[1]);
        if (nl == 2) o[1] = make_float2(f[2], f[3]);
    }
}

template <int DIM>
__global__ void __launch_bounds__(1024) k_encode_hash_lds(const float* __restrict__ x, int64_t n, GridArgs g,
                                                          int n_staged, float* __restrict__ out,
                                                          uint32_t* __restrict__ idx_dbg) {
    extern __shared__ __attribute__((aligned(16))) uint32_t hash_tab[];
    // the staged levels are consecutive in the tables: one copy brings them
    // all (the last word's second entry, if any, is padding)
    const uint32_t* src = reinterpret_cast<const uint32_t*>(g.tables) + g.offset[0];
    uint32_t m = 0;
    for (int l = 0; l < n_staged; ++l) m += g.size[l];
    for (uint32_t i = threadIdx.x; i < (m + 1) / 2 * 2; i += blockDim.x) hash_tab[i] = i < m ? src[i] : 0u;
    __syncthreads();
    const GridTabLds tab{(const uint32_t NERF_LDS_PTR)hash_tab};
    const int64_t p0 = (int64_t)blockIdx.x * kHashLdsTile;
    const int64_t p1 = p0 + kHashLdsTile < n ? p0 + kHashLdsTile : n;
    const int L = g.n_levels;
    constexpr int NC = 1 << DIM;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        float u[DIM];
#pragma unroll
        for (int a = 0; a < DIM; ++a) u[a] = x[DIM * p + a];
        uint32_t lo = 0;
        for (int l = 0; l < n_staged; l += 2) {
            const int nl = l + 1 < n_staged ? 2 : 1;
            float f[4] = {0.f, 0.f, 0.f, 0.f};
            for (int j = 0; j < nl; ++j) {
                if (g.mask[l + j] != 0.0f) {
                    GridLookup<DIM> q;
                    q.issue(tab, lo, g.res[l + j], true, g.tmask, u);
                    q.finish(g.mask[l + j], f[2 * j], f[2 * j + 1], idx_dbg ? idx_dbg + NC * (p * L + l + j) : nullptr);
                }
                lo += g.size[l + j];
            }
            store_levels(out, p, L, l, nl, f);
        }
    }
}

template <int DIM>
__global__ void __launch_bounds__(256) k_encode_hash(const float* __restrict__ x, int64_t n, GridArgs g, int l_first,
                                                     int tiles, float* __restrict__ out,
                                                     uint32_t* __restrict__ idx_dbg) {
    const int l = l_first + (int)(blockIdx.x / tiles) * kHashLpi;
    const int nl = g.n_levels - l < kHashLpi ? g.n_levels - l : kHashLpi;
    const int64_t p0 = (int64_t)(blockIdx.x % tiles) * (256 * kHashPts);
    const int L = g.n_levels;
    constexpr int NC = 1 << DIM;
    const GridTabGlobal tab(g);
    // (the points are read first: a later read would wait for every lookup)
    float u[kHashPts][DIM];
#pragma unroll
    for (int j = 0; j < kHashPts; ++j) {
        int64_t p = p0 + j * 256 + threadIdx.x;
        p = p < n ? p : n - 1;
#pragma unroll
        for (int a = 0; a < DIM; ++a) u[j][a] = x[DIM * p + a];
    }
    // every lookup of the thread (points past the end repeat the last point,
    // a missing second level repeats the first) is issued before any finishes;
    // a level with mask 0 is skipped (the mask is uniform over the workgroup)
    bool look[kHashLpi];
#pragma unroll
    for (int k = 0; k < kHashLpi; ++k) look[k] = k < nl && g.mask[l + k] != 0.0f;
    GridLookup<DIM> q[kHashPts][kHashLpi];
#pragma unroll
    for (int j = 0; j < kHashPts; ++j)
#pragma unroll
        for (int k = 0; k < kHashLpi; ++k) {
            const int lk = k < nl ? l + k : l;
            if (look[k]) q[j][k].issue(tab, (uint32_t)g.offset[lk], g.res[lk], g.direct[lk] != 0, g.tmask, u[j]);
        }
#pragma unroll
    for (int j = 0; j < kHashPts; ++j) {
        const int64_t p = p0 + j * 256 + threadIdx.x;
        if (p < n) {
            float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < kHashLpi; ++k)
                if (look[k])
                    q[j][k].finish(g.mask[l + k], f[2 * k], f[2 * k + 1],
                                   idx_dbg ? idx_dbg + NC * (p * L + l + k) : nullptr);
            store_levels(out, p, L, l, kHashLpi < 2 ? 1 : nl, f);
        }
    }
}

template <int DIM>
static void launch_encode_hash_t(const float* x, int64_t n, const GridArgs& g, float* out, uint32_t* idx,
                                 hipStream_t s) {
    // levels are in increasing resolution: the staged ones are a prefix of
    // direct levels whose tables fit LDS together
    int n_staged = 0;
    size_t lds_bytes = 0;
    while (n_staged < g.n_levels && g.direct[n_staged] &&
           lds_bytes + (size_t)g.size[n_staged] * 4 + 8 <= (size_t)kHashLdsMax) {
        lds_bytes += (size_t)g.size[n_staged] * 4;
        ++n_staged;
    }
    lds_bytes = (lds_bytes + 7) / 8 * 8;  // whole 8-byte words
    if (n_staged > 0)
        hipLaunchKernelGGL(k_encode_hash_lds<DIM>, dim3((unsigned)((n + kHashLdsTile - 1) / kHashLdsTile)),
                           dim3(1024), lds_bytes, s, x, n, g, n_staged, out, idx);
    if (n_staged < g.n_levels) {
        const int tiles = (int)((n + 256 * kHashPts - 1) / (256 * kHashPts));
        const int items = (g.n_levels - n_staged + kHashLpi - 1) / kHashLpi;
        hipLaunchKernelGGL(k_encode_hash<DIM>, dim3((unsigned)((int64_t)tiles * items)), dim3(256), 0, s, x, n, g,
                           n_staged, tiles, out, idx);
    }
}

void launch_encode_hash(const float* x, int64_t n, const GridArgs& g, float* out, uint32_t* idx, hipStream_t s) {
    if (g.dim == 2)
        launch_encode_hash_t<2>(x, n, g, out, idx, s);
    else
        launch_encode_hash_t<3>(x, n, g, out, idx, s);
}

// ===========================================================================
// Standalone compositing ("Spatial Intelligence - Part 1: NeRF", Section 1
// Theory, 3. Volume rendering; Section 2 Code, 5. Volume rendering): 16
// lanes per ray (one DPP row), 4 rays per wave.  A 64-sample chunk is four
// rounds of 16 consecutive samples, one per lane, so every access of a row
// is contiguous; each round's exclusive product scan of the survival
// factors over the row, times the product of all earlier rounds, gives the
// samples' transmittance.
// ===========================================================================
constexpr int kCompLanes = 16;  // one DPP row

// Lane i of a 16-lane row reads lane i - N of the row; the first N lanes get
// fill.
template <int N>
__device__ __forceinline__ float row_shr(float v, float fill) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                                 __builtin_bit_cast(int, v), 0x110 | N, 0xF, 0xF,
                                                                 false));
}

// e^x from the hardware base-2 exponential, and the logistic function with
// the hardware reciprocal (relative errors near 1e-6 for the arguments met
// here).
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float sigmoid_hw(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_hw(-x)); }

__global__ void __launch_bounds__(256) k_composite(const float* __restrict__ raw, const float* __restrict__ z,
                                                   const float* __restrict__ rd, int64_t n_rays, int n, int white,
                                                   float* __restrict__ rgb, float* __restrict__ depth,
                                                   float* __restrict__ acc, float* __restrict__ wout) {
    constexpr int G = kCompLanes;
    const int g = lane_id() & (G - 1);
    const int64_t r0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / G;
    const bool ray_ok = r0 < n_rays;  // past the end: repeat the last ray, store nothing
    const int64_t r = ray_ok ? r0 : n_rays - 1;
    const float dx = rd[3 * r], dy = rd[3 * r + 1], dz = rd[3 * r + 2];
    const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
    const float* zr = z + r * n;
    const f32x4* rr = reinterpret_cast<const f32x4*>(raw) + r * n;
    float* wr = wout ? wout + r * n : nullptr;
    float carry = 1.0f, sr = 0.f, sg = 0.f, sbl = 0.f, sd = 0.f, sa = 0.f;
    for (int c0 = 0; c0 < n; c0 += 4 * G) {
        // lane g takes samples c0 + 16i + g: every load and store of the row is contiguous
        float zi[4], al[4], sv[4], incl[4], tot[4];
        f32x4 rw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = c0 + G * i + g;
            al[i] = 0.0f;
            zi[i] = 0.0f;
            rw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s < n) {
                zi[i] = zr[s];
                const float delta = (s + 1 < n) ? (zr[s + 1] - zi[i]) * dn : 1e10f * dn;
                rw[i] = rr[s];
                al[i] = 1.0f - exp_hw(-fmaxf(rw[i][3], 0.0f) * delta);
            }
            sv[i] = s < n ? (1.0f - al[i] + 1e-10f) : 1.0f;
            float p = sv[i];
            p *= row_shr<1>(p, 1.0f);
            p *= row_shr<2>(p, 1.0f);
            p *= row_shr<4>(p, 1.0f);
            p *= row_shr<8>(p, 1.0f);
            incl[i] = p;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = __shfl(incl[i], G - 1, G);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = c0 + G * i + g;
            const float T = row_shr<1>(incl[i], 1.0f) * carry;
            if (s < n) {
                const float w = T * al[i];
                if (wr && ray_ok) wr[s] = w;
                sa += w;
                sd += w * zi[i];
                sr += w * sigmoid_hw(rw[i][0]);
                sg += w * sigmoid_hw(rw[i][1]);
                sbl += w * sigmoid_hw(rw[i][2]);
            }
            carry *= tot[i];
        }
    }
    // row sums, complete in the row's last lane
    sr += row_shr<1>(sr, 0.f), sg += row_shr<1>(sg, 0.f), sbl += row_shr<1>(sbl, 0.f), sd += row_shr<1>(sd, 0.f),
        sa += row_shr<1>(sa, 0.f);
    sr += row_shr<2>(sr, 0.f), sg += row_shr<2>(sg, 0.f), sbl += row_shr<2>(sbl, 0.f), sd += row_shr<2>(sd, 0.f),
        sa += row_shr<2>(sa, 0.f);
    sr += row_shr<4>(sr, 0.f), sg += row_shr<4>(sg, 0.f), sbl += row_shr<4>(sbl, 0.f), sd += row_shr<4>(sd, 0.f),
        sa += row_shr<4>(sa, 0.f);
    sr += row_shr<8>(sr, 0.f), sg += row_shr<8>(sg, 0.f), sbl += row_shr<8>(sbl, 0.f), sd += row_shr<8>(sd, 0.f),
        sa += row_shr<8>(sa, 0.f);
    if (g == G - 1 && ray_ok) {
        const float bg = white ? 1.0f - sa : 0.0f;
        rgb[3 * r] = sr + bg;
        rgb[3 * r + 1] = sg + bg;
        rgb[3 * r + 2] = sbl + bg;
        depth[r] = sd;
        acc[r] = sa;
    }
}

void launch_composite(const float* raw, const float* z, const float* rd, int64_t n_rays, int n, int white, float* rgb,
                      float* depth, float* acc, float* w, hipStream_t s) {
    const int64_t rays_per_block = 256 / kCompLanes;
    hipLaunchKernelGGL(k_composite, dim3((unsigned)((n_rays + rays_per_block - 1) / rays_per_block)), dim3(256), 0,
                       s, raw, z, rd, n_rays, n, white, rgb, depth, acc, w);
}

// ===========================================================================
// Standalone inverse-CDF resampling + merge: one wave per ray, per-wave LDS.
// ===========================================================================
constexpr int kMaxSamples = 256;

struct PdfLds {
    double cdf[kMaxSamples];
    float bins[kMaxSamples];
    float u[kMaxSamples];  // coarse samples followed by fine samples
    float w[kMaxSamples];
};

__global__ void __launch_bounds__(256) k_sample_pdf(const float* __restrict__ zc, const float* __restrict__ wc,
                                                    int64_t n_rays, int nc, int nf, uint64_t seed,
                                                    uint64_t ray_offset, float* __restrict__ zf_out,
                                                    int32_t* __restrict__ bin_out, float* __restrict__ z2_out) {
    __shared__ PdfLds lds_all[4];
    const int wave = threadIdx.x / kWave;
    PdfLds& L = lds_all[wave];
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= n_rays) return;
    const int lane = lane_id();
    for (int k = lane; k < nc; k += kWave) {
        L.u[k] = zc[r * nc + k];
        L.w[k] = wc[r * nc + k];
    }
    wave_lds_sync();
    sample_pdf_ray(L.u, L.w, nc, nf, seed, ray_offset + (uint64_t)r, L.bins, L.cdf, L.u + nc,
                   bin_out ? bin_out + r * nf : nullptr);
    if (zf_out)
        for (int m = lane; m < nf; m += kWave) zf_out[r * nf + m] = L.u[nc + m];
    if (z2_out) merge_samples(L.u, nc, L.u + nc, nf, L.bins, z2_out + r * (nc + nf));
}

void launch_sample_pdf(const float* zc, const float* wc, int64_t n_rays, int nc, int nf, uint64_t seed,
                       uint64_t ray_offset, float* zf, int32_t* bins, float* z2, hipStream_t s) {
    hipLaunchKernelGGL(k_sample_pdf, dim3((unsigned)((n_rays + 3) / 4)), dim3(256), 0, s, zc, wc, n_rays, nc, nf,
                       seed, ray_offset, zf, bins, z2);
}

}  // namespace nerf

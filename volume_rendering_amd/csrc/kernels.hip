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
// Frequency encoding: one thread per (point, frequency) writes the in_dim
// sines and in_dim cosines of that frequency; frequency slot 0 of threads
// with include_input also copies the input.
// ===========================================================================
template <typename OutT>
__device__ __forceinline__ void put(OutT* p, float v);
template <>
__device__ __forceinline__ void put<float>(float* p, float v) {
    *p = v;
}
template <>
__device__ __forceinline__ void put<__bf16>(__bf16* p, float v) {
    *p = to_bf16(v);
}

template <typename OutT>
__global__ void __launch_bounds__(256) k_encode_freq(const float* __restrict__ x, int64_t n, int d, int L, int inc,
                                                     int use_pi, OutT* __restrict__ out) {
    const int per = L + (inc ? 1 : 0);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n * per) return;
    const int64_t p = t / per;
    const int q = (int)(t - p * per);
    const int width = d * (inc + 2 * L);
    OutT* o = out + p * width;
    const float* xp = x + p * d;
    if (inc && q == 0) {
        for (int a = 0; a < d; ++a) put(o + a, xp[a]);
        return;
    }
    const int k = q - (inc ? 1 : 0);
    OutT* ok = o + d * inc + 2 * d * k;
    for (int a = 0; a < d; ++a) {
        const float arg = ldexpf(xp[a], k);
        float sn, cs;
        if (use_pi)
            sincospif(arg, &sn, &cs);
        else
            sincosf(arg, &sn, &cs);
        put(ok + a, sn);
        put(ok + d + a, cs);
    }
}

void launch_encode_freq(const float* x, int64_t n, int d, int L, int inc, int use_pi, int bf16, void* out,
                        hipStream_t s) {
    const int64_t tot = n * (L + (inc ? 1 : 0));
    const dim3 g((unsigned)((tot + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(k_encode_freq<__bf16>, g, dim3(256), 0, s, x, n, d, L, inc, use_pi, (__bf16*)out);
    else
        hipLaunchKernelGGL(k_encode_freq<float>, g, dim3(256), 0, s, x, n, d, L, inc, use_pi, (float*)out);
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
// Hash-grid encoding: one thread per (point, level).
// ===========================================================================
__global__ void __launch_bounds__(256) k_encode_hash(const float* __restrict__ x, int64_t n, GridArgs g,
                                                     float* __restrict__ out, uint32_t* __restrict__ idx_dbg) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n * g.n_levels) return;
    const int64_t p = t / g.n_levels;
    const int l = (int)(t - p * g.n_levels);
    float f0, f1;
    grid_level(g, l, x[3 * p], x[3 * p + 1], x[3 * p + 2], f0, f1, idx_dbg ? idx_dbg + 8 * t : nullptr);
    reinterpret_cast<float2*>(out)[t] = make_float2(f0, f1);
}

void launch_encode_hash(const float* x, int64_t n, const GridArgs& g, float* out, uint32_t* idx, hipStream_t s) {
    const int64_t tot = n * g.n_levels;
    hipLaunchKernelGGL(k_encode_hash, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, x, n, g, out, idx);
}

// ===========================================================================
// Standalone compositing: one wave per ray.
// ===========================================================================
__global__ void __launch_bounds__(256) k_composite(const float* __restrict__ raw, const float* __restrict__ z,
                                                   const float* __restrict__ rd, int64_t n_rays, int n, int white,
                                                   float* __restrict__ rgb, float* __restrict__ depth,
                                                   float* __restrict__ acc, float* __restrict__ wout) {
    const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (r >= n_rays) return;
    const float dx = rd[3 * r], dy = rd[3 * r + 1], dz = rd[3 * r + 2];
    const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
    const CompositeOut o = composite_ray(z + r * n, reinterpret_cast<const f32x4*>(raw) + r * n, n, dn,
                                         wout ? wout + r * n : nullptr, 0.0f);
    if (lane_id() == 0) {
        const float bg = white ? 1.0f - o.acc : 0.0f;
        rgb[3 * r] = o.r + bg;
        rgb[3 * r + 1] = o.g + bg;
        rgb[3 * r + 2] = o.b + bg;
        depth[r] = o.depth;
        acc[r] = o.acc;
    }
}

void launch_composite(const float* raw, const float* z, const float* rd, int64_t n_rays, int n, int white, float* rgb,
                      float* depth, float* acc, float* w, hipStream_t s) {
    const int64_t waves_per_block = 4;
    hipLaunchKernelGGL(k_composite, dim3((unsigned)((n_rays + waves_per_block - 1) / waves_per_block)), dim3(256), 0,
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

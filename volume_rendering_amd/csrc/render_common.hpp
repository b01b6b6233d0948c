// Fused per-ray forward renders for gfx950: one wave renders one ray from
// its first sample to its composited colour; samples, encodings and
// activations stay in registers and the wave's LDS, nothing intermediate
// goes to HBM.
//
// NeRF mode ("Spatial Intelligence - Part 1: NeRF", Section 2 Code,
// 6. Hierarchical sampling, render_rays): stratified samples -> coarse
// network -> compositing -> inverse-CDF resampling + merge -> fine network
// -> compositing.  Both passes run through one copy of the network code (the
// pass index selects weights and the sample source).
//
// Hash mode: stratified samples -> hash-grid features and harmonics ->
// field network -> compositing.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "mlp.hpp"
#include "raysteps.hpp"

namespace nerf {

constexpr int kMaxRaySamples = 256;
#ifndef NERF_RENDER_RING
#define NERF_RENDER_RING 6
#endif
constexpr int kRenderRing = NERF_RENDER_RING;  // weight ring slots next to 40 KB of per-wave state

struct RenderLds {
    float zc[kMaxRaySamples];  // first-pass samples, then the fine samples (union for the merge)
    float z2[kMaxRaySamples];  // merged samples of the second pass
    f32x4 raw[kMaxRaySamples];
    float w[kMaxRaySamples];
    union {
        double cdf[kMaxRaySamples];  // resampling (between the passes)
        int live[kMaxRaySamples];    // live samples of the pass being evaluated
    };
    float bins[kMaxRaySamples];
};

// ---------------------------------------------------------------------------
// Empty-space skipping and early termination ("Spatial Intelligence - Part
// 1: NeRF", Section 1 Theory, 4.2: uniform samples waste compute on empty
// space).  A ray's live samples (inside the box, in an occupied voxel) are
// listed in order and evaluated in dense blocks; a skipped sample has
// density 0, i.e. alpha 0 and a survival factor 1 - 0 + 1e-10 that rounds
// to 1 in float32, so leaving it out changes no product.  After each block
// the transmittance so far is updated, and the ray stops evaluating once it
// is below term_T (with a 1e-4 relative margin, so every sample the
// compositor keeps has been evaluated).
// ---------------------------------------------------------------------------

// Ascending indices of the live samples among zp[0..N) into list; returns
// their number.
__device__ __forceinline__ int live_samples(const RenderArgs& a, const float* zp, int N, const float (&o)[3],
                                            const float (&d)[3], int* list) {
    const int lane = lane_id();
    const unsigned long long below = (1ull << lane) - 1ull;
    int n = 0;
    for (int base = 0; base < N; base += kWave) {
        const int i = base + lane;
        bool lv = false;
        if (i < N) {
            float x[3];
#pragma unroll
            for (int k = 0; k < 3; ++k) x[k] = __fadd_rn(o[k], __fmul_rn(zp[i], d[k]));
            lv = box_occupied(a.occ, a.occ_res, a.vscale, a.box_lo, a.box_hi, x);
        }
        const unsigned long long m = __ballot(lv);
        NERF_DCHECK(!lv || n + __popcll(m & below) < kMaxRaySamples, kCheckRaySample);
        if (lv) list[n + __popcll(m & below)] = i;
        n += __popcll(m);
    }
    wave_lds_sync();
    return n;
}

// Every wave of the workgroup calls this once per block iteration `it` (the
// weight ring makes the waves run the same number of network passes); true
// while any wave still has a block to evaluate.  One workgroup barrier; the
// flags alternate between two rows so a fast wave's next write cannot meet
// a slow wave's read.
__device__ __forceinline__ bool workgroup_busy(bool busy, int it, int wave, int (&flags)[2][4]) {
    if (lane_id() == 0) flags[it & 1][wave] = busy ? 1 : 0;
    __syncthreads();
    const int* f = flags[it & 1];
    return (f[0] | f[1] | f[2] | f[3]) != 0;
}

// Product of (1 - alpha + 1e-10) over the evaluated samples j0 .. j0+M-1 of
// the pass (sample indices from list, or j itself when list is NULL).
__device__ __forceinline__ float block_survival(const float* zp, const f32x4* raw, const int* list, int j0, int M,
                                                int n_eval, int N, float dn) {
    const int lane = lane_id();
    const int j = j0 + lane;
    float surv = 1.0f;
    if (lane < M && j < n_eval) {
        const int i = list ? list[j] : j;
        const float delta = (i + 1 < N) ? (zp[i + 1] - zp[i]) * dn : 1e10f * dn;
        const float alpha = 1.0f - expf(-fmaxf(raw[i][3], 0.0f) * delta);
        surv = 1.0f - alpha + 1e-10f;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) surv *= __shfl_xor(surv, off, kWave);
    return surv;
}

template <class T, int KIND>
__global__ void __launch_bounds__(256) k_render_nerf(RenderArgs a) {
    __shared__ RenderLds lds_all[4];
    using Fam = NerfFamily<KIND>;
    constexpr Layer L0 = net_layers(KIND)[0];
    constexpr Layer LD = net_layers(KIND)[Fam::D + 2];
    constexpr int ES = seg_steps(L0.s0, T::prec);
    constexpr int DS = seg_steps(LD.s1, T::prec);
    constexpr int SB = T::SB;
    constexpr int M = 32 * SB;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    RenderLds& S = lds_all[wave];
    // every wave runs the same passes (the weight ring is shared); a wave past
    // the last ray renders the last ray again and stores nothing
    const int64_t r0 = (int64_t)blockIdx.x * 4 + wave;
    const bool live = r0 < a.n_rays;
    const int64_t r = live ? r0 : a.n_rays - 1;
    const int lane = lane_id();
    const uint64_t ray = a.ray_offset + (uint64_t)r;

    const float o[3] = {a.ro[3 * r], a.ro[3 * r + 1], a.ro[3 * r + 2]};
    const float d[3] = {a.rd[3 * r], a.rd[3 * r + 1], a.rd[3 * r + 2]};
    const float near = a.tn[r], far = a.tf[r];
    const float dn = sqrtf(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);

    typename T::Op denc[DS][SB];
    {
        float v[SB][3];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
            for (int k = 0; k < 3; ++k) v[sb][k] = d[k] / dn;
        enc_operands<Fam::LDIR>(denc, v, a.use_pi != 0, lane);
    }

    const int nc = a.n_coarse, nf = a.n_fine;
    const int npass = nf > 0 ? 2 : 1;
    constexpr int NBF = BiasRegion<KIND, T::prec>::floats;
    __shared__ __attribute__((aligned(16))) float bias_lds[2][NBF];
    __shared__ int busy_flags[2][4];
    bias_to_lds<KIND, T::prec>((NERF_AS_LDS float*)bias_lds[0], (const char*)a.coarse, threadIdx.x, blockDim.x);
    if (npass == 2)
        bias_to_lds<KIND, T::prec>((NERF_AS_LDS float*)bias_lds[1], (const char*)a.fine, threadIdx.x, blockDim.x);
    __syncthreads();
    // skipping or termination: rays evaluate different numbers of blocks
    const bool dynamic = a.occ != nullptr || a.term_T > 0.0f;
    int it = 0;
    for (int pass = 0; pass < npass; ++pass) {
        const int N = pass ? nc + nf : nc;
        const char* packed = pass ? (const char*)a.fine : (const char*)a.coarse;
        float* zp = pass ? S.z2 : S.zc;
        if (pass == 0) {
            for (int i = lane; i < nc; i += kWave) {
                const float u = a.jitter ? philox_uniform(a.seed, ray, (uint32_t)i, kStreamJitter) : 0.5f;
                S.zc[i] = stratified_z(near, far, i, nc, u);
            }
            wave_lds_sync();
        }
        int n_eval = N;
        if (a.occ) {
            n_eval = live_samples(a, zp, N, o, d, S.live);
            if (a.n_live && live && lane == 0) atomicAdd((unsigned long long*)a.n_live, (unsigned long long)n_eval);
        }
        if (dynamic) {
            for (int i = lane; i < N; i += kWave) S.raw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            wave_lds_sync();
        }
        const int nb = (n_eval + M - 1) / M;
        float T_run = 1.0f;
        bool stop = false;
        for (int b = 0;; ++b) {
            if (dynamic) {
                if (!workgroup_busy(!stop && b < nb, it++, wave, busy_flags)) break;
            } else if (b >= nb) {
                break;
            }
            const bool idle = stop || b >= nb;  // an idle wave evaluates sample 0 and stores nothing
            float x[SB][3];
            int si[SB];
            bool valid[SB];
#pragma unroll
            for (int sb = 0; sb < SB; ++sb) {
                const int j = b * M + sb * 32 + (lane & 31);
                valid[sb] = !idle && j < n_eval;
                si[sb] = valid[sb] ? (a.occ ? S.live[j] : j) : 0;
                NERF_DCHECK(si[sb] >= 0 && si[sb] < N && N <= kMaxRaySamples, kCheckRaySample);
                const float z = zp[si[sb]];
#pragma unroll
                for (int k = 0; k < 3; ++k) x[sb][k] = __fadd_rn(o[k], __fmul_rn(z, d[k]));
            }
            typename T::Op enc[ES][SB];
            enc_operands<Fam::LPOS>(enc, x, a.use_pi != 0, lane);
            f32x16 sig[SB], rgb[SB];
            const char* pk = opaque(packed);
            if constexpr (kLoopedF32<T, KIND>) {
                nerf_forward_f32_loop<KIND>(enc, denc, pk, (const NERF_AS_LDS float*)bias_lds[pass], sig, rgb, lane);
            } else {
                LdsStream<T, KIND, kRenderRing> ws(pk, lane, wave);
                nerf_forward<T, KIND>(enc, denc, ws, (const NERF_AS_LDS float*)bias_lds[pass], sig, rgb, lane);
            }
            if (lane < 32) {
#pragma unroll
                for (int sb = 0; sb < SB; ++sb)
                    if (valid[sb]) S.raw[si[sb]] = f32x4{rgb[sb][0], rgb[sb][1], rgb[sb][2], sig[sb][0]};
            }
            if (a.term_T > 0.0f && !idle) {
                wave_lds_sync();
                T_run *= block_survival(zp, S.raw, a.occ ? S.live : nullptr, b * M, M, n_eval, N, dn);
                stop = T_run < a.term_T * 0.9999f;
            }
        }
        wave_lds_sync();
        const CompositeOut c = composite_ray(zp, S.raw, N, dn, pass == 0 ? S.w : nullptr, a.term_T);
        wave_lds_sync();
        if (pass == 0 && a.dbg_w && live)
            for (int i = lane; i < nc; i += kWave) a.dbg_w[r * nc + i] = S.w[i];
        if (pass == npass - 1) {
            if (a.dbg_z && live)
                for (int i = lane; i < N; i += kWave) a.dbg_z[r * N + i] = zp[i];
            if (lane == 0 && live) {
                const float bg = a.white ? 1.0f - c.acc : 0.0f;
                a.rgb[3 * r] = c.r + bg;
                a.rgb[3 * r + 1] = c.g + bg;
                a.rgb[3 * r + 2] = c.b + bg;
                a.depth[r] = c.depth;
                a.acc[r] = c.acc;
            }
        } else {
            sample_pdf_ray(S.zc, S.w, nc, nf, a.seed, ray, S.bins, S.cdf, S.zc + nc, nullptr);
            merge_samples(S.zc, nc, S.zc + nc, nf, S.bins, S.z2);
        }
    }
}

// ---------------------------------------------------------------------------
// Hash-grid field render
// ---------------------------------------------------------------------------
template <int NS>
__device__ __forceinline__ void grid_operands(bf16x8 (&op)[NS][2], const GridArgs& g, const float (&u)[2][3],
                                              int lane) {
    static_assert(NS == 2, "32 grid features");
    const int h = lane >> 5;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 v;
#pragma unroll
            for (int jl = 0; jl < 4; ++jl) {
                float f0, f1;
                grid_level(g, 8 * s + 4 * h + jl, u[sb][0], u[sb][1], u[sb][2], f0, f1, nullptr);
                v[2 * jl] = to_bf16(f0);
                v[2 * jl + 1] = to_bf16(f1);
            }
            op[s][sb] = v;
        }
}

template <int NS>
__device__ __forceinline__ void grid_operands(bf16x8 (&op)[NS][1], const GridArgs& g, const float (&u)[1][3],
                                              int lane) {
    static_assert(NS == 2, "32 grid features");
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        bf16x8 v;
#pragma unroll
        for (int jl = 0; jl < 4; ++jl) {
            float f0, f1;
            grid_level(g, 8 * s + 4 * h + jl, u[0][0], u[0][1], u[0][2], f0, f1, nullptr);
            v[2 * jl] = to_bf16(f0);
            v[2 * jl + 1] = to_bf16(f1);
        }
        op[s][0] = v;
    }
}

template <int NS>
__device__ __forceinline__ void grid_operands(float (&op)[NS][1], const GridArgs& g, const float (&u)[1][3],
                                              int lane) {
    static_assert(NS == 16, "32 grid features");
    const int h = lane >> 5;
    float f0[8], f1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) grid_level(g, 8 * h + q, u[0][0], u[0][1], u[0][2], f0[q], f1[q], nullptr);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        // step s needs feature 2s+h = level s, component h; levels 8h..8h+7 are this lane's
        const float send = h ? f0[s % 8] : f1[s % 8];
        const float recv = __shfl_xor(send, 32, kWave);
        const float mine = h ? f1[s % 8] : f0[s % 8];
        op[s][0] = (s / 8 == h) ? mine : recv;
    }
}

template <int NS>
__device__ __forceinline__ void sh_operands(bf16x8 (&op)[NS][2], const float (&sh)[16], int lane) {
    const int h = lane >> 5;
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_bf16(h ? sh[8 + j] : sh[j]);
    op[0][0] = v;
    op[0][1] = v;
}

template <int NS>
__device__ __forceinline__ void sh_operands(bf16x8 (&op)[NS][1], const float (&sh)[16], int lane) {
    const int h = lane >> 5;
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_bf16(h ? sh[8 + j] : sh[j]);
    op[0][0] = v;
}

template <int NS>
__device__ __forceinline__ void sh_operands(float (&op)[NS][1], const float (&sh)[16], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) op[s][0] = h ? sh[2 * s + 1] : sh[2 * s];
}

// One sample block per wave (TBF16S1) halves the registers so that two
// workgroups share a CU: the table gathers of one wave then overlap the
// vector and matrix work of another.  The weight ring is two slots deep to
// fit two workgroups' LDS.
template <class T>
constexpr int kHashRenderGroupsPerCu = T::SB == 1 && T::prec == PREC_BF16 ? 2 : 1;
template <class T>
constexpr int kHashRenderRing = kHashRenderGroupsPerCu<T> == 2 ? 2 : kRenderRing;

template <class T>
__global__ void __launch_bounds__(256, kHashRenderGroupsPerCu<T>) k_render_hash(RenderArgs a, GridArgs g) {
    __shared__ RenderLds lds_all[4];
    constexpr int K = NET_HASH_FIELD;
    constexpr int FS = seg_steps(net_layers(K)[0].s0, T::prec);
    constexpr int DS = seg_steps(net_layers(K)[4].s1, T::prec);
    constexpr int SB = T::SB;
    constexpr int M = 32 * SB;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    RenderLds& S = lds_all[wave];
    const int64_t r0 = (int64_t)blockIdx.x * 4 + wave;
    const bool live = r0 < a.n_rays;
    const int64_t r = live ? r0 : a.n_rays - 1;
    const int lane = lane_id();
    const uint64_t ray = a.ray_offset + (uint64_t)r;
    const float o[3] = {a.ro[3 * r], a.ro[3 * r + 1], a.ro[3 * r + 2]};
    const float d[3] = {a.rd[3 * r], a.rd[3 * r + 1], a.rd[3 * r + 2]};
    const float near = a.tn[r], far = a.tf[r];
    const float dn = sqrtf(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    const float lo = a.box_lo, span = __fsub_rn(a.box_hi, a.box_lo);

    typename T::Op shop[DS][SB];
    {
        float sh[16];
        sh16_eval(d[0] / dn, d[1] / dn, d[2] / dn, sh);
        sh_operands(shop, sh, lane);
    }
    __shared__ __attribute__((aligned(16))) float bias_lds[BiasRegion<NET_HASH_FIELD, T::prec>::floats];
    __shared__ int busy_flags[2][4];
    bias_to_lds<NET_HASH_FIELD, T::prec>((NERF_AS_LDS float*)bias_lds, (const char*)a.coarse, threadIdx.x, blockDim.x);
    __syncthreads();
    const int N = a.n_coarse;
    for (int i = lane; i < N; i += kWave) {
        const float uj = a.jitter ? philox_uniform(a.seed, ray, (uint32_t)i, kStreamJitter) : 0.5f;
        S.zc[i] = stratified_z(near, far, i, N, uj);
    }
    wave_lds_sync();
    const bool dynamic = a.occ != nullptr || a.term_T > 0.0f;
    int n_eval = N;
    if (a.occ) {
        n_eval = live_samples(a, S.zc, N, o, d, S.live);
        if (a.n_live && live && lane == 0) atomicAdd((unsigned long long*)a.n_live, (unsigned long long)n_eval);
    }
    if (dynamic) {
        for (int i = lane; i < N; i += kWave) S.raw[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        wave_lds_sync();
    }
    const int nb = (n_eval + M - 1) / M;
    float T_run = 1.0f;
    bool stop = false;
    for (int b = 0;; ++b) {
        if (dynamic) {
            if (!workgroup_busy(!stop && b < nb, b, wave, busy_flags)) break;
        } else if (b >= nb) {
            break;
        }
        const bool idle = stop || b >= nb;
        float u[SB][3];
        int si[SB];
        bool valid[SB];
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            const int j = b * M + sb * 32 + (lane & 31);
            valid[sb] = !idle && j < n_eval;
            si[sb] = valid[sb] ? (a.occ ? S.live[j] : j) : 0;
            const float z = S.zc[si[sb]];
#pragma unroll
            for (int k = 0; k < 3; ++k)
                u[sb][k] = __fdiv_rn(__fsub_rn(__fadd_rn(o[k], __fmul_rn(z, d[k])), lo), span);
        }
        typename T::Op feats[FS][SB];
        grid_operands(feats, g, u, lane);
        f32x16 sig[SB], rgb[SB];
        const char* pk = opaque((const char*)a.coarse);
        LdsStream<T, NET_HASH_FIELD, kHashRenderRing<T>> ws(pk, lane, wave);
        hash_field_forward<T>(feats, shop, ws, (const NERF_AS_LDS float*)bias_lds, sig, rgb, lane);
        if (lane < 32) {
#pragma unroll
            for (int sb = 0; sb < SB; ++sb)
                if (valid[sb]) S.raw[si[sb]] = f32x4{rgb[sb][0], rgb[sb][1], rgb[sb][2], sig[sb][0]};
        }
        if (a.term_T > 0.0f && !idle) {
            wave_lds_sync();
            T_run *= block_survival(S.zc, S.raw, a.occ ? S.live : nullptr, b * M, M, n_eval, N, dn);
            stop = T_run < a.term_T * 0.9999f;
        }
    }
    wave_lds_sync();
    const CompositeOut c = composite_ray(S.zc, S.raw, N, dn, nullptr, a.term_T);
    if (a.dbg_z && live)
        for (int i = lane; i < N; i += kWave) a.dbg_z[r * N + i] = S.zc[i];
    if (lane == 0 && live) {
        const float bg = a.white ? 1.0f - c.acc : 0.0f;
        a.rgb[3 * r] = c.r + bg;
        a.rgb[3 * r + 1] = c.g + bg;
        a.rgb[3 * r + 2] = c.b + bg;
        a.depth[r] = c.depth;
        a.acc[r] = c.acc;
    }
}

}  // namespace nerf

// One training step of the hash-grid INR for gfx950 ("Instant-NGP - Visual
// Experiments (a 2D multiresolution hash grid)", shared toolkit: HashGrid2D,
// HashINR, train; Experiment 2): multiresolution lookups into learnable
// float32 tables, a decoder with one hidden ReLU layer, the mean squared
// error, the gradient of every table entry and decoder parameter, Adam.
//
// Parameters are one flat float32 vector: the tables (levels back to back,
// two features per entry), then W1 [hidden][2L], b1, W2 [n_out][hidden], b2.
//
// Gradients are carried in units of the output residual y - target and
// scaled by 2/(n n_out) (the derivative of the mean) only at the end.
//
//   k_inr_pad      the decoder zero-padded to the kernel's tile sizes
//   k_inr_decode   one thread per point (consecutive points on consecutive
//                  lanes): lookups, decoder forward and backward (padded
//                  weights by uniform scalar loads), the feature gradient of
//                  every level out to HBM (level-major), and the decoder
//                  gradient -- W1, b1 and W2 as fp32 MFMA contractions over the
//                  wave's points (staged through LDS 16 at a time), b2 and the
//                  squared error per lane -- summed per workgroup in wave order
//   k_inr_scatter  one workgroup per (level, range of at most 4096 entries,
//                  chunk of points): the chunk's feature gradients spread over
//                  their corners' entries (runs of consecutive points per
//                  thread, a corner's sum held in registers while its entry
//                  stays the same), accumulated in LDS as 64-bit fixed
//                  point (integer LDS atomics are some thirty times faster than
//                  float ones here, and integer sums do not depend on the
//                  order of the additions), one partial per chunk out; levels
//                  too large for a few ranges accumulate with global float
//                  atomics instead
//   k_inr_post     per parameter: the partials summed in chunk order, scaled,
//                  the gradient out, Adam; the loss from the squared errors
//
// Multiply-adds are fused (fmaf): single rounding, as close to the exact
// definition as float32 gets.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "inr_plan.hpp"
#include "launch.hpp"
#include "optim.hpp"
#include "raysteps.hpp"

namespace nerf {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct InrStep {
    int64_t tab_floats;     // all table floats
    int64_t lds_tab_floats; // table floats of the levels scattered through LDS (a prefix)
    int lds_levels;         // those levels
    int iters;              // points per thread of the decoder kernel
    int part_w;             // floats per decoder partial
    int64_t scat_chunk;     // points per scatter chunk (a multiple of 4 per thread)
    int scat_chunks;
    int scat_jobs;
    int64_t dstride;        // points per level slice of dfeat (n rounded up to even)
    float* dfeat;           // [L][dstride][2]: feature gradients (residual units)
    float* part_dec;        // [decode groups][part_w]
    float* part_tab;        // [scatter chunks][lds_tab_floats]
    float* grad;            // flat gradient (the global-atomic levels accumulate here)
    float dy_scale;         // 2 / (n n_out)
};

// Padded decoder: one row of RW = FM + 8 floats per hidden unit j (W1[j][0..FM),
// b1[j], W2[0..3][j], 3 zeros), then b2[0..3] and 4 zeros, then W1 transposed
// ([FM][HM], for the per-level feature gradient), then W2 ([4][HM], for the
// outputs); zeros outside the real sizes.
__global__ void __launch_bounds__(256) k_inr_pad(const float* __restrict__ dec, int H, int F, int O, int HM, int FM,
                                                 float* __restrict__ wp) {
    const float* W1 = dec;
    const float* b1 = W1 + H * F;
    const float* W2 = b1 + H;
    const float* b2 = W2 + O * H;
    const int RW = FM + 8;
    const int n = HM * RW + 8 + FM * HM + 4 * HM;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        float v = 0.0f;
        if (i < HM * RW) {
            const int j = i / RW, c = i % RW;
            if (j < H) {
                if (c < FM)
                    v = c < F ? W1[j * F + c] : 0.0f;
                else if (c == FM)
                    v = b1[j];
                else if (c - FM - 1 < O)
                    v = W2[(c - FM - 1) * H + j];
            }
        } else if (i < HM * RW + 8) {
            const int o = i - HM * RW;
            if (o < O) v = b2[o];
        } else if (i < HM * RW + 8 + FM * HM) {
            const int k = (i - HM * RW - 8) / HM, j = (i - HM * RW - 8) % HM;
            if (j < H && k < F) v = W1[j * F + k];
        } else {
            const int o = (i - HM * RW - 8 - FM * HM) / HM, j = (i - HM * RW - 8 - FM * HM) % HM;
            if (j < H && o < O) v = W2[o * H + j];
        }
        wp[i] = v;
    }
}

// One level's parameters, read where they are used through an opaque index
// (derived per-level values kept for every level through the point loop
// would not fit in SGPRs).
struct Level {
    int N;
    uint32_t off;
    bool direct;
    float mask;
};
__device__ __forceinline__ Level level_params(const GridArgs& g, int l) {
    int li = l;
    asm volatile("" : "+s"(li));
    return Level{g.res[li], (uint32_t)g.offset[li], g.direct[li] != 0, g.mask[li]};
}

// b^e in 32 bits (the entries of a direct level: (N+1)^DIM).
__device__ __forceinline__ uint32_t ipow_u32(int b, int e) {
    uint32_t r = 1u;
    for (int i = 0; i < e; ++i) r *= (uint32_t)b;
    return r;
}

// A level at point u: the 2^DIM corners' absolute table entries and
// multilinear weights (cell c = u N in float32, corners clamped to [0, N],
// corner bits lexicographic, first axis most significant).
template <int DIM>
__device__ __forceinline__ void level_corners(const Level& lv, uint32_t tmask, const float (&u)[DIM],
                                              uint32_t (&e)[1 << DIM], float (&wt)[1 << DIM]) {
    const int N = lv.N;
    int c0[DIM];
    float fr[DIM];
#pragma unroll
    for (int k = 0; k < DIM; ++k) {
        const float c = __fmul_rn(u[k], (float)N);
        const float f = floorf(c);
        fr[k] = c - f;
        c0[k] = (int)f;
    }
#pragma unroll
    for (int q = 0; q < (1 << DIM); ++q) {
        int ci[DIM];
        float wq = 1.0f;
#pragma unroll
        for (int k = 0; k < DIM; ++k) {
            const int bit = (q >> (DIM - 1 - k)) & 1;
            ci[k] = min(max(c0[k] + bit, 0), N);
            wq *= bit ? fr[k] : 1.0f - fr[k];
        }
        // both indexings, then a select: no branch per corner
        uint32_t idx_d, idx_h;
        if constexpr (DIM == 3) {
            idx_d = grid_index(ci[0], ci[1], ci[2], N, true, tmask);
            idx_h = grid_index(ci[0], ci[1], ci[2], N, false, tmask);
        } else {
            idx_d = grid_index(ci[0], ci[1], N, true, tmask);
            idx_h = grid_index(ci[0], ci[1], N, false, tmask);
        }
        NERF_DCHECK(lv.direct ? idx_d < ipow_u32(N + 1, DIM) : idx_h <= tmask, kCheckGridIndex);
        e[q] = lv.off + (lv.direct ? idx_d : idx_h);
        wt[q] = wq;
    }
}

// One padded decoder row (uniform address: scalar loads).
template <int RW>
__device__ __forceinline__ void load_row(const float* src, float (&dst)[RW]) {
#pragma unroll
    for (int c = 0; c < RW; ++c) dst[c] = src[c];
}

// Sum over the wave, the same value in every lane (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Orders the wave's LDS accesses around a hand-over between its lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DIM, int HM, int FM>
__global__ void __launch_bounds__(kInrThreads) k_inr_decode(GridArgs g, HashInrArgs a, InrStep f,
                                                            const float* __restrict__ wp) {
    // staged point: dpre | h | feat | dy[0..3], 1, 0 ... (16), padded to a
    // stride of 20 banks mod 32 (16-byte row writes of 8 lanes cover every
    // bank; the operand reads of 4 rows x 16 columns meet at most 2-way)
    constexpr int SW = inr_stage_width(HM, FM);
    constexpr int LM = FM / 2;
    constexpr int HT = HM / 16, FT = FM / 16;
    constexpr int RW = FM + 8;  // padded decoder row
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* stage = lds + wave * (kInrStageRows * SW);

    // C[j][k] over the wave's points: dpre[j] feat[k] (W1), h[j] dy[k] (W2),
    // dpre[j] [dy, 1][k] (b1 in column 4)
    f32x4 cw1[HT][FT], cw2[HT], cb1[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        cw2[t] = cb1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < FT; ++u) cw1[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float db2[4], sq = 0.0f;
#pragma unroll
    for (int o = 0; o < 4; ++o) db2[o] = 0.0f;

    for (int it = 0; it < f.iters; ++it) {
        const int64_t p = ((int64_t)blockIdx.x * f.iters + it) * kInrThreads + tid;
        const bool live = p < a.n;
        // the padded decoder is read by uniform (scalar) loads -- from LDS
        // every broadcast read would still return 64 lanes of data -- one row
        // at a time as each pass uses it; a scheduling fence after each row
        // keeps the other rows' loads out, and opaque offsets keep them from
        // being hoisted out of the point loop or shared between passes (any
        // of which would hold the decoder in SGPRs, more than there are)
        int foff = 0, boff = 0;
        asm volatile("" : "+s"(foff), "+s"(boff));
        const float* wf = wp + foff;
        const float* wb = wp + boff;
        // per-iteration copies of the level and output counts: the
        // comparisons against them are then made where they are used, not
        // kept for every level and output as lane masks in SGPRs
        int L = g.n_levels, O = a.n_out;
        asm volatile("" : "+s"(L), "+s"(O));
        float feat[FM], h[HM], dpre[HM], dy[4];
#pragma unroll
        for (int k = 0; k < FM; ++k) feat[k] = 0.0f;
#pragma unroll
        for (int j = 0; j < HM; ++j) h[j] = dpre[j] = 0.0f;
#pragma unroll
        for (int o = 0; o < 4; ++o) dy[o] = 0.0f;
        if (live) {
            float u[DIM];
#pragma unroll
            for (int k = 0; k < DIM; ++k) u[k] = a.x[p * DIM + k];
            // lookups
#pragma unroll
            for (int l = 0; l < LM; ++l) {
                if (l >= L) continue;
                const Level lv = level_params(g, l);
                uint32_t e[1 << DIM];
                float wt[1 << DIM];
                level_corners<DIM>(lv, g.tmask, u, e, wt);
                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int q = 0; q < (1 << DIM); ++q) {
                    const float2 v = *reinterpret_cast<const float2*>(a.params + 2 * (size_t)e[q]);
                    a0 = fmaf(wt[q], v.x, a0);
                    a1 = fmaf(wt[q], v.y, a1);
                }
                feat[2 * l] = lv.mask * a0;
                feat[2 * l + 1] = lv.mask * a1;
            }
            // decoder forward: the hidden units row by row, then the outputs
            // (each pass over uniform data of its own, so that no weight
            // waits in registers for a later use)
#pragma unroll
            for (int j = 0; j < HM; ++j) {
                float w[FM + 1];
                load_row<FM + 1>(wf + j * RW, w);
                float s = w[FM];
#pragma unroll
                for (int k = 0; k < FM; ++k) s = fmaf(w[k], feat[k], s);
                h[j] = fmaxf(s, 0.0f);
                __builtin_amdgcn_sched_barrier(0);
            }
            float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                if (o >= O) break;  // uniform
                const float* w2 = wf + HM * RW + 8 + FM * HM + o * HM;
                float s = wf[HM * RW + o];
#pragma unroll
                for (int j = 0; j < HM; ++j) s = fmaf(w2[j], h[j], s);
                y[o] = s;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                if (o >= O) continue;
                const float d = y[o] - a.target[p * O + o];
                sq = fmaf(d, d, sq);
                dy[o] = d;
                if (a.pred) a.pred[p * O + o] = y[o];
                db2[o] += d;
            }
            // decoder backward: the hidden pre-activation gradient (zero where
            // the ReLU output is zero), output by output from W2's rows
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                if (o >= O) break;  // uniform
                const float* w2 = wb + HM * RW + 8 + FM * HM + o * HM;
#pragma unroll
                for (int j = 0; j < HM; ++j) dpre[j] = fmaf(dy[o], w2[j], dpre[j]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < HM; ++j) dpre[j] = h[j] > 0.0f ? dpre[j] : 0.0f;
            // each level's feature gradient (dpre against two columns of W1),
            // out to the level's slice; a loop that is not unrolled keeps one
            // level's values live at a time
#pragma unroll 1
            for (int l = 0; l < L; ++l) {
                const Level lv = level_params(g, l);
                const float* c0 = wb + HM * RW + 8 + (2 * l) * HM;  // W1 columns 2l, 2l+1
                float df0 = 0.0f, df1 = 0.0f;
#pragma unroll
                for (int j = 0; j < HM; ++j) {
                    df0 = fmaf(dpre[j], c0[j], df0);
                    df1 = fmaf(dpre[j], c0[HM + j], df1);
                }
                *reinterpret_cast<float2*>(f.dfeat + 2 * ((size_t)l * f.dstride + p)) =
                    make_float2(lv.mask * df0, lv.mask * df1);
            }
        }
        // the decoder products, 16 points per round, 4 per MFMA (16x16x4:
        // operand lane m + 16 kk holds row m of point kk)
#pragma unroll
        for (int r = 0; r < 64 / kInrStageRows; ++r) {
            if ((lane >> 4) == r) {
                float* row = stage + (lane & 15) * SW;
#pragma unroll
                for (int j = 0; j < HM; j += 4) {
                    *reinterpret_cast<f32x4*>(row + j) = f32x4{dpre[j], dpre[j + 1], dpre[j + 2], dpre[j + 3]};
                    *reinterpret_cast<f32x4*>(row + HM + j) = f32x4{h[j], h[j + 1], h[j + 2], h[j + 3]};
                }
#pragma unroll
                for (int k = 0; k < FM; k += 4)
                    *reinterpret_cast<f32x4*>(row + 2 * HM + k) = f32x4{feat[k], feat[k + 1], feat[k + 2], feat[k + 3]};
                *reinterpret_cast<f32x4*>(row + 2 * HM + FM) = f32x4{dy[0], dy[1], dy[2], dy[3]};
                *reinterpret_cast<f32x4*>(row + 2 * HM + FM + 4) = f32x4{live ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 8; k < 16; k += 4)
                    *reinterpret_cast<f32x4*>(row + 2 * HM + FM + k) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            wave_sync();
#pragma unroll
            for (int s4 = 0; s4 < kInrStageRows / 4; ++s4) {
                const float* row = stage + (4 * s4 + (lane >> 4)) * SW;
                const int c = lane & 15;
                const float by = row[2 * HM + FM + c];
                float bf[FT];
#pragma unroll
                for (int uu = 0; uu < FT; ++uu) bf[uu] = row[2 * HM + 16 * uu + c];
#pragma unroll
                for (int t = 0; t < HT; ++t) {
                    const float ad = row[16 * t + c], ah = row[HM + 16 * t + c];
#pragma unroll
                    for (int uu = 0; uu < FT; ++uu)
                        cw1[t][uu] = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, bf[uu], cw1[t][uu], 0, 0, 0);
                    cw2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ah, by, cw2[t], 0, 0, 0);
                    cb1[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, by, cb1[t], 0, 0, 0);
                }
            }
            wave_sync();
        }
    }

    const int F = 2 * g.n_levels, H = a.hidden, O = a.n_out;
    // the wave's partial, into its own staging slice (which holds it: pm < 16
    // SW): W1, b1, W2, b2 gradients, then the squared-error sum (accumulator
    // lane n + 16 (m/4), register m%4 holds C[m][n])
    float* part = stage;
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int j = 16 * t + 4 * (lane >> 4) + rr, n = lane & 15;
#pragma unroll
            for (int uu = 0; uu < FT; ++uu)
                if (j < H && 16 * uu + n < F) part[j * F + 16 * uu + n] = cw1[t][uu][rr];
            if (j < H && n < O) part[H * F + H + n * H + j] = cw2[t][rr];
            if (j < H && n == 4) part[H * F + j] = cb1[t][rr];
        }
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        const float s = wave_sum(db2[o]);
        if (o < O && lane == o) part[H * F + H + O * H + o] = s;
    }
    const float sqs = wave_sum(sq);
    if (lane == 0) part[H * F + H + O * H + O] = sqs;

    // the workgroup's partial: the waves' in wave order
    __syncthreads();
    const int pm = H * F + H + O * H + O;
    float* pd = f.part_dec + (size_t)blockIdx.x * f.part_w;
    for (int i = tid; i <= pm; i += kInrThreads) {
        float v = lds[i];
#pragma unroll
        for (int w = 1; w < kInrWaves; ++w) v += lds[w * (kInrStageRows * SW) + i];
        pd[i] = v;
    }
}

// 64-bit fixed point of the table-gradient sums a thread adds at once: 2^-32
// residual units, clamped to +-2^11 (a thread's run has at most 512 points;
// an entry receives at most 4 x 2^17 such sums per chunk, so its sum stays
// below 2^62).
constexpr float kFixScale = 4294967296.0f;
constexpr float kFixClamp = 2048.0f;

__device__ __forceinline__ unsigned long long to_fixed(float v) {
    v = fminf(fmaxf(v, -kFixClamp), kFixClamp);
    return (unsigned long long)__float2ll_rn(v * kFixScale);
}

// Scatter jobs, in level order: each level of the LDS prefix in ranges of
// kInrScatEntries entries, then one job per global-atomic level.  The jobs of
// one chunk run on one XCD (workgroup ids that agree mod 8), where they share
// the chunk's points in L2.
template <int DIM>
__global__ void __launch_bounds__(kInrThreads) k_inr_scatter(GridArgs g, HashInrArgs a, InrStep f) {
    extern __shared__ __attribute__((aligned(16))) unsigned long long acc[];  // [2 * kInrScatEntries]
    const int tid = threadIdx.x;
    const int xcd = (int)(blockIdx.x & 7u), slot = (int)(blockIdx.x >> 3);
    int job = slot % f.scat_jobs;
    const int chunk = (slot / f.scat_jobs) * 8 + xcd;
    if (chunk >= f.scat_chunks) return;
    int l = 0, r0 = 0;
    for (; l < g.n_levels - 1; ++l) {
        const int ranges = l < f.lds_levels ? (g.size[l] + kInrScatEntries - 1) / kInrScatEntries : 1;
        if (job < ranges) break;
        job -= ranges;
    }
    const bool use_lds = l < f.lds_levels;
    if (use_lds) r0 = job * kInrScatEntries;
    const Level lv{g.res[l], (uint32_t)g.offset[l], g.direct[l] != 0, g.mask[l]};
    const int n_ent = use_lds ? min(kInrScatEntries, g.size[l] - r0) : 0;
    for (int i = tid; i < 2 * n_ent; i += kInrThreads) acc[i] = 0ull;
    __syncthreads();
    // each thread takes a run of consecutive points and keeps one pending sum
    // per corner, added to the accumulators only when the corner's entry
    // changes: neighbouring points share the entries of coarse levels
    const int64_t p0 = (int64_t)chunk * f.scat_chunk;
    const int64_t p1 = p0 + f.scat_chunk < a.n ? p0 + f.scat_chunk : a.n;
    const int64_t per = f.scat_chunk / kInrThreads;  // a multiple of 4, also in a short last chunk
    const int64_t pb = p0 + (int64_t)tid * per;
    const int64_t pe = pb + per < p1 ? pb + per : p1;  // pe <= pb: nothing to do
    const float* dl = f.dfeat + 2 * (size_t)l * f.dstride;
    constexpr int NC = 1 << DIM;
    constexpr uint32_t kNone = 0xffffffffu;
    // pending sums: float32, in the thread's own fixed order; rounded to
    // fixed point when added to the LDS accumulators
    uint32_t pend[NC];
    float g0[NC], g1[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
        pend[q] = kNone;
        g0[q] = g1[q] = 0.0f;
    }
    if (lv.mask != 0.0f) {
        // 4 points per load group, 16-byte loads (x 16-byte aligned, runs
        // starting at multiples of 4 points)
        constexpr int U = 4;
        for (int64_t pg = pb; pg < pe; pg += U) {
            float ux[U][DIM];
            float2 dfs[U];
            if (pg + U <= pe) {
#pragma unroll
                for (int i = 0; i < U * DIM; i += 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(a.x + pg * DIM + i);
#pragma unroll
                    for (int c = 0; c < 4; ++c) ux[(i + c) / DIM][(i + c) % DIM] = v[c];
                }
#pragma unroll
                for (int i = 0; i < U; i += 2) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(dl + 2 * (pg + i));
                    dfs[i] = make_float2(v[0], v[1]);
                    dfs[i + 1] = make_float2(v[2], v[3]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const int64_t pi = pg + i < pe ? pg + i : pe - 1;
#pragma unroll
                    for (int k = 0; k < DIM; ++k) ux[i][k] = a.x[pi * DIM + k];
                    dfs[i] = *reinterpret_cast<const float2*>(dl + 2 * pi);
                }
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                if (pg + i >= pe) continue;
                const float2 df = dfs[i];
                uint32_t e[NC];
                float wt[NC];
                level_corners<DIM>(lv, g.tmask, ux[i], e, wt);
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    if (use_lds) {
                        const uint32_t k = e[q] - lv.off - (uint32_t)r0;
                        const uint32_t key = k < (uint32_t)n_ent ? k : kNone;
                        const float v0 = wt[q] * df.x, v1 = wt[q] * df.y;
                        if (key != pend[q]) {
                            if (pend[q] != kNone) {
                                atomicAdd(acc + 2 * pend[q], to_fixed(g0[q]));
                                atomicAdd(acc + 2 * pend[q] + 1, to_fixed(g1[q]));
                            }
                            pend[q] = key;
                            g0[q] = v0;
                            g1[q] = v1;
                        } else {
                            g0[q] += v0;
                            g1[q] += v1;
                        }
                    } else {
                        const float v0 = wt[q] * df.x, v1 = wt[q] * df.y;
                        if (e[q] != pend[q]) {
                            if (pend[q] != kNone) {
                                atomicAdd(f.grad + 2 * (size_t)pend[q], f.dy_scale * g0[q]);
                                atomicAdd(f.grad + 2 * (size_t)pend[q] + 1, f.dy_scale * g1[q]);
                            }
                            pend[q] = e[q];
                            g0[q] = v0;
                            g1[q] = v1;
                        } else {
                            g0[q] += v0;
                            g1[q] += v1;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NC; ++q) {
            if (pend[q] == kNone) continue;
            if (use_lds) {
                atomicAdd(acc + 2 * pend[q], to_fixed(g0[q]));
                atomicAdd(acc + 2 * pend[q] + 1, to_fixed(g1[q]));
            } else {
                atomicAdd(f.grad + 2 * (size_t)pend[q], f.dy_scale * g0[q]);
                atomicAdd(f.grad + 2 * (size_t)pend[q] + 1, f.dy_scale * g1[q]);
            }
        }
    }
    __syncthreads();
    if (use_lds) {
        float* pt = f.part_tab + (size_t)chunk * f.lds_tab_floats + 2 * ((size_t)lv.off + r0);
        for (int i = tid; i < 2 * n_ent; i += kInrThreads)
            pt[i] = (float)((double)(long long)acc[i] * (1.0 / 4294967296.0));
    }
}

// Per parameter q: the gradient (partials summed in a fixed order: 4
// interleaved slices of the rows, then the slices; times the derivative of
// the mean), written out, and the Adam step.  A block takes 64 parameters;
// the last block sums the squared-error partials into the loss.
__global__ void __launch_bounds__(256) k_inr_post(HashInrArgs a, InrStep f, int64_t P, int groups, int pm, int adam,
                                                  float c1, float c2, float loss_scale) {
    __shared__ double dpart[256];
    __shared__ float red[4][64];
    if (blockIdx.x == gridDim.x - 1) {
        double s = 0.0;
        for (int r = threadIdx.x; r < groups; r += blockDim.x) s += (double)f.part_dec[(size_t)r * f.part_w + pm];
        dpart[threadIdx.x] = s;
        __syncthreads();
        for (int hh = 128; hh >= 1; hh >>= 1) {
            if ((int)threadIdx.x < hh) dpart[threadIdx.x] += dpart[threadIdx.x + hh];
            __syncthreads();
        }
        if (threadIdx.x == 0) a.loss[0] = (float)(dpart[0] * (double)loss_scale);
        return;
    }
    const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int64_t q = (int64_t)blockIdx.x * 64 + c;
    float s = 0.0f;
    if (q < f.lds_tab_floats) {
#pragma unroll 4
        for (int w = r; w < f.scat_chunks; w += 4) s += f.part_tab[(size_t)w * f.lds_tab_floats + q];
    } else if (q >= f.tab_floats && q < P) {
        const int64_t d = q - f.tab_floats;
#pragma unroll 4
        for (int w = r; w < groups; w += 4) s += f.part_dec[(size_t)w * f.part_w + d];
    }
    red[r][c] = s;
    __syncthreads();
    if (r != 0 || q >= P) return;
    float gq;
    if (q >= f.lds_tab_floats && q < f.tab_floats) {
        gq = f.grad[q];  // accumulated by atomics, already scaled
    } else {
        gq = f.dy_scale * ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c]));
        f.grad[q] = gq;
    }
    if (adam) adam_update(a.params, a.adam_m, a.adam_v, q, gq, a.lr, a.beta1, a.beta2, a.eps, c1, c2);
}

template <int DIM, int HM, int FM>
void launch_decode_t(const GridArgs& g, const HashInrArgs& a, const InrShape& sh, const InrStep& f, const float* wp,
                     hipStream_t s) {
    hipLaunchKernelGGL((k_inr_decode<DIM, HM, FM>), dim3((unsigned)sh.groups), dim3(kInrThreads), sh.lds_bytes, s, g,
                       a, f, wp);
}

template <int DIM>
void launch_decode_dim(const GridArgs& g, const HashInrArgs& a, const InrShape& sh, const InrStep& f, const float* wp,
                       hipStream_t s) {
    if (sh.hm == 32 && sh.fm == 16)
        launch_decode_t<DIM, 32, 16>(g, a, sh, f, wp, s);
    else if (sh.hm == 32)
        launch_decode_t<DIM, 32, 32>(g, a, sh, f, wp, s);
    else if (sh.fm == 16)
        launch_decode_t<DIM, 64, 16>(g, a, sh, f, wp, s);
    else
        launch_decode_t<DIM, 64, 32>(g, a, sh, f, wp, s);
}

}  // namespace

void launch_hash_inr_step(const GridArgs& g, const HashInrArgs& a, hipStream_t s) {
    InrWs w{};
    hash_inr_workspace_layout(g, a.hidden, a.n_out, a.n, (char*)a.workspace, &w);
    const InrShape sh = inr_shape(g, a.hidden, a.n_out, a.n);
    const int64_t P = hash_inr_param_count(g, a.hidden, a.n_out);
    InrStep f{};
    f.tab_floats = sh.tab_floats;
    f.lds_tab_floats = sh.lds_tab_floats;
    f.lds_levels = sh.lds_levels;
    f.iters = sh.iters;
    f.part_w = sh.part_w;
    f.scat_chunk = sh.scat_chunk;
    f.scat_chunks = sh.scat_chunks;
    f.scat_jobs = sh.scat_jobs;
    f.dstride = sh.dstride;
    f.dfeat = w.dfeat;
    f.part_dec = w.part_dec;
    f.part_tab = w.part_tab;
    f.grad = a.grad ? a.grad : w.grad;
    f.dy_scale = (float)(2.0 / ((double)a.n * (double)a.n_out));
    // the levels past the LDS prefix accumulate atomically from zero
    if (sh.tab_floats > sh.lds_tab_floats)
        launch_fill_f32(f.grad + sh.lds_tab_floats, sh.tab_floats - sh.lds_tab_floats, 0.0f, s);
    hipLaunchKernelGGL(k_inr_pad, dim3((unsigned)((sh.weight_floats + 255) / 256)), dim3(256), 0, s,
                       (const float*)(a.params + sh.tab_floats), a.hidden, 2 * g.n_levels, a.n_out, sh.hm, sh.fm, w.wpad);
    if (g.dim == 3)
        launch_decode_dim<3>(g, a, sh, f, w.wpad, s);
    else
        launch_decode_dim<2>(g, a, sh, f, w.wpad, s);
    const dim3 scat((unsigned)((int64_t)sh.scat_jobs * ((sh.scat_chunks + 7) / 8 * 8)));
    const size_t scat_lds = 16 * (size_t)kInrScatEntries;
    if (g.dim == 3)
        hipLaunchKernelGGL(k_inr_scatter<3>, scat, dim3(kInrThreads), scat_lds, s, g, a, f);
    else
        hipLaunchKernelGGL(k_inr_scatter<2>, scat, dim3(kInrThreads), scat_lds, s, g, a, f);
    const int adam = a.adam_m && a.adam_v && a.step >= 1;
    float c1 = 1.0f, c2 = 1.0f;
    if (adam) adam_corrections(a.beta1, a.beta2, a.step, &c1, &c2);
    hipLaunchKernelGGL(k_inr_post, dim3((unsigned)((P + 63) / 64 + 1)), dim3(256), 0, s, a, f, P, sh.groups, sh.pm,
                       adam, c1, c2, (float)(1.0 / ((double)a.n * (double)a.n_out)));
}

}  // namespace nerf

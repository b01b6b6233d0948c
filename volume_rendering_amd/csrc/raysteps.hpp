// Per-wave building blocks shared by the standalone kernels and the fused
// render: compositing of one ray, inverse-CDF resampling plus merge of one
// ray, spherical harmonics and multiresolution hash-grid lookups.
#pragma once

#include <hip/hip_fp16.h>

#include "common.hpp"
#include "launch.hpp"

namespace nerf {

// ---------------------------------------------------------------------------
// Alpha compositing of one ray by one wave ("Spatial Intelligence - Part 1:
// NeRF", Section 1 Theory, 3. Volume rendering; Section 2 Code, 5. Volume
// rendering in code).  Samples are taken 64 at a time, one per lane; the
// exclusive transmittance product is a wave-level multiplicative scan whose
// last value carries into the next 64 samples.  `term_T` > 0 zeroes sample i
// and every later sample once T_i < term_T.
// ---------------------------------------------------------------------------
struct CompositeOut {
    float r, g, b, depth, acc;
};

__device__ __forceinline__ CompositeOut composite_ray(const float* z, const f32x4* raw, int n, float dnorm,
                                                      float* w_out, float term_T) {
    const int lane = lane_id();
    float carry = 1.0f;
    float sr = 0.f, sg = 0.f, sbl = 0.f, sd = 0.f, sa = 0.f;
    bool stopped = false;
    for (int base = 0; base < n; base += kWave) {
        const int i = base + lane;
        const bool valid = i < n;
        float alpha = 0.f, zi = 0.f;
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
        if (valid) {
            zi = z[i];
            const float delta = (i + 1 < n) ? (z[i + 1] - zi) * dnorm : 1e10f * dnorm;
            r = raw[i];
            const float sigma = fmaxf(r[3], 0.0f);
            alpha = 1.0f - expf(-sigma * delta);
        }
        const float surv = valid ? (1.0f - alpha + 1e-10f) : 1.0f;
        const float incl = wave_scan_mul(surv);
        float excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 1.0f;
        const float T = carry * excl;
        bool stop_here = false;
        if (term_T > 0.0f) {
            // first sample of this block (in order) with T < term_T, unless already stopped
            const unsigned long long m = __ballot(valid && T < term_T);
            const int first = m ? __builtin_ctzll(m) : kWave;
            stop_here = stopped || (lane >= first);
            if (m) stopped = true;
        }
        float w = (valid && !stop_here) ? T * alpha : 0.0f;
        if (valid && w_out) w_out[i] = w;
        sa += w;
        sd += w * zi;
        sr += w * sigmoidf_(r[0]);
        sg += w * sigmoidf_(r[1]);
        sbl += w * sigmoidf_(r[2]);
        carry *= __shfl(incl, kWave - 1, kWave);
        if (stopped && term_T > 0.0f) break;
    }
    CompositeOut o;
    o.r = wave_sum(sr);
    o.g = wave_sum(sg);
    o.b = wave_sum(sbl);
    o.depth = wave_sum(sd);
    o.acc = wave_sum(sa);
    return o;
}

// ---------------------------------------------------------------------------
// Inverse-CDF resampling of one ray by one wave (Section 1 Theory, 4.2
// Hierarchical volume sampling; Section 2 Code, 6. Hierarchical sampling).
// zc[0..nc) coarse samples, wc their weights.  Scratch: bins (nc-1 floats),
// cdf (nc-1 doubles).  The cdf is the exact float64 running sum of
// w'_j = w_{j+1} + 1e-5 divided by its total, so every comparison with u is
// decided exactly as in any other exact evaluation.  Writes the fine samples
// to zf[0..nf) (may alias zc + nc) and optionally bin indices.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void sample_pdf_ray(const float* zc, const float* wc, int nc, int nf, uint64_t seed,
                                               uint64_t ray, float* bins, double* cdf, float* zf,
                                               int32_t* bin_out) {
    const int lane = lane_id();
    const int B = nc - 2;  // weights used: w[1..nc-2]
    for (int k = lane; k < nc - 1; k += kWave) bins[k] = __fmul_rn(0.5f, __fadd_rn(zc[k], zc[k + 1]));
    double carry = 0.0;
    for (int base = 0; base < B; base += kWave) {
        const int j = base + lane;
        NERF_DCHECK(j >= B || (wc[j + 1] >= 0.0f && wc[j + 1] <= 100.0f), kCheckPdfWeight);
        const double v = j < B ? (double)__fadd_rn(wc[j + 1], 1e-5f) : 0.0;
        const double incl = wave_scan_add_f64(v);
        if (j < B) cdf[j + 1] = carry + incl;
        carry += __shfl(incl, kWave - 1, kWave);
    }
    wave_lds_sync();
    const double total = carry;
    for (int k = lane; k <= B; k += kWave) cdf[k] = k == 0 ? 0.0 : cdf[k] / total;
    wave_lds_sync();
    for (int m = lane; m < nf; m += kWave) {
        const double u = (double)philox_uniform(seed, ray, (uint32_t)m, kStreamPdf);
        int lo = 0, hi = B + 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (cdf[mid] <= u)
                lo = mid + 1;
            else
                hi = mid;
        }
        NERF_DCHECK(lo >= 1 && lo <= B, kCheckPdfBin);
        const int below = lo - 1 > 0 ? lo - 1 : 0;
        const int above = lo < B ? lo : B;
        const double cb = cdf[below];
        const double denom = fmax(__dsub_rn(cdf[above], cb), 1e-5);
        const double t = __ddiv_rn(__dsub_rn(u, cb), denom);
        const double bb = (double)bins[below];
        const double ba = (double)bins[above];
        zf[m] = (float)__dadd_rn(bb, __dmul_rn(t, __dsub_rn(ba, bb)));
        if (bin_out) bin_out[m] = lo;
    }
    wave_lds_sync();
}

// Ascending sort of in[0..n), n <= 64*K, into out[0..n) by a bitonic
// network across the wave: element 64k + lane is held in v[k] (padding
// +inf); partners closer than 64 are exchanged between lanes, farther ones
// between registers of a lane.  min/max return one of their operands, so the
// output is exactly the sorted input.
template <int K>
__device__ __forceinline__ void wave_sort(const float* in, int n, float* out) {
    constexpr int LOG = K == 1 ? 6 : (K == 2 ? 7 : 8);
    static_assert(64 * K == (1 << LOG), "K in {1, 2, 4}");
    const int lane = lane_id();
    float v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = 64 * k + lane;
        v[k] = i < n ? in[i] : __builtin_inff();
    }
#pragma unroll
    for (int st = 1; st <= LOG; ++st) {
#pragma unroll
        for (int t = st - 1; t >= 0; --t) {
            const int kk = 1 << st, j = 1 << t;
            float nv[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int i = 64 * k + lane;
                const float p = j < kWave ? __shfl_xor(v[k], j, kWave) : v[k ^ (j / kWave)];
                const bool take_min = ((i & kk) == 0) == ((i & j) == 0);
                nv[k] = take_min ? fminf(v[k], p) : fmaxf(v[k], p);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = nv[k];
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = 64 * k + lane;
        if (i < n) out[i] = v[k];
    }
}

__device__ __forceinline__ void wave_sort_n(const float* in, int n, float* out) {
    if (n <= 64)
        wave_sort<1>(in, n, out);
    else if (n <= 128)
        wave_sort<2>(in, n, out);
    else
        wave_sort<4>(in, n, out);
}

// Merge of ascending a[0..na) and b[0..nb) into out[0..na+nb): a[e] goes to
// e + #{b < a[e]}, b[m] to m + #{a <= b[m]}, a permutation that lists the
// union in ascending order (equal values are equal floats, so which of two
// equal elements lands first does not change the output).
__device__ __forceinline__ void merge_sorted(const float* a, int na, const float* b, int nb, float* out) {
    const int lane = lane_id();
    for (int e = lane; e < na; e += kWave) {
        const float v = a[e];
        int lo = 0, hi = nb;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (b[mid] < v)
                lo = mid + 1;
            else
                hi = mid;
        }
        NERF_DCHECK(e + lo < na + nb, kCheckMerge);
        out[e + lo] = v;
    }
    for (int m = lane; m < nb; m += kWave) {
        const float v = b[m];
        int lo = 0, hi = na;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a[mid] <= v)
                lo = mid + 1;
            else
                hi = mid;
        }
        NERF_DCHECK(m + lo < na + nb, kCheckMerge);
        out[m + lo] = v;
    }
}

// Ascending union of the first-pass samples zc[0..nc) and the resampled
// zf[0..nf) into out (the input to the second pass).  Jittered stratified
// samples are ascending already (checked; sorted here otherwise); the
// resampled ones are sorted first.  tmp holds nc + nf floats.
__device__ __forceinline__ void merge_samples(const float* zc, int nc, const float* zf, int nf, float* tmp,
                                              float* out) {
    const int lane = lane_id();
    bool asc = true;
    for (int e = lane; e + 1 < nc; e += kWave) asc = asc && (zc[e] <= zc[e + 1]);
    const float* A = zc;
    if (__ballot(!asc) != 0ull) {
        wave_sort_n(zc, nc, tmp + nf);
        A = tmp + nf;
    }
    wave_sort_n(zf, nf, tmp);
    wave_lds_sync();
    merge_sorted(A, nc, tmp, nf, out);
    wave_lds_sync();
}

// ---------------------------------------------------------------------------
// Voxels of a regular grid over the scene box: floor((x - lo) * scale) of
// rounded float32 operations, clamped to the grid.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int grid_coord(float t, float scale, int res) {
    const float f = floorf(__fmul_rn(t, scale));
    return (int)fminf(fmaxf(f, 0.0f), (float)(res - 1));  // NaN -> 0
}

// Inside the closed box [lo, hi]^3 and in an occupied voxel of the bitset
// (bit v%32 of word v/32, v = (vx*res + vy)*res + vz, formed in 64 bits).
__device__ __forceinline__ bool box_occupied(const uint32_t* occ, int res, float scale, float lo, float hi,
                                             const float (&x)[3]) {
    bool inside = true;
    int v[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        inside = inside && (x[a] >= lo) && (x[a] <= hi);
        v[a] = grid_coord(__fsub_rn(x[a], lo), scale, res);
    }
    const uint64_t r = (uint64_t)res;
    const uint64_t vox = ((uint64_t)v[0] * r + (uint64_t)v[1]) * r + (uint64_t)v[2];
    NERF_DCHECK((vox >> 5) < (r * r * r + 31u) / 32u, kCheckVoxel);
    return inside && ((occ[vox >> 5] >> (uint32_t)(vox & 31u)) & 1u);
}

// ---------------------------------------------------------------------------
// Real spherical harmonics, degrees 0..3, orthonormal, no Condon-Shortley
// phase; order: l, then m = -l..l.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void sh16_eval(float x, float y, float z, float (&o)[16]) {
    const float xx = x * x, yy = y * y, zz = z * z;
    o[0] = 0.28209479177387814f;
    o[1] = 0.4886025119029199f * y;
    o[2] = 0.4886025119029199f * z;
    o[3] = 0.4886025119029199f * x;
    o[4] = 1.0925484305920792f * x * y;
    o[5] = 1.0925484305920792f * y * z;
    o[6] = 0.31539156525252005f * (3.0f * zz - 1.0f);
    o[7] = 1.0925484305920792f * x * z;
    o[8] = 0.5462742152960396f * (xx - yy);
    o[9] = 0.5900435899266435f * y * (3.0f * xx - yy);
    o[10] = 2.890611442640554f * x * y * z;
    o[11] = 0.4570457994644658f * y * (5.0f * zz - 1.0f);
    o[12] = 0.3731763325901154f * z * (5.0f * zz - 3.0f);
    o[13] = 0.4570457994644658f * x * (5.0f * zz - 1.0f);
    o[14] = 1.445305721320277f * z * (xx - yy);
    o[15] = 0.5900435899266435f * x * (xx - 3.0f * yy);
}

// ---------------------------------------------------------------------------
// Multiresolution hash grid ("Instant-NGP - Visual Experiments", shared
// toolkit, 2D as printed and extended to 3D).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t grid_index(int ix, int iy, int iz, int N, bool direct, uint32_t tmask) {
    if (direct) return (uint32_t)((ix * (N + 1) + iy) * (N + 1) + iz);
    return ((uint32_t)ix ^ ((uint32_t)iy * 2654435761u) ^ ((uint32_t)iz * 805459861u)) & tmask;
}
__device__ __forceinline__ uint32_t grid_index(int ix, int iy, int N, bool direct, uint32_t tmask) {
    if (direct) return (uint32_t)(ix * (N + 1) + iy);
    return ((uint32_t)ix ^ ((uint32_t)iy * 2654435761u)) & tmask;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Grid tables for the lookups, addressed by absolute entry (level offset +
// index; entry = two float16 features in 32 bits, the first in the low
// half), read in aligned 8-byte words.  Global tables go through a buffer
// resource: a load whose entry is not needed gets an out-of-range offset and
// returns 0 without touching memory, so every load issues unconditionally.
struct GridTabGlobal {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit GridTabGlobal(const GridArgs& g)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.tables), (short)0, g.bytes, kBufferWord3)) {}
    __device__ __forceinline__ u32x2 word(uint32_t a) const {
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(a * 4u), 0, 0));
    }
    __device__ __forceinline__ uint32_t entry_unless(uint32_t a, bool skip) const {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)(skip ? kBufferOutOfRange : a * 4u), 0, 0);
    }
};

// Tables staged in LDS (8-byte aligned, padded to whole words).
struct GridTabLds {
    const uint32_t NERF_LDS_PTR t;
    __device__ __forceinline__ u32x2 word(uint32_t a) const { return *reinterpret_cast<const u32x2 NERF_LDS_PTR>(t + a); }
    __device__ __forceinline__ uint32_t entry_unless(uint32_t a, bool) const { return t[a]; }
};

__device__ __forceinline__ float half_lo(uint32_t e) { return __half2float(__ushort_as_half((unsigned short)(e & 0xFFFFu))); }
__device__ __forceinline__ float half_hi(uint32_t e) { return __half2float(__ushort_as_half((unsigned short)(e >> 16))); }

// One level lookup in DIM dimensions (resolution N, direct or hashed,
// entries from absolute entry `off` of `tab`) at a unit-cube point, in two
// phases so that the loads of several lookups can be in flight together:
// issue() computes the corner entries and starts their loads, finish()
// interpolates.
//
// The 2^DIM corners are taken in pairs along the axis whose neighbours are
// often adjacent entries: the last axis on direct levels (entries idx,
// idx + 1), x on hashed levels (for even ix the entries idx and idx ^ 1).
// The aligned 8-byte word holding a pair's first entry is always read; the
// second entry is read separately only when it lies in another word.
template <int DIM>
struct GridLookup {
    static_assert(DIM == 2 || DIM == 3, "2D or 3D grids");
    static constexpr int NP = 1 << (DIM - 1);  // corner pairs
    u32x2 W[NP];
    uint32_t B[NP], A0[NP], A1[NP];
    bool P[NP];
    float w[DIM];
    uint32_t off;
    bool direct;

    // Corner offsets of pair q: the pair axis takes 0 and 1, the bits of q
    // (most significant first) the other axes.
    __device__ static __forceinline__ void deltas(int q, bool direct, int (&d0)[DIM], int (&d1)[DIM]) {
        const int ax = direct ? DIM - 1 : 0;
        int bit = DIM - 2;
#pragma unroll
        for (int a = 0; a < DIM; ++a) {
            const bool pa = a == ax;
            const int v = pa ? 0 : (q >> bit) & 1;
            d0[a] = v;
            d1[a] = pa ? 1 : v;
            bit -= pa ? 0 : 1;
        }
    }

    // entries of a level's table: (N+1)^DIM direct, T hashed
    __device__ static __forceinline__ uint32_t level_entries(int N, bool direct, uint32_t tmask) {
        uint32_t e = 1u;
        for (int a = 0; a < DIM; ++a) e *= (uint32_t)(N + 1);
        return direct ? e : tmask + 1u;
    }

    __device__ static __forceinline__ uint32_t index(const int (&i)[DIM], int N, bool direct, uint32_t tmask) {
        if constexpr (DIM == 3)
            return grid_index(i[0], i[1], i[2], N, direct, tmask);
        else
            return grid_index(i[0], i[1], N, direct, tmask);
    }

    template <class Tab>
    __device__ __forceinline__ void issue(const Tab& tab, uint32_t off_, int N, bool direct_, uint32_t tmask,
                                          const float (&u)[DIM]) {
        off = off_;
        direct = direct_;
        int c0[DIM];
#pragma unroll
        for (int a = 0; a < DIM; ++a) {
            const float c = __fmul_rn(u[a], (float)N);
            const float f = floorf(c);
            w[a] = c - f;
            c0[a] = (int)f;
        }
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            int d0[DIM], d1[DIM], ia[DIM], ib[DIM];
            deltas(q, direct, d0, d1);
#pragma unroll
            for (int a = 0; a < DIM; ++a) {
                ia[a] = min(max(c0[a] + d0[a], 0), N);
                ib[a] = min(max(c0[a] + d1[a], 0), N);
            }
            A0[q] = off + index(ia, N, direct, tmask);
            A1[q] = off + index(ib, N, direct, tmask);
            NERF_DCHECK(A0[q] - off < level_entries(N, direct, tmask) && A1[q] - off < level_entries(N, direct, tmask),
                        kCheckGridIndex);
            P[q] = (A0[q] >> 1) == (A1[q] >> 1);
            W[q] = tab.word(A0[q] & ~1u);
            B[q] = tab.entry_unless(A1[q], P[q]);
        }
    }

    // Features (f0, f1) times `scale`; corner indices optionally to
    // idx_out[0..2^DIM) (lexicographic, x most significant).
    __device__ __forceinline__ void finish(float scale, float& f0, float& f1, uint32_t* idx_out) const {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            int d0[DIM], d1[DIM];
            deltas(q, direct, d0, d1);
            float wt0 = 1.0f, wt1 = 1.0f;
            int k0 = 0, k1 = 0;
#pragma unroll
            for (int a = 0; a < DIM; ++a) {
                wt0 *= d0[a] ? w[a] : 1.0f - w[a];
                wt1 *= d1[a] ? w[a] : 1.0f - w[a];
                k0 = 2 * k0 + d0[a];
                k1 = 2 * k1 + d1[a];
            }
            if (idx_out) {
                idx_out[k0] = A0[q] - off;
                idx_out[k1] = A1[q] - off;
            }
            const uint32_t e0 = (A0[q] & 1u) ? W[q].y : W[q].x;
            const uint32_t e1 = P[q] ? ((A1[q] & 1u) ? W[q].y : W[q].x) : B[q];
            a0 += wt0 * half_lo(e0);
            a1 += wt0 * half_hi(e0);
            a0 += wt1 * half_lo(e1);
            a1 += wt1 * half_hi(e1);
        }
        f0 = scale * a0;
        f1 = scale * a1;
    }
};

// Level l of the 3D grid g (tables in global memory), times the level's
// mask.  Used where the level differs between lanes (the fused render), so
// a level is looked up even when its mask is 0: skipping it there would
// split the wave.
__device__ __forceinline__ void grid_level(const GridArgs& g, int l, float ux, float uy, float uz, float& f0, float& f1,
                                           uint32_t* idx_out) {
    const GridTabGlobal tab(g);
    const float u[3] = {ux, uy, uz};
    GridLookup<3> q;
    q.issue(tab, (uint32_t)g.offset[l], g.res[l], g.direct[l] != 0, g.tmask, u);
    q.finish(g.mask[l], f0, f1, idx_out);
}

}  // namespace nerf

// Shared device helpers for the gfx950 kernels: the Philox generator,
// wave-level scans, bfloat16 packing and float32 steps with explicit
// rounding.  Only code built for gfx950 (wave64, MFMA) lives here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nerf {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Index checks of the checked build (-DNERF_CHECK): a failed check sets its
// bit in this translation unit's device word (an atomic or; nothing traps,
// so a bad index is reported after the run instead of faulting the GPU).
// nerf_check_flags() reads and clears the words of every unit.  Without
// NERF_CHECK the checks compile to nothing.
// ---------------------------------------------------------------------------
enum CheckBit : unsigned {
    kCheckGridIndex = 0,    // hash-grid corner index outside its level's table
    kCheckRaySample = 1,    // sample index outside a ray's sample arrays
    kCheckPdfBin = 2,       // inverse-CDF bin outside 1 .. n_coarse - 2
    kCheckMerge = 3,        // merged sample position outside the merged array
    kCheckVoxel = 4,        // occupancy word outside the bitset
    kCheckCell = 5,         // cell id outside the cell grid
    kCheckLiveEntry = 6,    // live-list entry or bucket slot outside the workspace
    kCheckCompactLds = 7,   // compaction entry outside the workgroup's LDS list
    kCheckPdfWeight = 8,    // inverse-CDF weight outside its precondition: finite, in [0, 100]
};
#ifdef NERF_CHECK
int check_register(unsigned (*take)());
static __device__ unsigned g_check_word;
#define NERF_DCHECK(cond, bit)                                                   \
    do {                                                                         \
        if (!(cond)) atomicOr(&::nerf::g_check_word, 1u << (unsigned)(bit));    \
    } while (0)
// This unit's word, cleared after the read (all bits set if the read failed).
static unsigned check_take() {
    unsigned v = 0u, zero = 0u;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_word), sizeof v) != hipSuccess) return ~0u;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_word), &zero, sizeof zero) != hipSuccess) return ~0u;
    return v;
}
static const int g_check_registered = check_register(&check_take);
#else
#define NERF_DCHECK(cond, bit) \
    do {                       \
    } while (0)
#endif

// Pointer into LDS (address space 3): reads through it are LDS reads.
#define NERF_LDS_PTR __attribute__((address_space(3)))*

// Buffer resource word 3 for raw byte-addressed loads (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;
// A byte offset beyond any buffer this library builds: such a load returns
// 0 without accessing memory.
constexpr uint32_t kBufferOutOfRange = 0xFFFFFFF0u;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64-bit products with
// the key bumped by the Weyl constants between rounds.  Only the first
// output word is used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_w0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32 x 32 -> 64-bit product each (v_mad_u64_u32), not separate
        // low and high multiplies
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
    }
    return c0;
}

// Uniform in [0, 1 - 2^-24] on the 2^-24 grid from the top 24 bits.
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t ray, uint32_t index, uint32_t stream) {
    const uint32_t w = philox_w0((uint32_t)ray, index, (uint32_t)(ray >> 32), stream, (uint32_t)seed,
                                 (uint32_t)(seed >> 32));
    return (float)(w >> 8) * 0x1p-24f;
}

constexpr uint32_t kStreamJitter = 0;
constexpr uint32_t kStreamPdf = 1;

// Stratified sample i of n on [near, far] as rounded float32 operations:
// z = near + ((far - near)/n) * (i + u).
__device__ __forceinline__ float stratified_z(float near, float far, int i, int n, float u) {
    const float step = __fdiv_rn(__fsub_rn(far, near), (float)n);
    return __fadd_rn(near, __fmul_rn(step, __fadd_rn((float)i, u)));
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Orders this wave's LDS traffic: every lane's earlier LDS writes are visible
// to every lane of the wave after the call.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Hides a wave-uniform pointer from loop-invariant code motion, so weight
// loads inside a per-block loop stay next to their use instead of being
// hoisted (and kept live) across the whole loop.
template <class P>
__device__ __forceinline__ P* opaque(P* p) {
    asm volatile("" : "+s"(p));
    return p;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Inclusive product scan over the 64 lanes.
__device__ __forceinline__ float wave_scan_mul(float v) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(v, off, kWave);
        if (l >= off) v *= o;
    }
    return v;
}

// Inclusive sum scan over the 64 lanes (float64).
__device__ __forceinline__ double wave_scan_add_f64(double v) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off, kWave);
        if (l >= off) v += o;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Numerics
// ---------------------------------------------------------------------------
__device__ __forceinline__ __bf16 to_bf16(float f) { return (__bf16)f; }  // v_cvt_pk_bf16_f32, nearest even
__device__ __forceinline__ float bf16_round(float f) { return (float)(__bf16)f; }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// (sin(pi t), cos(pi t)).  t = q/2 + r with q = rint(2t) and |r| <= 1/4, both
// exact in float32; sin(pi r) and cos(pi r) from their Taylor series through
// degree 9 and 10 (truncation below 2.5e-8 for |pi r| <= pi/4), evaluated by
// Horner's rule; the quadrant q mod 4 rotates the pair.
__device__ __forceinline__ void sincospi_taylor(float t, float& s, float& c) {
    const float q = rintf(2.0f * t);
    const float r = fmaf(-0.5f, q, t);
    const float r2 = r * r;
    constexpr float a1 = 3.14159265358979312f, a3 = -5.16771278004996937f, a5 = 2.55016403987734508f,
                    a7 = -0.599264529320791883f, a9 = 0.082145886611128191f;  // pi^j (-1)^((j-1)/2) / j!
    constexpr float b2 = -4.934802200544679f, b4 = 4.0587121264167676f, b6 = -1.33526276885458928f,
                    b8 = 0.235330630358893123f, b10 = -0.0258068913900140508f;  // pi^j (-1)^(j/2) / j!
    const float S = r * fmaf(fmaf(fmaf(fmaf(a9, r2, a7), r2, a5), r2, a3), r2, a1);
    const float C = fmaf(fmaf(fmaf(fmaf(fmaf(b10, r2, b8), r2, b6), r2, b4), r2, b2), r2, 1.0f);
    const int qi = (int)(q - 4.0f * floorf(q * 0.25f));  // q mod 4, exact for any float q
    const float ss = (qi & 1) ? C : S, cc = (qi & 1) ? S : C;
    s = (qi & 2) ? -ss : ss;
    c = ((qi + 1) & 2) ? -cc : cc;
}


}  // namespace nerf

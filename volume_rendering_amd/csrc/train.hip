// One training step of a NeRF-family network for gfx950 ("Spatial
// Intelligence - Part 1: NeRF", Section 1 Theory, 5. Training: the squared
// error between rendered and true colours; Section 2 Code, 7. Training loop:
// MSE of the rendered rgb, Adam).  One network pass: stratified samples ->
// encodings -> network -> compositing -> loss -> gradients of every weight
// and bias -> Adam.
//
// Unlike the fused render, a training step keeps every layer's input in HBM
// (the weight gradients need them): the network runs layer by layer as
// matrix products on the matrix cores (bfloat16 operands with float32
// accumulation, or float32 throughout), with
//   forward and input gradients   C[m][n] = sum_k A[m][k] B[n][k]  (k contiguous;
//                                 A may be two segments, e.g. [hidden, encoding])
//   weight gradients               C[m][n] = sum_k A[k][m] B[k][n]  (k = samples,
//                                 split over workgroups, partial sums added in a
//                                 fixed order, so results are deterministic)
// Activation rows are padded with zero columns to multiples of 32, the k step
// of a tile.
#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>

#include "common.hpp"
#include "launch.hpp"
#include "mlp.hpp"
#include "nets.hpp"
#include "optim.hpp"
#include "train_plan.hpp"

namespace nerf {

namespace {

__device__ __forceinline__ float elt_f(float v) { return v; }
__device__ __forceinline__ float elt_f(__bf16 v) { return (float)v; }
template <class T>
__device__ __forceinline__ T elt_from(float v);
template <>
__device__ __forceinline__ float elt_from<float>(float v) { return v; }
template <>
__device__ __forceinline__ __bf16 elt_from<__bf16>(float v) { return (__bf16)v; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Matrix products
//
// One tile scheme for both products.  A workgroup of four waves (2 x 2)
// computes an output tile of 64*RB rows x 64*CB columns; each wave owns
// RB x CB blocks of 32 x 32, one matrix-engine accumulator each
// (v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x2_f32).  Tile row i is the
// instruction's A operand and tile column j its B operand, so a lane's
// accumulator r holds rows 8(r/4) + 4(lane/32) + r%4 of column lane%32.
// Operands stream through a double-buffered LDS ring in k-steps of 64 bytes
// per row (32 bfloat16 or 16 float32 values; rows padded by 16 bytes); the
// next step's global loads are in flight while the current step multiplies.
// ---------------------------------------------------------------------------
template <class T, int KB = 64>
struct Tl {
    static constexpr int PER = 16 / (int)sizeof(T);  // elements per 16 bytes
    static constexpr int BK = KB / (int)sizeof(T);   // k per step (KB bytes per row)
    static constexpr int P = BK + PER;               // LDS row pitch (elements)
};

struct SegA {
    const void* p;
    int ld;       // elements per row
    int kpad;     // columns (k) of this segment, a multiple of 32
    int row_div;  // row of product row m is m / row_div
};

// Forward and input-gradient products: C[m][n] = sum_k A[m][k] B[n][k]
// (tile rows: n; tile columns: m).
struct GemmNT {
    SegA a0, a1;        // a1.kpad == 0: one segment
    const void* b;      // [N][ldb], ldb >= a0.kpad + a1.kpad
    int ldb;
    int M, N;           // product rows, columns (N a multiple of 32)
    const float* bias;  // [N] or NULL
    int relu;
    const void* mask;   // keep C[m][n] only where mask[m*ldm + n] > 0, or NULL
    int ldm;
    // bfloat16 direct-copy products only: the same mask as one bit per element
    // (bit n%8 of byte bits_in[m*ldbits + n/8]); bits_out receives the bits of
    // C > 0 as stored
    const unsigned char* bits_in;
    unsigned char* bits_out;
    int ldbits;
    void* c;
    int ldc, c_col0, n_store, c_f32;  // stores columns n < n_store at c[m*ldc + c_col0 + n]
};

// Weight gradients: part[split][m][n] = sum over the split's k of
// A[k][m] B[k / b_row_div][n] (tile rows: m; tile columns: n), and with
// bpart the bias gradients bpart[split][m] = sum over the split's k of A[k][m].
struct GemmTN {
    const void* a;  // [K][lda], m contiguous
    int lda, M;     // M (a multiple of 32) <= lda
    const void* b;  // [K / b_row_div][ldb], n contiguous
    int ldb, N, b_row_div;
    int K, k_chunk;  // samples, samples per split (a multiple of 64)
    float* part;     // [splits][M][N]
    float* bpart;    // [splits][M] or NULL
};

// ROWS rows x one k-step of a row-major (k contiguous) matrix: 4 pieces of
// 16 bytes per row; rows at or beyond R read as zero.
template <class T, int ROWS>
struct DirectTile {
    static constexpr int UNITS = ROWS * 4;
    static constexpr int UPT = (UNITS + 255) / 256;
    u32x4 v[UPT];

    __device__ __forceinline__ void load(const T* src, int ld, int row_div, int r0, int R, int k, int tid) {
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const int u = tid + 256 * q;
            v[q] = u32x4{0u, 0u, 0u, 0u};
            if (UNITS % 256 == 0 || u < UNITS) {
                const int r = r0 + (u >> 2);
                if (r < R) {
                    const int row = row_div == 1 ? r : r / row_div;
                    v[q] = *reinterpret_cast<const u32x4*>(src + (size_t)row * ld + k + (u & 3) * Tl<T>::PER);
                }
            }
        }
    }
    __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const int u = tid + 256 * q;
            if (UNITS % 256 == 0 || u < UNITS)
                *reinterpret_cast<u32x4*>(lds + (u >> 2) * Tl<T>::P + (u & 3) * Tl<T>::PER) = v[q];
        }
    }
};

// One k-step of both operands of a weight-gradient product, k-major in
// memory (columns contiguous), transposed into LDS rows [column][k]: TR
// columns of A (the row tile), then TC columns of B (the column tile).  A
// unit is PER k-rows x PER columns, 16 bytes per k-row, transposed in
// registers; the units of both tiles are dealt to the threads in turn
// (thread t takes units t, t + 256, ...), whole waves to one tile.  The loads
// are buffer loads over the split's rows, issued by every thread whatever its
// units: a unit past the last, a column past the matrix or a k past the split
// gets an offset beyond the buffer and reads zeros.  With no branch around
// them the compiler counts the loads in flight exactly and waits for the one
// step it stores, not for the step behind it.  RD: B's row of sample k is
// k / row_div.
template <class T, int TR, int TC, int KB, bool RD>
struct TnTiles {
    static constexpr int PER = Tl<T, KB>::PER, BK = Tl<T, KB>::BK, P = Tl<T, KB>::P;
    static constexpr int KU = BK / PER;  // units along k
    static constexpr int RU = KU * (TR / PER), UNITS = RU + KU * (TC / PER);
    static constexpr int NU = (UNITS + 255) / 256;  // units per thread
    static_assert(RU % 64 == 0 && UNITS % 64 == 0, "units in whole waves");
    union Piece {
        u32x4 u;
        T e[PER];
    };
    __amdgpu_buffer_rsrc_t rs[NU];  // wave-uniform: A's or B's
    const char* base[NU];           // wave-uniform: the split's first row of A or B
    bool of_b[NU];                  // wave-uniform
    int ld[NU], c[NU], kq[NU], dst[NU];
    bool live[NU];
    uint32_t voff[NU][PER];  // without RD: byte offset of each piece from its step's first row
    int row_div, first_b;
    Piece v[2][NU][PER];  // two steps in flight

    __device__ __forceinline__ void setup(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, const char* pa,
                                          const char* pb, const GemmTN& g, int m0, int n0, int first, int tid) {
        const int wave_base = __builtin_amdgcn_readfirstlane(tid & ~63);
        row_div = g.b_row_div;
        first_b = first;
#pragma unroll
        for (int q = 0; q < NU; ++q) {
            const int w0 = wave_base + 256 * q;  // the wave's first unit
            const bool is_a = w0 < RU;
            of_b[q] = !is_a;
            rs[q] = is_a ? ra : rb;
            base[q] = is_a ? pa : pb;
            ld[q] = is_a ? g.lda : g.ldb;
            // consecutive units step through k first: the 64 lanes of one
            // LDS store then cover 16 distinct 16-byte bank groups
            const int u = tid + 256 * q - (is_a ? 0 : RU);
            const int cl = (u / KU) * PER;
            kq[q] = (u % KU) * PER;
            c[q] = (is_a ? m0 : n0) + cl;
            live[q] = w0 < UNITS && c[q] < (is_a ? g.M : g.N);
            dst[q] = (is_a ? 0 : TR * P) + cl * P + kq[q];
#pragma unroll
            for (int r = 0; r < PER; ++r)
                voff[q][r] = live[q] ? (uint32_t)(((kq[q] + r) * ld[q] + c[q]) * (int)sizeof(T)) : kBufferOutOfRange;
        }
    }
    // k-rows k0 + kq .. of every unit into buffer b; k0 relative to the split start kb
    __device__ __forceinline__ void load(int b, int kb, int k0, int k_len) {
        if constexpr (!RD) {
            // a resource over the split's rows from k0 on: rows past the split
            // fall outside it and read zeros, so the per-lane offsets stay fixed
#pragma unroll
            for (int q = 0; q < NU; ++q) {
                const int rem = k_len - k0, rowb = ld[q] * (int)sizeof(T);
                const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<char*>(base[q]) + (size_t)(k0 > 0 ? k0 : 0) * rowb, (short)0, rem > 0 ? rem * rowb : 0,
                    kBufferWord3);
#pragma unroll
                for (int r = 0; r < PER; ++r)
                    v[b][q][r].u =
                        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)voff[q][r], 0, 0));
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < NU; ++q)
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const int k = k0 + kq[q] + r;  // within the split
                int row = k;
                if constexpr (RD)
                    if (of_b[q]) row = (kb + k) / row_div - first_b;
                const uint32_t off =
                    live[q] && k < k_len ? (uint32_t)((row * ld[q] + c[q]) * (int)sizeof(T)) : 0x7FFFF000u;
                v[b][q][r].u = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[q], (int)off, 0, 0));
            }
    }
    __device__ __forceinline__ void store(int b, T* lds) const {
#pragma unroll
        for (int q = 0; q < NU; ++q)
            if (live[q]) {
#pragma unroll
                for (int cc = 0; cc < PER; ++cc) {
                    Piece w;
#pragma unroll
                    for (int r = 0; r < PER; ++r) w.e[r] = v[b][q][r].e[cc];
                    *reinterpret_cast<u32x4*>(lds + dst[q] + cc * P) = w.u;
                }
            }
    }
};

// acc += (the wave's rows of the row tile) x (its columns of the column tile)
// over one k-step.  R and C point at the wave's first row of each tile.
template <class T, int RB, int CB, int KB = 64>
__device__ __forceinline__ void wave_mma(f32x16 (&acc)[RB][CB], const T* R, const T* C, int lane) {
    constexpr int P = Tl<T, KB>::P;
    const int l32 = lane & 31, h = lane >> 5;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int ks = 0; ks < Tl<T, KB>::BK / 16; ++ks) {
            bf16x8 a[RB], b[CB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(R + (32 * i + l32) * P + 16 * ks + 8 * h);
#pragma unroll
            for (int j = 0; j < CB; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(C + (32 * j + l32) * P + 16 * ks + 8 * h);
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < Tl<T, KB>::BK / 2; ++ks) {
            float a[RB], b[CB];
#pragma unroll
            for (int i = 0; i < RB; ++i) a[i] = R[(32 * i + l32) * P + 2 * ks + h];
#pragma unroll
            for (int j = 0; j < CB; ++j) b[j] = C[(32 * j + l32) * P + 2 * ks + h];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
}

template <class T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)x[e];
    } else {
        const float4 x = *reinterpret_cast<const float4*>(p);
        v[0] = x.x;
        v[1] = x.y;
        v[2] = x.z;
        v[3] = x.w;
    }
}

template <class T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]) {
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)v[e];
        *reinterpret_cast<bf16x4*>(p) = x;
    } else {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <class T, int RB, int CB>
__global__ void __launch_bounds__(256) k_gemm_nt(GemmNT g) {
    constexpr int P = Tl<T>::P, BK = Tl<T>::BK, TR = 64 * RB, TC = 64 * CB;
    // epilogue staging: per phase PH block-rows (128 bytes of features) of both halves
    constexpr int PH = (int)(128 / (32 * sizeof(T))) < RB ? (int)(128 / (32 * sizeof(T))) : RB;
    constexpr int FW = 32 * PH;                         // features per half and phase
    constexpr int SP = 2 * FW + (int)(16 / sizeof(T));  // staged row pitch (elements)
    constexpr int RING = (TR + TC) * P, STAGE = TC * SP;
    __shared__ __attribute__((aligned(16))) T lds_all[2 * RING > STAGE ? 2 * RING : STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int n0 = blockIdx.y * TR, m0 = blockIdx.x * TC;
    DirectTile<T, TR> rt;
    DirectTile<T, TC> ct;
    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};
    const int K = g.a0.kpad + g.a1.kpad;
    auto load = [&](int k0) {
        rt.load((const T*)g.b, g.ldb, 1, n0, g.N, k0, tid);
        if (k0 < g.a0.kpad)  // a k-step never straddles the segments
            ct.load((const T*)g.a0.p, g.a0.ld, g.a0.row_div, m0, g.M, k0, tid);
        else
            ct.load((const T*)g.a1.p, g.a1.ld, g.a1.row_div, m0, g.M, k0 - g.a0.kpad, tid);
    };
    load(0);
    rt.store(lds_all, tid);
    ct.store(lds_all + TR * P, tid);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) load(k0 + BK);
        const T* cur = lds_all + buf * RING;
        wave_mma<T, RB, CB>(acc, cur + wr * 32 * RB * P, cur + TR * P + wc * 32 * CB * P, lane);
        if (more) {
            T* nxt = lds_all + (buf ^ 1) * RING;
            rt.store(nxt, tid);
            ct.store(nxt + TR * P, tid);
        }
        __syncthreads();
        buf ^= 1;
    }
    const int l32 = lane & 31, h = lane >> 5;
    if (!g.c_f32 && g.n_store == g.N && g.c_col0 == 0) {
        // Through LDS, so that every row leaves as whole 128-byte lines: in
        // phase p each wave stages PH block-rows (128 bytes of features per
        // row) of its accumulators, after bias and ReLU, as [sample][half,
        // feature]; then 16-byte pieces go out along the rows, masked.
        constexpr int PPR = 2 * FW * (int)sizeof(T) / 16;  // 16-byte pieces per staged row
        T* st = lds_all;
#pragma unroll
        for (int p = 0; p < RB / PH; ++p) {
#pragma unroll
            for (int ii = 0; ii < PH; ++ii) {
                const int i = p * PH + ii;
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int ml = wc * 32 * CB + 32 * j + l32;
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int fl = 32 * ii + 8 * gq + 4 * h;  // feature within the half and phase
                        const int n = n0 + wr * 32 * RB + 32 * i + 8 * gq + 4 * h;
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = acc[i][j][4 * gq + e] + (g.bias && n < g.N ? g.bias[n + e] : 0.0f);
                            if (g.relu) v[e] = fmaxf(v[e], 0.0f);
                        }
                        store4<T>(st + ml * SP + wr * FW + fl, v);
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < TC * PPR / 256; ++q) {
                const int u = tid + 256 * q;
                const int ml = u / PPR, pc = u % PPR;
                const int half = pc / (PPR / 2), e0 = (pc % (PPR / 2)) * (int)(16 / sizeof(T));
                const int m = m0 + ml;
                const int n = n0 + half * 32 * RB + p * FW + e0;
                if (m < g.M && n < g.N) {
                    union {
                        u32x4 u;
                        T e[16 / sizeof(T)];
                    } x, mk;
                    x.u = *reinterpret_cast<const u32x4*>(st + ml * SP + half * FW + e0);
                    if (g.mask) {
                        mk.u = *reinterpret_cast<const u32x4*>((const T*)g.mask + (size_t)m * g.ldm + n);
#pragma unroll
                        for (int e = 0; e < (int)(16 / sizeof(T)); ++e)
                            if (!(elt_f(mk.e[e]) > 0.0f)) x.e[e] = elt_from<T>(0.0f);
                    }
                    *reinterpret_cast<u32x4*>((T*)g.c + (size_t)m * g.ldc + g.c_col0 + n) = x.u;
                }
            }
            __syncthreads();
        }
        return;
    }
    // narrow float32 outputs (the heads into raw): element stores
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int m = m0 + wc * 32 * CB + 32 * j + l32;
        if (m >= g.M) continue;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int n = n0 + wr * 32 * RB + 32 * i + 8 * gq + 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e >= g.n_store) continue;
                    float x = acc[i][j][4 * gq + e] + (g.bias ? g.bias[n + e] : 0.0f);
                    if (g.relu) x = fmaxf(x, 0.0f);
                    if (g.mask && !(elt_f(((const T*)g.mask)[(size_t)m * g.ldm + n + e]) > 0.0f)) x = 0.0f;
                    const size_t at = (size_t)m * g.ldc + g.c_col0 + n + e;
                    if (g.c_f32)
                        ((float*)g.c)[at] = x;
                    else
                        ((T*)g.c)[at] = elt_from<T>(x);
                }
            }
        }
    }
}

// Forward and input-gradient products in bfloat16 with the operand tiles
// copied global -> LDS by direct buffer loads (no register staging), three
// k-steps deep: while step t multiplies, steps t+1 and t+2 are in flight.
// 2 x WC waves: two along the product's columns (the weights), WC along its
// rows (the samples); more waves along the samples share one weight tile
// among more samples.
// A tile row is 64 bytes (32 k) whose four 16-byte pieces are XOR-swizzled
// by row, so that the operand reads (32 rows at one k offset) fall in
// distinct banks.  Each copy instruction fills 1 KB of LDS (16 rows); rows
// past the matrix get an out-of-range offset and read as zero.
constexpr int kDmaStages = 3;
constexpr uint32_t kDmaSkip = 0x7FFFF000u;  // offset beyond any tile: the copy reads zeros

// Two bfloat16 in one word (the first in the low half), rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}
typedef short s16x2 __attribute__((ext_vector_type(2)));
// max(x, 0) of both bfloat16 halves, as int16: negative values and -0 become +0.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t d) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, d), s16x2{0, 0}));
}
// Bit 0: the low bfloat16 is > 0; bit 1: the high one is (-0, negatives and
// zero give 0; as int16 the positive values are exactly 1..0x7FFF).
__device__ __forceinline__ uint32_t pos_bits_bf16x2(uint32_t d) {
    const s16x2 t = __builtin_elementwise_max(
        __builtin_elementwise_min(__builtin_bit_cast(s16x2, d), s16x2{1, 1}), s16x2{0, 0});
    const uint32_t u = __builtin_bit_cast(uint32_t, t);
    return (u & 1u) | ((u >> 15) & 2u);
}
// The low / high bfloat16 of d where bit 0 / bit 1 of b is set, else 0.
__device__ __forceinline__ uint32_t mask_bf16x2(uint32_t d, uint32_t b) {
    const int lo = (int)(b << 31) >> 31, hi = (int)(b << 30) >> 31;
    return d & (((uint32_t)hi & 0xFFFF0000u) | ((uint32_t)lo & 0xFFFFu));
}

// Workgroup barrier over LDS traffic only: the wave's LDS operations are
// complete, its global stores may still be in flight (__syncthreads() would
// wait for those too).
__device__ __forceinline__ void lds_barrier() {
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}

// 16 bytes per lane from the buffer at byte offset off into LDS at
// dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (NERF_AS_LDS void*)dst, 16, (int)off, 0, 0, 0);
}

template <int RB, int CB, int WC = 2>
__global__ void __launch_bounds__(128 * WC) k_gemm_nt_dma(GemmNT g) {
    using T = __bf16;
    constexpr int NT = 128 * WC;  // threads
    constexpr int TR = 64 * RB, TC = 32 * CB * WC;
    constexpr int STAGE = (TR + TC) * 64;  // bytes
    constexpr int NW = NT / 64;                        // waves
    constexpr int QR = TR / (16 * NW), QC = TC / (16 * NW);  // 1 KB (16-row) copies per wave per step
    constexpr int PH = 2 < RB ? 2 : RB;        // epilogue: block-rows per phase (128 bytes of features)
    constexpr int FW = 32 * PH;
    constexpr int SP = 2 * FW + 8;             // staged row pitch (elements)
    constexpr int RING = kDmaStages * STAGE, EPI = TC * SP * 2;
    constexpr int PPR = 2 * FW * 2 / 16;  // epilogue: 16-byte pieces per staged row
    constexpr int NPH = RB / PH, NQ = TC * PPR / NT;
    static_assert(TC * PPR % NT == 0 && NT % PPR == 0, "epilogue pieces per thread");
    __shared__ __attribute__((aligned(1024))) char lds[RING > EPI ? RING : EPI];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    const int n0 = blockIdx.y * TR, m0 = blockIdx.x * TC;
    const int K = g.a0.kpad + g.a1.kpad, nk = K / 32;
    const int l32 = lane & 31, h = lane >> 5, sw = swz(l32);

    // The bias (as the accumulators' start) and the epilogue's mask bits are
    // loaded before the first copies, so that their latency overlaps the
    // ring's fill instead of stalling the epilogue.
    // Rows n >= N and pieces past M or N are never stored, so their loads
    // read a clamped in-range address and keep whatever they get.  The loads
    // land straight in their registers (one per output tile, the row offset
    // hidden from the compiler so that it neither merges them nor waits for
    // them before the products need them).
    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (g.bias) {  // uniform
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    int n = n0 + wr * 32 * RB + 32 * i + 8 * gq + 4 * h;
                    n = n < g.N ? n : 0;
                    asm volatile("" : "+v"(n));
                    const float4 x = *reinterpret_cast<const float4*>(g.bias + n);
                    acc[i][j][4 * gq] = x.x;
                    acc[i][j][4 * gq + 1] = x.y;
                    acc[i][j][4 * gq + 2] = x.z;
                    acc[i][j][4 * gq + 3] = x.w;
                }
            } else {
                acc[i][j] = f32x16{};
            }
        }
    // epilogue piece q of phase p: staged row tid / PPR + q * NT / PPR, piece tid % PPR
    const int e_pc = tid % PPR, e_half = e_pc / (PPR / 2), e_e0 = (e_pc % (PPR / 2)) * 8;
    uint32_t mbits[NPH][NQ];
#pragma unroll
    for (int p = 0; p < NPH; ++p)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int m = m0 + tid / PPR + q * (NT / PPR);
            const int n = n0 + e_half * 32 * RB + p * FW + e_e0;
            const size_t at = m < g.M && n < g.N ? (size_t)m * g.ldbits + n / 8 : 0;
            mbits[p][q] = g.bits_in ? g.bits_in[at] : 0xFFu;
        }
    compiler_fence();

    // buffer resources over this tile's rows of the weights and of each activation segment
    const int nrows = g.N - n0 < TR ? g.N - n0 : TR;
    const __amdgpu_buffer_rsrc_t rb = dma_rsrc((const T*)g.b + (size_t)n0 * g.ldb, nrows * g.ldb * 2);
    const int mend = g.M - m0 < TC ? g.M : m0 + TC;  // one past the tile's last product row
    __amdgpu_buffer_rsrc_t rs[2];
    int first[2];
    const SegA* seg[2] = {&g.a0, &g.a1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const SegA& a = *seg[q];
        const int rd = a.row_div > 0 ? a.row_div : 1;
        first[q] = m0 / rd;
        const int last = (mend - 1) / rd;
        rs[q] = dma_rsrc((const T*)a.p + (size_t)first[q] * a.ld, a.kpad ? (last - first[q] + 1) * a.ld * 2 : 0);
    }
    // per-lane source offsets of this wave's copies (16 rows of 4 pieces each)
    uint32_t vr[QR], vc[2][QC];
#pragma unroll
    for (int q = 0; q < QR; ++q) {
        const int row = (wave * QR + q) * 16 + (lane >> 2);
        const int pc = (lane & 3) ^ swz(row);
        vr[q] = n0 + row < g.N ? (uint32_t)(row * g.ldb * 2 + pc * 16) : kDmaSkip;
    }
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
        const SegA& a = *seg[sg];
        const int rd = a.row_div > 0 ? a.row_div : 1;
#pragma unroll
        for (int q = 0; q < QC; ++q) {
            const int row = (wave * QC + q) * 16 + (lane >> 2);
            const int pc = (lane & 3) ^ swz(row);
            const int m = m0 + row;
            vc[sg][q] = m < g.M ? (uint32_t)((m / rd - first[sg]) * a.ld * 2 + pc * 16) : kDmaSkip;
        }
    }
    auto issue = [&](int t) {
        char* slot = lds + (t % kDmaStages) * STAGE;
        const uint32_t kb = (uint32_t)t * 64u;  // byte offset of the step in a weight row
#pragma unroll
        for (int q = 0; q < QR; ++q) dma16(rb, slot + (wave * QR + q) * 1024, vr[q] + kb);
        const bool s0 = t * 32 < g.a0.kpad;
        const uint32_t ka = s0 ? kb : kb - (uint32_t)g.a0.kpad * 2u;
#pragma unroll
        for (int q = 0; q < QC; ++q)
            dma16(s0 ? rs[0] : rs[1], slot + TR * 64 + (wave * QC + q) * 1024, (s0 ? vc[0][q] : vc[1][q]) + ka);
    };
#pragma unroll
    for (int t = 0; t < kDmaStages - 1; ++t)
        if (t < nk) issue(t);
    for (int t = 0; t < nk; ++t) {
        // steps issued after step t: min(stages - 2, nk - 1 - t)
        const int later = nk - 1 - t < kDmaStages - 2 ? nk - 1 - t : kDmaStages - 2;
        static_assert(kDmaStages >= 2 && kDmaStages <= 4, "waits below");
        if (later >= 2)
            wait_vm_lgkm0<2 * (QR + QC)>();
        else if (later == 1)
            wait_vm_lgkm0<QR + QC>();
        else
            wait_vm_lgkm0<0>();
        // A bare barrier: __syncthreads() would add the workgroup fence, which
        // waits for every copy in flight (vmcnt(0)), the later steps' too.
        // Each wave has waited for its own copies of step t and for its LDS
        // reads of step t - 1 above, so after the barrier slot t is complete
        // and the slot of step t + stages - 1 (that of t - 1) is free.
        compiler_fence();
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        if (t + kDmaStages - 1 < nk) issue(t + kDmaStages - 1);
        const char* slot = lds + (t % kDmaStages) * STAGE;
        const char* R = slot + (wr * 32 * RB) * 64;
        const char* C = slot + TR * 64 + (wc * 32 * CB) * 64;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int off = (((2 * ks + h) ^ sw) * 16);
            bf16x8 a[RB], b[CB];
#pragma unroll
            for (int i = 0; i < RB; ++i) a[i] = *reinterpret_cast<const bf16x8*>(R + (32 * i + l32) * 64 + off);
#pragma unroll
            for (int j = 0; j < CB; ++j) b[j] = *reinterpret_cast<const bf16x8*>(C + (32 * j + l32) * 64 + off);
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with the ring before the epilogue reuses it
    // Epilogue through LDS (as k_gemm_nt): whole 128-byte lines per row
    T* st = reinterpret_cast<T*>(lds);
#pragma unroll
    for (int p = 0; p < NPH; ++p) {
#pragma unroll
        for (int ii = 0; ii < PH; ++ii) {
            const int i = p * PH + ii;
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int ml = wc * 32 * CB + 32 * j + l32;
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int fl = 32 * ii + 8 * gq + 4 * h;
                    // pack, then ReLU as a packed integer max (a negative
                    // bfloat16, -0 included, is a negative int16)
                    uint32_t w2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        w2[e] = pack_bf16x2(acc[i][j][4 * gq + 2 * e], acc[i][j][4 * gq + 2 * e + 1]);
                        if (g.relu) w2[e] = relu_bf16x2(w2[e]);
                    }
                    *reinterpret_cast<uint2*>(st + ml * SP + wr * FW + fl) = make_uint2(w2[0], w2[1]);
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int ml = tid / PPR + q * (NT / PPR);
            const int m = m0 + ml;
            const int n = n0 + e_half * 32 * RB + p * FW + e_e0;
            if (m < g.M && n < g.N) {
                union {
                    u32x4 u;
                    T e[8];
                } x, mk;
                x.u = *reinterpret_cast<const u32x4*>(st + ml * SP + e_half * FW + e_e0);
                if (g.bits_in) {
                    const uint32_t mb = mbits[p][q];
#pragma unroll
                    for (int w = 0; w < 4; ++w) x.u[w] = mask_bf16x2(x.u[w], mb >> (2 * w));
                } else if (g.mask) {
                    mk.u = *reinterpret_cast<const u32x4*>((const T*)g.mask + (size_t)m * g.ldm + n);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (!(elt_f(mk.e[e]) > 0.0f)) x.e[e] = elt_from<T>(0.0f);
                }
                *reinterpret_cast<u32x4*>((T*)g.c + (size_t)m * g.ldc + n) = x.u;
                if (g.bits_out) {
                    uint32_t mb = 0;
#pragma unroll
                    for (int w = 0; w < 4; ++w) mb |= pos_bits_bf16x2(x.u[w]) << (2 * w);
                    g.bits_out[(size_t)m * g.ldbits + n / 8] = (unsigned char)mb;
                }
            }
        }
        if (p + 1 < NPH) lds_barrier();
    }
}

// s + the N elements of an LDS row (16-byte aligned), in a fixed order.
template <class T, int N>
__device__ __forceinline__ float row_sum(const T* row, float s) {
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int k = 0; k < N; k += 8) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + k);
#pragma unroll
            for (int e = 0; e < 8; e += 2) s = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{x[e], x[e + 1]}, one, s, false);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N; k += 4) {
            const float4 x = *reinterpret_cast<const float4*>(row + k);
            s += x.x;
            s += x.y;
            s += x.z;
            s += x.w;
        }
    }
    return s;
}

// Weight gradients, k-steps of 128 bytes per row, two steps of loads in
// flight in registers while the step in LDS is multiplied.
template <class T, int RB, int CB, bool RD>
__global__ void __launch_bounds__(256) k_gemm_tn(GemmTN g) {
    constexpr int KB = 128;
    constexpr int P = Tl<T, KB>::P, BK = Tl<T, KB>::BK, TR = 64 * RB, TC = 64 * CB;
    __shared__ __attribute__((aligned(16))) T lds[2][(TR + TC) * P];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;
    // The grid is one-dimensional.  Workgroups are dealt to the eight XCDs
    // round robin (linear id mod 8), and each XCD has its own L2: the output
    // tiles of one split of the samples get ids that are equal mod 8, so the
    // workgroups that read the same operand rows share one L2.  Splits are
    // padded to a multiple of 8; the padding exits at once.
    const int n_mt = (g.M + TR - 1) / TR, n_nt = (g.N + TC - 1) / TC, tiles = n_mt * n_nt;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int tile = slot % tiles, split = xcd + 8 * (slot / tiles);
    if (split * g.k_chunk >= g.K) return;
    const int mt = tile % n_mt, nt = tile / n_mt;
    const int m0 = mt * TR, n0 = nt * TC;
    const int kb = split * g.k_chunk;
    const int ke = kb + g.k_chunk < g.K ? kb + g.k_chunk : g.K;
    const int kl = ke - kb;
    const bool bias = g.bpart && nt == 0 && tid < TR;
    f32x16 acc[RB][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};
    float bsum = 0.0f;
    // buffer resources over the split's rows of both operands
    const int bfirst = kb / g.b_row_div, blast = (ke - 1) / g.b_row_div;
    const __amdgpu_buffer_rsrc_t ra = dma_rsrc((const T*)g.a + (size_t)kb * g.lda, kl * g.lda * (int)sizeof(T));
    const __amdgpu_buffer_rsrc_t rb =
        dma_rsrc((const T*)g.b + (size_t)bfirst * g.ldb, (blast - bfirst + 1) * g.ldb * (int)sizeof(T));
    TnTiles<T, TR, TC, KB, RD> tt;
    tt.setup(ra, rb, (const char*)g.a + (size_t)kb * g.lda * sizeof(T),
             (const char*)g.b + (size_t)bfirst * g.ldb * sizeof(T), g, m0, n0, bfirst, tid);
    // an even number of steps (a step past the split multiplies zeros)
    const int ns = ((kl + BK - 1) / BK + 1) / 2 * 2;
    tt.load(0, kb, 0, kl);
    tt.store(0, lds[0]);
    tt.load(1, kb, BK, kl);
    tt.load(0, kb, 2 * BK, kl);
    lds_barrier();
    // step s is in lds[s % 2], steps s + 1 and s + 2 in register buffers (s + 1) % 2 and s % 2
    auto step = [&](auto par, int s) {
        constexpr int p = decltype(par)::value;
        if (bias) bsum = row_sum<T, BK>(lds[p] + tid * P, bsum);
        wave_mma<T, RB, CB, KB>(acc, lds[p] + wr * 32 * RB * P, lds[p] + TR * P + wc * 32 * CB * P, lane);
        tt.store(p ^ 1, lds[p ^ 1]);
        tt.load(p ^ 1, kb, (s + 3) * BK, kl);
        lds_barrier();
    };
    for (int s = 0; s < ns; s += 2) {
        step(IntC<0>{}, s);
        step(IntC<1>{}, s + 1);
    }
    float* out = g.part + (size_t)split * g.M * g.N;
    const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int n = n0 + wc * 32 * CB + 32 * j + l32;
        if (n >= g.N) continue;
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wr * 32 * RB + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < g.M) out[(size_t)m * g.N + n] = acc[i][j][r];
            }
    }
    if (bias && m0 + tid < g.M) g.bpart[(size_t)split * g.M + m0 + tid] = bsum;
}

// out[off + m*ld + col0 + n] = sum over splits of part[s][m][n], for m < rows,
// n < cols; N a multiple of 4.  A workgroup takes 32 column quads; its 8
// groups of 32 threads sum every 8th split each (group g: splits g, g + 8,
// ... in order), and the group sums are added in group order, a fixed order
// on every call.
struct RedJob {
    const float* part;
    int M, N, rows, cols;
    float* out;
    int64_t off;
    int ld, col0;
    int blocks;  // workgroups of this job
};
constexpr int kRedGroups = 8;

inline RedJob red_job(const float* part, int M, int N, int rows, int cols, float* out, int64_t off, int ld, int col0) {
    const int64_t quads = (int64_t)rows * ((cols + 3) / 4);
    return RedJob{part, M, N, rows, cols, out, off, ld, col0, (int)((quads + 31) / 32)};
}

// Two reductions in one launch: job a's workgroups, then job b's (b.blocks 0: none).
__global__ void __launch_bounds__(256) k_reduce(RedJob a, RedJob b, int splits) {
    __shared__ float4 red[kRedGroups][32];
    const bool first = (int)blockIdx.x < a.blocks;
    const RedJob& j = first ? a : b;
    const int blk = first ? (int)blockIdx.x : (int)blockIdx.x - a.blocks;
    const int l32 = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int cq = (j.cols + 3) / 4;
    const int64_t t = (int64_t)blk * 32 + l32;
    const bool ok = t < (int64_t)j.rows * cq;
    const int m = ok ? (int)(t / cq) : 0, n = ok ? 4 * (int)(t % cq) : 0;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok) {
#pragma unroll 4
        for (int q = grp; q < splits; q += kRedGroups) {
            const float4 x = *reinterpret_cast<const float4*>(j.part + ((size_t)q * j.M + m) * j.N + n);
            s.x += x.x;
            s.y += x.y;
            s.z += x.z;
            s.w += x.w;
        }
    }
    red[grp][l32] = s;
    __syncthreads();
    if (grp != 0 || !ok) return;
#pragma unroll
    for (int g2 = 1; g2 < kRedGroups; ++g2) {
        const float4 x = red[g2][l32];
        s.x += x.x;
        s.y += x.y;
        s.z += x.z;
        s.w += x.w;
    }
    const float v[4] = {s.x, s.y, s.z, s.w};
    float* o = j.out + j.off + (int64_t)m * j.ld + j.col0 + n;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (n + e < j.cols) o[e] = v[e];
}

// ---------------------------------------------------------------------------
// Weights: flat float32 parameters (nerf_pack_mlp order, row-major) into
// padded matrices of the product element type
// ---------------------------------------------------------------------------
struct AsmBlock {
    int r0, c0, nr, nc;
    int64_t src;  // flat offset of element (0, 0)
    int src_ld;
    int transpose;  // dst[r0+i][c0+j] = flat[src + j*src_ld + i] instead of flat[src + i*src_ld + j]
};
struct AsmArgs {
    void* dst;
    int rows, ld, f32, nblocks;
    AsmBlock b[2];
};
// Up to kAsmJobs matrices per launch; job q covers elements start[q] ..
// start[q + 1] - 1 of the launch.
constexpr int kAsmJobs = 16;
struct AsmBatch {
    int n;
    int64_t start[kAsmJobs + 1];
    AsmArgs job[kAsmJobs];
};

template <class T>
__global__ void __launch_bounds__(256) k_assemble(AsmBatch bt, const float* flat) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= bt.start[bt.n]) return;
    int q = 0;
    while (q + 1 < bt.n && t >= bt.start[q + 1]) ++q;
    const AsmArgs& a = bt.job[q];
    const int64_t e = t - bt.start[q];
    const int r = (int)(e / a.ld), c = (int)(e % a.ld);
    float v = 0.0f;
    for (int k = 0; k < a.nblocks; ++k) {
        const AsmBlock& bk = a.b[k];
        const int i = r - bk.r0, j = c - bk.c0;
        if (i >= 0 && i < bk.nr && j >= 0 && j < bk.nc)
            v = flat[bk.src + (bk.transpose ? (int64_t)j * bk.src_ld + i : (int64_t)i * bk.src_ld + j)];
    }
    if (a.f32)
        ((float*)a.dst)[e] = v;
    else
        ((T*)a.dst)[e] = elt_from<T>(v);
}

// ---------------------------------------------------------------------------
// Samples, encodings, compositing with its gradient, loss, Adam
// ---------------------------------------------------------------------------

// Frequency encoding of a 3-vector into a padded row: [x, sin(2^k pi x) x3,
// cos(2^k pi x) x3 for k < L], zero padding to `ld`.
template <class T>
__device__ __forceinline__ void encode_row(const float (&x)[3], int L, int use_pi, T* row, int ld) {
    int c = 0;
#pragma unroll
    for (int a = 0; a < 3; ++a) row[c++] = elt_from<T>(x[a]);
    for (int k = 0; k < L; ++k) {
        float sn[3], cs[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const float arg = ldexpf(x[a], k);  // exact
            if (use_pi)
                sincospi_taylor(arg, sn[a], cs[a]);
            else
                sincosf(arg, &sn[a], &cs[a]);
        }
#pragma unroll
        for (int a = 0; a < 3; ++a) row[c++] = elt_from<T>(sn[a]);
#pragma unroll
        for (int a = 0; a < 3; ++a) row[c++] = elt_from<T>(cs[a]);
    }
    for (; c < ld; ++c) row[c] = elt_from<T>(0.0f);
}

// Sample depths (stratified, or the caller's z_in), points and position
// encodings.
template <class T>
__global__ void __launch_bounds__(256) k_train_samples(const float* __restrict__ ro, const float* __restrict__ rd,
                                                       const float* __restrict__ tn, const float* __restrict__ tf,
                                                       const float* __restrict__ z_in, int64_t R, int N,
                                                       uint64_t seed, uint64_t ray_offset, int jitter, int L,
                                                       int use_pi, float* __restrict__ z, T* E, int ldE) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= R * N) return;
    const int64_t r = s / N;
    const int i = (int)(s - r * N);
    float zi;
    if (z_in) {
        zi = z_in[s];
    } else {
        const float u = jitter ? philox_uniform(seed, ray_offset + (uint64_t)r, (uint32_t)i, kStreamJitter) : 0.5f;
        zi = stratified_z(tn[r], tf[r], i, N, u);
    }
    z[s] = zi;
    float x[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) x[k] = __fadd_rn(ro[3 * r + k], __fmul_rn(zi, rd[3 * r + k]));
    encode_row<T>(x, L, use_pi, E + s * ldE, ldE);
}

template <class T>
__global__ void __launch_bounds__(256) k_train_dirs(const float* __restrict__ rd, int64_t R, int L, int use_pi, T* V,
                                                    int ldV) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    const float d[3] = {rd[3 * r], rd[3 * r + 1], rd[3 * r + 2]};
    const float dn = sqrtf(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    const float v[3] = {d[0] / dn, d[1] / dn, d[2] / dn};
    encode_row<T>(v, L, use_pi, V + r * ldV, ldV);
}

constexpr int kTrainMaxSamples = 256;

// One wave per ray: compositing ("Spatial Intelligence - Part 1: NeRF",
// Section 2 Code, 5. Volume rendering in code), the ray's squared error and
// the gradient of the mean squared error with respect to raw = (rgb_raw,
// sigma_raw) of every sample.  With c = sigmoid(rgb_raw), s_i = 1 - alpha_i
// + 1e-10, T_i the exclusive product of s, w_i = T_i alpha_i and
// e_i = dL/drgb . c_i (white background: . (c_i - 1)):
//   dL/drgb_raw_i   = w_i dL/drgb * c_i (1 - c_i)
//   dL/dalpha_i     = T_i (e_i - R_i),  R_i = e_{i+1} alpha_{i+1} + s_{i+1} R_{i+1}
//   dL/dsigma_raw_i = dL/dalpha_i delta_i (1 - alpha_i) [sigma_raw_i > 0].
// R is a suffix recursion: affine maps x -> a + b x composed across the wave.
template <class T>
__global__ void __launch_bounds__(256) k_composite_train(const float* __restrict__ raw, const float* __restrict__ z,
                                                         const float* __restrict__ rd,
                                                         const float* __restrict__ target, int64_t R, int N,
                                                         int white, float inv_count, T* d_rgb, T* d_sig,
                                                         float* __restrict__ rgb_out, float* __restrict__ sq_err,
                                                         float* __restrict__ w_out) {
    struct Lds {
        float alpha[kTrainMaxSamples], s[kTrainMaxSamples], trans[kTrainMaxSamples], w[kTrainMaxSamples];
        float delta[kTrainMaxSamples], c[kTrainMaxSamples][3];
    };
    __shared__ Lds lds_all[4];
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= R) return;
    Lds& S = lds_all[wave];
    const float* zr = z + r * N;
    const float4* rr = reinterpret_cast<const float4*>(raw) + r * N;
    const float dx = rd[3 * r], dy = rd[3 * r + 1], dz = rd[3 * r + 2];
    const float dn = sqrtf(dx * dx + dy * dy + dz * dz);
    float carry = 1.0f, sr = 0.f, sg = 0.f, sb = 0.f, sa = 0.f;
    for (int base = 0; base < N; base += kWave) {
        const int i = base + lane;
        const bool valid = i < N;
        float alpha = 0.0f, delta = 0.0f;
        float4 rw = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
            delta = (i + 1 < N) ? (zr[i + 1] - zr[i]) * dn : 1e10f * dn;
            rw = rr[i];
            alpha = 1.0f - expf(-fmaxf(rw.w, 0.0f) * delta);
        }
        const float s = valid ? 1.0f - alpha + 1e-10f : 1.0f;
        const float incl = wave_scan_mul(s);
        float excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 1.0f;
        const float Ti = carry * excl;
        const float w = valid ? Ti * alpha : 0.0f;
        const float c0 = sigmoidf_(rw.x), c1 = sigmoidf_(rw.y), c2 = sigmoidf_(rw.z);
        if (valid) {
            S.alpha[i] = alpha;
            S.s[i] = s;
            S.trans[i] = Ti;
            S.w[i] = w;
            S.delta[i] = delta;
            S.c[i][0] = c0;
            S.c[i][1] = c1;
            S.c[i][2] = c2;
            if (w_out) w_out[r * N + i] = w;
            sr += w * c0;
            sg += w * c1;
            sb += w * c2;
            sa += w;
        }
        carry *= __shfl(incl, kWave - 1, kWave);
    }
    sr = wave_sum(sr);
    sg = wave_sum(sg);
    sb = wave_sum(sb);
    sa = wave_sum(sa);
    const float bg = white ? 1.0f - sa : 0.0f;
    const float rgb[3] = {sr + bg, sg + bg, sb + bg};
    float g[3], sq = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float e = rgb[k] - target[3 * r + k];
        g[k] = 2.0f * e * inv_count;
        sq += e * e;
    }
    if (lane == 0) {
        sq_err[r] = sq;
        if (rgb_out)
            for (int k = 0; k < 3; ++k) rgb_out[3 * r + k] = rgb[k];
    }
    wave_lds_sync();
    const float cw = white ? 1.0f : 0.0f;
    float carry_R = 0.0f;  // R at the last sample of the chunk after the current one
    const int last_base = (N - 1) / kWave * kWave;
    for (int base = last_base; base >= 0; base -= kWave) {
        const int i = base + lane;
        const bool valid = i < N;
        float e = 0.0f, a = 0.0f, b = 1.0f;
        if (valid) {
            e = g[0] * (S.c[i][0] - cw) + g[1] * (S.c[i][1] - cw) + g[2] * (S.c[i][2] - cw);
            a = e * S.alpha[i];
            b = S.s[i];
        }
        // inclusive suffix composition h_i = f_i o f_{i+1} o ... o f_63, f(x) = a + b x
        float A = a, B = b;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float A2 = __shfl_down(A, off, kWave), B2 = __shfl_down(B, off, kWave);
            if (lane + off < kWave) {
                A = A + B * A2;
                B = B * B2;
            }
        }
        float An = __shfl_down(A, 1, kWave), Bn = __shfl_down(B, 1, kWave);
        if (lane == kWave - 1) {
            An = 0.0f;
            Bn = 1.0f;
        }
        const float Ri = An + Bn * carry_R;
        carry_R = __shfl(A, 0, kWave) + __shfl(B, 0, kWave) * carry_R;
        if (valid) {
            const int64_t sidx = r * N + i;
            const float d_alpha = S.trans[i] * (e - Ri);
            const float d_sigma = rr[i].w > 0.0f ? d_alpha * S.delta[i] * (1.0f - S.alpha[i]) : 0.0f;
            T* dr = d_rgb + sidx * 32;
            T* ds = d_sig + sidx * 32;
#pragma unroll
            for (int k = 0; k < 3; ++k) dr[k] = elt_from<T>(S.w[i] * g[k] * S.c[i][k] * (1.0f - S.c[i][k]));
            for (int k = 3; k < 32; ++k) dr[k] = elt_from<T>(0.0f);
            ds[0] = elt_from<T>(d_sigma);
            for (int k = 1; k < 32; ++k) ds[k] = elt_from<T>(0.0f);
        }
    }
}

}  // namespace

namespace {

// bfloat16 products with whole-width bfloat16 outputs: the direct-copy kernel
void gemm_nt_dma(const GemmNT& g, hipStream_t s) {
    const unsigned gx4 = (unsigned)((g.M + 255) / 256), gx2 = (unsigned)((g.M + 127) / 128);
    if (g.N > 128)
        hipLaunchKernelGGL((k_gemm_nt_dma<4, 2, 2>), dim3(gx2, (unsigned)((g.N + 255) / 256)), dim3(256), 0, s, g);
    else if (g.N > 64)
        hipLaunchKernelGGL((k_gemm_nt_dma<2, 2>), dim3(gx2, 1), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((k_gemm_nt_dma<1, 4>), dim3(gx4, 1), dim3(256), 0, s, g);
}

template <class T>
void gemm_nt(const GemmNT& g, hipStream_t s) {
    // tile rows: the product's columns n (weights); tile columns: its rows m (samples)
    const unsigned gx4 = (unsigned)((g.M + 255) / 256), gx2 = (unsigned)((g.M + 127) / 128);
    if constexpr (sizeof(T) == 2) {
        if (!g.c_f32 && g.n_store == g.N && g.c_col0 == 0) {
            gemm_nt_dma(g, s);
            return;
        }
    }
    if (g.N > 128)
        hipLaunchKernelGGL((k_gemm_nt<T, 4, 2>), dim3(gx2, (unsigned)((g.N + 255) / 256)), dim3(256), 0, s, g);
    else if (g.N > 64)
        hipLaunchKernelGGL((k_gemm_nt<T, 2, 2>), dim3(gx2, 1), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((k_gemm_nt<T, 1, 4>), dim3(gx4, 1), dim3(256), 0, s, g);
}

// Weight gradient of one input segment: part = A^T B over each split of the
// samples, then the ordered reduction into the flat gradient; with b_off >= 0
// also the bias gradient (the column sums of A).
template <class T>
void grad_w(const TrainBufs& b, const void* dpre, int ld_dpre, int rows, int rows_pad, const void* in, int ld_in,
            int cols, int cols_pad, int row_div, int64_t S, float* grad, int64_t w_off, int in_total, int col0,
            int64_t b_off, hipStream_t s) {
    GemmTN g{};
    g.a = dpre;
    g.lda = ld_dpre;
    g.M = rows_pad;
    g.b = in;
    g.ldb = ld_in;
    g.N = cols_pad;
    g.b_row_div = row_div;
    g.K = (int)S;
    g.k_chunk = b.k_chunk;
    g.part = (float*)b.ptr[BPART];
    g.bpart = b_off >= 0 ? (float*)b.ptr[BBPART] : nullptr;
    const int RB = rows_pad > 64 ? 2 : 1, CB = cols_pad > 64 ? 2 : 1;
    const int tiles = ((rows_pad + 64 * RB - 1) / (64 * RB)) * ((cols_pad + 64 * CB - 1) / (64 * CB));
    const dim3 grid((unsigned)(tiles * ((b.splits + 7) / 8 * 8)));  // XCD-grouped, see k_gemm_tn
    if (row_div != 1) {  // B rows per ray: the direction encodings, 32 columns in every network
        if (RB == 2)
            hipLaunchKernelGGL((k_gemm_tn<T, 2, 1, true>), grid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_gemm_tn<T, 1, 1, true>), grid, dim3(256), 0, s, g);
    } else if (RB == 2 && CB == 2)
        hipLaunchKernelGGL((k_gemm_tn<T, 2, 2, false>), grid, dim3(256), 0, s, g);
    else if (RB == 2)
        hipLaunchKernelGGL((k_gemm_tn<T, 2, 1, false>), grid, dim3(256), 0, s, g);
    else if (CB == 2)
        hipLaunchKernelGGL((k_gemm_tn<T, 1, 2, false>), grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((k_gemm_tn<T, 1, 1, false>), grid, dim3(256), 0, s, g);
    const RedJob rw = red_job((const float*)b.ptr[BPART], rows_pad, cols_pad, rows, cols, grad, w_off, in_total, col0);
    // bias partials [split][rows_pad]: one row of rows_pad columns per split
    RedJob rbias = red_job((const float*)b.ptr[BBPART], 1, rows_pad, 1, rows, grad, b_off, 0, 0);
    if (b_off < 0) rbias.blocks = 0;
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)(rw.blocks + rbias.blocks)), dim3(256), 0, s, rw, rbias, b.splits);
}

// Collects weight-assembly jobs and launches them kAsmJobs at a time.
template <class T>
struct Assembler {
    const float* flat;
    hipStream_t s;
    AsmBatch bt{};

    void add(void* dst, int rows, int ld, int f32, std::initializer_list<AsmBlock> blocks) {
        if (bt.n == kAsmJobs) flush();
        AsmArgs& a = bt.job[bt.n];
        a = AsmArgs{};
        a.dst = dst;
        a.rows = rows;
        a.ld = ld;
        a.f32 = f32;
        for (const AsmBlock& k : blocks) a.b[a.nblocks++] = k;
        bt.start[bt.n + 1] = bt.start[bt.n] + (int64_t)rows * ld;
        ++bt.n;
    }
    void flush() {
        if (bt.n == 0) return;
        const int64_t n = bt.start[bt.n];
        hipLaunchKernelGGL(k_assemble<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, bt, flat);
        bt = AsmBatch{};
    }
};

template <class T>
void train_step_t(int kind, const TrainArgs& t, hipStream_t s) {
    const NetPlan p = make_plan(kind);
    const Layer* L = net_layers(kind);
    TrainBufs b{};
    train_workspace_layout(kind, sizeof(T) == 2, t.n_rays, t.n_samples, (char*)t.workspace, &b);
    const int64_t R = t.n_rays, S = R * t.n_samples;
    const int N = t.n_samples, W = p.W, D = p.D;
    const int nl = D + 4;
    const int SIG = D, FEAT = D + 1, DIR = D + 2, RGB = D + 3;
    float* grad = t.grad ? t.grad : (float*)b.ptr[BGRAD];

    // --- weights of this step ------------------------------------------------
    Assembler<T> as{t.params, s};
    for (int l = 0; l < nl; ++l) {
        const int no = pad32(L[l].n_out);
        const int w1 = L[l].s0.width, w2 = L[l].s1.width;
        const int k1 = L[l].s0.kind == SEG_HIDDEN ? pad32(w1) : p.ldE;
        const int k2 = L[l].s1.kind == SEG_NONE ? 0 : (l == DIR ? p.ldV : p.ldE);
        const int it = p.in_total[l];
        if (k2)
            as.add(b.wf[l], no, k1 + k2, 0,
                   {AsmBlock{0, 0, L[l].n_out, w1, p.w_off[l], it, 0},
                    AsmBlock{0, k1, L[l].n_out, w2, p.w_off[l] + w1, it, 0}});
        else
            as.add(b.wf[l], no, k1, 0, {AsmBlock{0, 0, L[l].n_out, w1, p.w_off[l], it, 0}});
        as.add(b.wt[l], k1, no, 0, {AsmBlock{0, 0, w1, L[l].n_out, p.w_off[l], it, 1}});
        as.add(b.bias[l], 1, no, 1, {AsmBlock{0, 0, 1, L[l].n_out, p.b_off[l], 0, 0}});
    }
    // d(last hidden) = [dF, dSIG] [W_feature^T ; W_sigma^T]
    as.add(b.wt_head, W, W + 32, 0,
           {AsmBlock{0, 0, W, W, p.w_off[FEAT], W, 1}, AsmBlock{0, W, W, 1, p.w_off[SIG], W, 1}});
    as.flush();

    // --- samples and encodings -----------------------------------------------
    hipLaunchKernelGGL(k_train_samples<T>, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, s, t.ro, t.rd, t.tn, t.tf,
                       t.z_in, R, N, t.seed, t.ray_offset, t.jitter, p.Lpos, t.use_pi, (float*)b.ptr[BZ],
                       (T*)b.ptr[BE], p.ldE);
    hipLaunchKernelGGL(k_train_dirs<T>, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s, t.rd, R, p.Ldir, t.use_pi,
                       (T*)b.ptr[BV], p.ldV);

    // --- forward -------------------------------------------------------------
    auto H = [&](int l) { return b.ptr[BH0 + l]; };
    for (int l = 0; l < D; ++l) {
        GemmNT g{};
        g.a0 = l == 0 ? SegA{b.ptr[BE], p.ldE, p.ldE, 1} : SegA{H(l - 1), W, W, 1};
        if (L[l].s1.kind == SEG_ENC) g.a1 = SegA{b.ptr[BE], p.ldE, p.ldE, 1};
        g.b = b.wf[l];
        g.ldb = g.a0.kpad + g.a1.kpad;
        g.M = (int)S;
        g.N = W;
        g.bias = b.bias[l];
        g.relu = 1;
        g.c = H(l);
        g.ldc = W;
        g.n_store = W;
        g.bits_out = b.hbits[l];  // bfloat16 steps only (NULL otherwise)
        g.ldbits = W / 8;
        gemm_nt<T>(g, s);
    }
    {
        GemmNT g{};  // density head -> raw column 3 (float32)
        g.a0 = SegA{H(D - 1), W, W, 1};
        g.b = b.wf[SIG];
        g.ldb = W;
        g.M = (int)S;
        g.N = 32;
        g.bias = b.bias[SIG];
        g.c = b.ptr[BRAW];
        g.ldc = 4;
        g.c_col0 = 3;
        g.n_store = 1;
        g.c_f32 = 1;
        gemm_nt<T>(g, s);
        g.b = b.wf[FEAT];  // feature (no activation)
        g.N = W;
        g.bias = b.bias[FEAT];
        g.c = b.ptr[BF];
        g.ldc = W;
        g.c_col0 = 0;
        g.n_store = W;
        g.c_f32 = 0;
        gemm_nt<T>(g, s);
        g.a0 = SegA{b.ptr[BF], W, W, 1};  // direction layer on [feature, direction encoding of the ray]
        g.a1 = SegA{b.ptr[BV], p.ldV, p.ldV, N};
        g.b = b.wf[DIR];
        g.ldb = W + p.ldV;
        g.N = p.ldG;
        g.bias = b.bias[DIR];
        g.relu = 1;
        g.c = b.ptr[BG];
        g.ldc = p.ldG;
        g.n_store = p.ldG;
        g.bits_out = b.gbits;
        g.ldbits = p.ldG / 8;
        gemm_nt<T>(g, s);
        g.bits_out = nullptr;
        g.a0 = SegA{b.ptr[BG], p.ldG, p.ldG, 1};  // rgb head -> raw columns 0..2
        g.a1 = SegA{};
        g.b = b.wf[RGB];
        g.ldb = p.ldG;
        g.N = 32;
        g.bias = b.bias[RGB];
        g.relu = 0;
        g.c = b.ptr[BRAW];
        g.ldc = 4;
        g.n_store = 3;
        g.c_f32 = 1;
        gemm_nt<T>(g, s);
    }

    // --- compositing, loss and d raw -------------------------------------------
    const float inv_count = (float)(1.0 / (3.0 * (double)R));
    hipLaunchKernelGGL(k_composite_train<T>, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s,
                       (const float*)b.ptr[BRAW], (const float*)b.ptr[BZ], t.rd, t.target, R, N, t.white, inv_count,
                       (T*)b.ptr[BDRGB], (T*)b.ptr[BDSIG], t.rgb_out, (float*)b.ptr[BSQ], t.w_out);
    hipLaunchKernelGGL(k_train_loss, dim3(1), dim3(256), 0, s, (const float*)b.ptr[BSQ], R, inv_count, t.loss);

    // --- backward ----------------------------------------------------------------
    // rgb head
    grad_w<T>(b, b.ptr[BDRGB], 32, 3, 32, b.ptr[BG], p.ldG, p.DW, p.ldG, 1, S, grad, p.w_off[RGB], p.in_total[RGB], 0,
              p.b_off[RGB], s);
    {
        GemmNT g{};  // dG = dRGB W_rgb, masked by G > 0
        g.a0 = SegA{b.ptr[BDRGB], 32, 32, 1};
        g.b = b.wt[RGB];
        g.ldb = 32;
        g.M = (int)S;
        g.N = p.ldG;
        g.mask = b.ptr[BG];
        g.ldm = p.ldG;
        g.bits_in = b.gbits;  // used instead of mask where present
        g.ldbits = p.ldG / 8;
        g.c = b.ptr[BDG];
        g.ldc = p.ldG;
        g.n_store = p.ldG;
        gemm_nt<T>(g, s);
    }
    // direction layer: weights over [feature, direction encoding]
    grad_w<T>(b, b.ptr[BDG], p.ldG, p.DW, p.ldG, b.ptr[BF], W, W, W, 1, S, grad, p.w_off[DIR], p.in_total[DIR], 0,
              p.b_off[DIR], s);
    grad_w<T>(b, b.ptr[BDG], p.ldG, p.DW, p.ldG, b.ptr[BV], p.ldV, p.de, p.ldV, N, S, grad, p.w_off[DIR],
              p.in_total[DIR], W, -1, s);
    {
        GemmNT g{};  // dF = dG W_dir[:, :W]
        g.a0 = SegA{b.ptr[BDG], p.ldG, p.ldG, 1};
        g.b = b.wt[DIR];
        g.ldb = pad32(p.DW);
        g.M = (int)S;
        g.N = W;
        g.c = b.ptr[BDF];
        g.ldc = W;
        g.n_store = W;
        gemm_nt<T>(g, s);
    }
    // feature and density heads
    grad_w<T>(b, b.ptr[BDF], W, W, W, H(D - 1), W, W, W, 1, S, grad, p.w_off[FEAT], W, 0, p.b_off[FEAT], s);
    grad_w<T>(b, b.ptr[BDSIG], 32, 1, 32, H(D - 1), W, W, W, 1, S, grad, p.w_off[SIG], W, 0, p.b_off[SIG], s);
    void* dh = b.ptr[BDH0];
    void* dh_next = b.ptr[BDH1];
    {
        GemmNT g{};  // d(last hidden) = [dF, dSIG] [W_feature ; W_sigma], masked
        g.a0 = SegA{b.ptr[BDF], W, W, 1};
        g.a1 = SegA{b.ptr[BDSIG], 32, 32, 1};
        g.b = b.wt_head;
        g.ldb = W + 32;
        g.M = (int)S;
        g.N = W;
        g.mask = H(D - 1);
        g.ldm = W;
        g.bits_in = b.hbits[D - 1];
        g.ldbits = W / 8;
        g.c = dh;
        g.ldc = W;
        g.n_store = W;
        gemm_nt<T>(g, s);
    }
    // hidden layers, last to first
    for (int l = D - 1; l >= 0; --l) {
        if (l == 0) {
            grad_w<T>(b, dh, W, W, W, b.ptr[BE], p.ldE, p.pe, p.ldE, 1, S, grad, p.w_off[0], p.in_total[0], 0,
                      p.b_off[0], s);
        } else {
            grad_w<T>(b, dh, W, W, W, H(l - 1), W, W, W, 1, S, grad, p.w_off[l], p.in_total[l], 0, p.b_off[l], s);
            if (L[l].s1.kind == SEG_ENC)
                grad_w<T>(b, dh, W, W, W, b.ptr[BE], p.ldE, p.pe, p.ldE, 1, S, grad, p.w_off[l], p.in_total[l], W,
                          -1, s);
        }
        if (l > 0) {
            GemmNT g{};  // d(previous hidden) = d_pre W_l[:, :W], masked by that layer's output
            g.a0 = SegA{dh, W, W, 1};
            g.b = b.wt[l];
            g.ldb = W;
            g.M = (int)S;
            g.N = W;
            g.mask = H(l - 1);
            g.ldm = W;
            g.bits_in = b.hbits[l - 1];
            g.ldbits = W / 8;
            g.c = dh_next;
            g.ldc = W;
            g.n_store = W;
            gemm_nt<T>(g, s);
            void* tmp = dh;
            dh = dh_next;
            dh_next = tmp;
        }
    }

    // --- Adam ------------------------------------------------------------------
    if (t.adam_m && t.adam_v && t.step >= 1)
        adam_step(t.params, t.adam_m, t.adam_v, grad, p.P, t.lr, t.beta1, t.beta2, t.eps, t.step, s);
}

}  // namespace

void launch_train_step(int kind, int bf16, const TrainArgs& t, hipStream_t s) {
    if (bf16)
        train_step_t<__bf16>(kind, t, s);
    else
        train_step_t<float>(kind, t, s);
}

}  // namespace nerf

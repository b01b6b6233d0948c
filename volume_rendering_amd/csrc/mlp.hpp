// Fused radiance-network evaluation on the gfx950 matrix cores.
//
// One wave evaluates the network on 32*SB samples (bf16: 64, f32: 32).
// Activations never leave registers: a layer's accumulators are rounded
// (bf16) or copied (f32) straight into the B operands of the next layer
// (layout in nets.hpp).  Weight tiles are read from the packed buffer in
// the order the layer loops consume them.  Layers run output-block major so
// only 32*SB accumulators are live at a time, next to the input and output
// activations of the layer.
#pragma once

#include "common.hpp"
#include "nets.hpp"

namespace nerf {

struct TBF16 {
    static constexpr int prec = PREC_BF16;
    static constexpr int SB = 2;
    using Op = bf16x8;
    __device__ static __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

struct TF32 {
    static constexpr int prec = PREC_F32;
    static constexpr int SB = 1;
    using Op = float;
    __device__ static __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

template <class T, int KIND, int LAYER>
struct LayerInfo {
    static constexpr Layer L = net_layers(KIND)[LAYER];
    static constexpr int S1 = seg_steps(L.s0, T::prec);
    static constexpr int S2 = seg_steps(L.s1, T::prec);
    static constexpr int OB = out_blocks(L.n_out);
    static constexpr size_t tiles = net_tile_offset(KIND, T::prec, LAYER);
    static constexpr size_t bias = net_bias_offset(KIND, T::prec, LAYER);
};

// Steps of the output of LAYER as an input of the next layer.
template <class T, int KIND, int LAYER>
constexpr int out_steps() {
    return seg_steps(Seg{SEG_HIDDEN, net_layers(KIND)[LAYER].n_out, 0}, T::prec);
}

__device__ __forceinline__ f32x16 load_bias16(const float* __restrict__ bias, int ob, int h) {
    const f32x4* p = reinterpret_cast<const f32x4*>(bias) + (ob * 2 + h) * 4;
    const f32x4 a = p[0], b = p[1], c = p[2], d = p[3];
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const f32x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x8 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

template <class T, int S1, int S2, class In1, class In2>
__device__ __forceinline__ void mma_block(f32x16 (&acc)[T::SB], const In1& in1, const In2& in2,
                                          const typename T::Op* __restrict__ t, int lane) {
#pragma unroll
    for (int s = 0; s < S1; ++s) {
        const typename T::Op a = t[s * kWave + lane];
#pragma unroll
        for (int sb = 0; sb < T::SB; ++sb) acc[sb] = T::mma(a, in1[s][sb], acc[sb]);
    }
#pragma unroll
    for (int s = 0; s < S2; ++s) {
        const typename T::Op a = t[(S1 + s) * kWave + lane];
#pragma unroll
        for (int sb = 0; sb < T::SB; ++sb) acc[sb] = T::mma(a, in2[s][sb], acc[sb]);
    }
}

template <bool RELU>
__device__ __forceinline__ float act(float v) {
    return RELU ? fmaxf(v, 0.0f) : v;
}

template <bool RELU, class Out>
__device__ __forceinline__ void store_hidden(TBF16, const f32x16 (&acc)[2], Out& out, int ob) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = to_bf16(act<RELU>(acc[sb][8 * q + j]));
            out[2 * ob + q][sb] = v;
        }
}

template <bool RELU, class Out>
__device__ __forceinline__ void store_hidden(TF32, const f32x16 (&acc)[1], Out& out, int ob) {
#pragma unroll
    for (int r = 0; r < 16; ++r) out[16 * ob + r][0] = act<RELU>(acc[0][r]);
}

// A hidden layer: out = act(W [in1, in2] + b), kept as next-layer operands.
template <class T, int KIND, int LAYER, class In1, class In2, class Out>
__device__ __forceinline__ void dense_layer(const In1& in1, const In2& in2, Out& out, const char* __restrict__ packed,
                                            int lane) {
    using I = LayerInfo<T, KIND, LAYER>;
    const typename T::Op* tiles = reinterpret_cast<const typename T::Op*>(packed + I::tiles);
    const float* bias = reinterpret_cast<const float*>(packed + I::bias);
    const int h = lane >> 5;
#pragma unroll
    for (int ob = 0; ob < I::OB; ++ob) {
        const f32x16 b = load_bias16(bias, ob, h);
        f32x16 acc[T::SB];
#pragma unroll
        for (int sb = 0; sb < T::SB; ++sb) acc[sb] = b;
        mma_block<T, I::S1, I::S2>(acc, in1, in2, tiles + (size_t)ob * (I::S1 + I::S2) * kWave, lane);
        store_hidden<I::L.relu != 0>(T{}, acc, out, ob);
    }
}

// A head (one output block, no activation): raw accumulators.
template <class T, int KIND, int LAYER, class In1, class In2>
__device__ __forceinline__ void dense_head(const In1& in1, const In2& in2, f32x16 (&acc)[T::SB],
                                           const char* __restrict__ packed, int lane) {
    using I = LayerInfo<T, KIND, LAYER>;
    static_assert(I::OB == 1, "head layers have one output block");
    const typename T::Op* tiles = reinterpret_cast<const typename T::Op*>(packed + I::tiles);
    const float* bias = reinterpret_cast<const float*>(packed + I::bias);
    const f32x16 b = load_bias16(bias, 0, lane >> 5);
#pragma unroll
    for (int sb = 0; sb < T::SB; ++sb) acc[sb] = b;
    mma_block<T, I::S1, I::S2>(acc, in1, in2, tiles, lane);
}

// ---------------------------------------------------------------------------
// NeRF family: hidden layers 0..D-1 (skip segment where the layer has one),
// then density head D, feature D+1, direction layer D+2, rgb head D+3.
// ---------------------------------------------------------------------------
template <int KIND>
struct NerfFamily {
    static constexpr int D = net_n_layers(KIND) - 4;
    static constexpr int LPOS = net_layers(KIND)[0].s0.L;
    static constexpr int LDIR = net_layers(KIND)[D + 2].s1.L;
};

template <class T, int KIND, int I, int D, class H, class E>
__device__ __forceinline__ void hidden_chain(H& cur, H& nxt, const E& enc, const char* __restrict__ packed, int lane) {
    if constexpr (I < D) {
        dense_layer<T, KIND, I>(cur, enc, nxt, packed, lane);  // enc is read only by a skip layer (S2 > 0)
        hidden_chain<T, KIND, I + 1, D>(nxt, cur, enc, packed, lane);
    }
}

// enc: position-encoding operands; denc: direction-encoding operands.
// sig[sb] accumulator 0 and rgb[sb] accumulators 0..2 of lanes 0..31 hold the
// outputs of sample (sb*32 + lane).
template <class T, int KIND, class E, class DE>
__device__ __forceinline__ void nerf_forward(const E& enc, const DE& denc, const char* __restrict__ packed,
                                             f32x16 (&sig)[T::SB], f32x16 (&rgb)[T::SB], int lane) {
    using Fam = NerfFamily<KIND>;
    constexpr int D = Fam::D;
    constexpr int HS = out_steps<T, KIND, 0>();
    constexpr int GS = out_steps<T, KIND, D + 2>();
    typename T::Op hA[HS][T::SB], hB[HS][T::SB];
    dense_layer<T, KIND, 0>(enc, enc, hA, packed, lane);
    hidden_chain<T, KIND, 1, D>(hA, hB, enc, packed, lane);
    // the last hidden layer (index D-1) wrote hB when D-1 is odd, else hA
    auto& hl = ((D - 1) % 2 == 1) ? hB : hA;
    auto& hf = ((D - 1) % 2 == 1) ? hA : hB;
    dense_head<T, KIND, D>(hl, hl, sig, packed, lane);
    dense_layer<T, KIND, D + 1>(hl, hl, hf, packed, lane);
    typename T::Op g[GS][T::SB];
    dense_layer<T, KIND, D + 2>(hf, denc, g, packed, lane);
    dense_head<T, KIND, D + 3>(g, g, rgb, packed, lane);
}

// Hash-grid field: density 0, 1; density head 2; feature 3; colour 4 (with
// harmonics), 5; rgb head 6.
template <class T, class FE, class DE>
__device__ __forceinline__ void hash_field_forward(const FE& feats, const DE& sh, const char* __restrict__ packed,
                                                   f32x16 (&sig)[T::SB], f32x16 (&rgb)[T::SB], int lane) {
    constexpr int K = NET_HASH_FIELD;
    constexpr int HS = out_steps<T, K, 0>();
    typename T::Op hA[HS][T::SB], hB[HS][T::SB];
    dense_layer<T, K, 0>(feats, feats, hA, packed, lane);
    dense_layer<T, K, 1>(hA, hA, hB, packed, lane);
    dense_head<T, K, 2>(hB, hB, sig, packed, lane);
    dense_layer<T, K, 3>(hB, hB, hA, packed, lane);
    dense_layer<T, K, 4>(hA, sh, hB, packed, lane);
    dense_layer<T, K, 5>(hB, hB, hA, packed, lane);
    dense_head<T, K, 6>(hA, hA, rgb, packed, lane);
}

// ---------------------------------------------------------------------------
// Input operands
// ---------------------------------------------------------------------------

// Value pair P of the frequency encoding of (x0, x1, x2) with L frequencies.
__device__ __forceinline__ void enc_pair_value(int P, int L, float x0, float x1, float x2, bool use_pi, float& a,
                                               float& b) {
    if (P < 3 * L) {
        const int k = P / 3;
        const int ax = P - 3 * k;
        const float v = ax == 0 ? x0 : (ax == 1 ? x1 : x2);
        const float arg = ldexpf(v, k);  // exact
        if (use_pi)
            sincospif(arg, &a, &b);
        else
            sincosf(arg, &a, &b);
    } else if (P == 3 * L) {
        a = x0;
        b = x1;
    } else if (P == 3 * L + 1) {
        a = x2;
        b = 0.0f;
    } else {
        a = 0.0f;
        b = 0.0f;
    }
}

template <int NS>
__device__ __forceinline__ void enc_operands(bf16x8 (&enc)[NS][2], int L, const float (&x)[2][3], bool use_pi,
                                             int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            bf16x8 v;
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                float a, b;
                enc_pair_value(8 * s + 4 * h + jp, L, x[sb][0], x[sb][1], x[sb][2], use_pi, a, b);
                v[2 * jp] = to_bf16(a);
                v[2 * jp + 1] = to_bf16(b);
            }
            enc[s][sb] = v;
        }
}

template <int NS>
__device__ __forceinline__ void enc_operands(float (&enc)[NS][1], int L, const float (&x)[1][3], bool use_pi,
                                             int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int p = 0; p < NS / 2; ++p) {
        float a, b;
        enc_pair_value(2 * p + h, L, x[0][0], x[0][1], x[0][2], use_pi, a, b);
        enc[2 * p][0] = a;
        enc[2 * p + 1][0] = b;
    }
}

// Operands of a segment read from a row-major float32 matrix (`row[sb]`
// points at the sample's row), following the packer's slot order.
template <int NS>
__device__ __forceinline__ void row_operands(bf16x8 (&op)[NS][2], Seg seg, const float* const (&row)[2], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = seg_col(seg, PREC_BF16, s, h, j);
                v[j] = to_bf16(c >= 0 ? row[sb][c] : 0.0f);
            }
            op[s][sb] = v;
        }
}

template <int NS>
__device__ __forceinline__ void row_operands(float (&op)[NS][1], Seg seg, const float* const (&row)[1], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c = seg_col(seg, PREC_F32, s, h, 0);
        op[s][0] = c >= 0 ? row[0][c] : 0.0f;
    }
}

}  // namespace nerf

// Standalone network evaluation on encoded inputs (kernel template).
#pragma once

#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "mlp.hpp"

namespace nerf {

constexpr int kMlpRing = 8;  // 128 KB weight ring

// ===========================================================================
// Standalone network evaluation on encoded inputs: one wave per 32*SB
// samples.
// ===========================================================================
template <class T, int KIND>
__global__ void __launch_bounds__(256) k_mlp(const char* __restrict__ packed, const float* __restrict__ enc_x,
                                             const float* __restrict__ enc_v, int64_t n, int spr,
                                             float* __restrict__ raw) {
    constexpr int NL = net_n_layers(KIND);
    constexpr Layer L0 = net_layers(KIND)[0];
    // the layer that takes the direction input as its second segment
    constexpr int DL = (KIND == NET_HASH_FIELD) ? 4 : NL - 2;
    constexpr Layer LD = net_layers(KIND)[DL];
    constexpr int ES = seg_steps(L0.s0, T::prec);
    constexpr int DS = seg_steps(LD.s1, T::prec);
    constexpr int M = 32 * T::SB;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // every wave of the workgroup runs the network (the weight ring is shared);
    // waves past the end compute on clamped rows and store nothing
    const int64_t base = ((int64_t)blockIdx.x * 4 + wave) * M;
    const float* xr[T::SB];
    const float* vr[T::SB];
#pragma unroll
    for (int sb = 0; sb < T::SB; ++sb) {
        int64_t s = base + sb * 32 + (lane & 31);
        if (s >= n) s = n - 1;
        xr[sb] = enc_x + s * L0.s0.width;
        vr[sb] = enc_v + (s / spr) * LD.s1.width;
    }
    typename T::Op enc[ES][T::SB], denc[DS][T::SB];
    row_operands(enc, L0.s0, xr, lane);
    row_operands(denc, LD.s1, vr, lane);
    __shared__ __attribute__((aligned(16))) float bias_lds[BiasRegion<KIND, T::prec>::floats];
    bias_to_lds<KIND, T::prec>((NERF_AS_LDS float*)bias_lds, packed, threadIdx.x, blockDim.x);
    __syncthreads();
    const NERF_AS_LDS float* bias = (const NERF_AS_LDS float*)bias_lds;
    f32x16 sig[T::SB], rgb[T::SB];
    if constexpr (kLoopedF32<T, KIND>) {
        nerf_forward_f32_loop<KIND>(enc, denc, packed, bias, sig, rgb, lane);
    } else {
        LdsStream<T, KIND, kMlpRing> ws(packed, lane, wave);
        if constexpr (KIND == NET_HASH_FIELD)
            hash_field_forward<T>(enc, denc, ws, bias, sig, rgb, lane);
        else
            nerf_forward<T, KIND>(enc, denc, ws, bias, sig, rgb, lane);
    }
    if (lane < 32) {
#pragma unroll
        for (int sb = 0; sb < T::SB; ++sb) {
            const int64_t s = base + sb * 32 + lane;
            if (s < n) reinterpret_cast<f32x4*>(raw)[s] = f32x4{rgb[sb][0], rgb[sb][1], rgb[sb][2], sig[sb][0]};
        }
    }
}

template <class T, int KIND>
static void launch_mlp_t(const void* packed, const float* ex, const float* ev, int64_t n, int spr, float* raw,
                         hipStream_t s) {
    constexpr int M = 32 * T::SB;
    const int64_t waves = (n + M - 1) / M;
    hipLaunchKernelGGL((k_mlp<T, KIND>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const char*)packed, ex,
                       ev, n, spr, raw);
}

}  // namespace nerf

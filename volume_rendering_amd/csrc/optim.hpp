// Kernels shared by the training steps: the loss as an ordered sum, and
// Adam (Kingma and Ba, "Adam: A Method for Stochastic Optimization",
// Algorithm 1) with bias correction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace nerf {
namespace {

// loss = scale * sum of vals[0..n), accumulated in float64 in a fixed order
// (one workgroup of 256 threads).
__global__ void __launch_bounds__(256) k_train_loss(const float* __restrict__ vals, int64_t n, float scale,
                                                    float* __restrict__ loss) {
    __shared__ double part[256];
    double s = 0.0;
    for (int64_t r = threadIdx.x; r < n; r += blockDim.x) s += (double)vals[r];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
        if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = (float)(part[0] * (double)scale);
}

// Adam on parameter i given its gradient gi; c1 = 1/(1-b1^t), c2 = 1/(1-b2^t).
__device__ __forceinline__ void adam_update(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
                                            int64_t i, float gi, float lr, float b1, float b2, float eps, float c1,
                                            float c2) {
    const float mi = b1 * m[i] + (1.0f - b1) * gi;
    const float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
    m[i] = mi;
    v[i] = vi;
    p[i] -= lr * (mi * c1) / (sqrtf(vi * c2) + eps);
}

// One Adam step on P parameters.
__global__ void __launch_bounds__(256) k_adam(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
                                              const float* __restrict__ g, int64_t P, float lr, float b1, float b2,
                                              float eps, float c1, float c2) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= P) return;
    adam_update(p, m, v, i, g[i], lr, b1, b2, eps, c1, c2);
}

// Bias corrections of step t >= 1, computed in float64 on the host.
inline void adam_corrections(float b1, float b2, int64_t t, float* c1, float* c2) {
    *c1 = (float)(1.0 / (1.0 - std::pow((double)b1, (double)t)));
    *c2 = (float)(1.0 / (1.0 - std::pow((double)b2, (double)t)));
}

// Launches the Adam step for step t >= 1.
inline void adam_step(float* p, float* m, float* v, const float* g, int64_t P, float lr, float b1, float b2, float eps,
                      int64_t t, hipStream_t s) {
    float c1, c2;
    adam_corrections(b1, b2, t, &c1, &c2);
    hipLaunchKernelGGL(k_adam, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, s, p, m, v, g, P, lr, b1, b2, eps, c1,
                       c2);
}

}  // namespace
}  // namespace nerf

// Fused hash-grid field render kernels and the render dispatch.
#include "render_common.hpp"

namespace nerf {

void launch_render_hash(int bf16, const RenderArgs& a, const GridArgs& g, hipStream_t s) {
    const dim3 grid((unsigned)((a.n_rays + 3) / 4));
    if (bf16)
        hipLaunchKernelGGL(k_render_hash<TBF16S1>, grid, dim3(256), 0, s, a, g);
    else
        hipLaunchKernelGGL(k_render_hash<TF32>, grid, dim3(256), 0, s, a, g);
}

void launch_render_nerf(int kind, int bf16, const RenderArgs& a, hipStream_t s) {
    if (bf16)
        launch_render_nerf_bf16(kind, a, s);
    else
        launch_render_nerf_f32(kind, a, s);
}

}  // namespace nerf

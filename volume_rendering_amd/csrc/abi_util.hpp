// Error reporting shared by the C ABI translation units.
#pragma once

#include "nerf_mi355x.h"

// Records a printf-style message as this thread's last error and returns s.
nerf_status nerf_fail(nerf_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

namespace nerf {

// nerf_render with an optional fixed workspace: fixed_ws (device, fixed_bytes
// long) replaces cfg->workspace and any allocation in the many-network mode,
// and the chunk is chosen to fit it.
nerf_status render_entry(const float* rays_o, const float* rays_d, const float* t_near, const float* t_far,
                         int64_t n_rays, const nerf_weights* w, const nerf_render_cfg* cfg, float* rgb, float* depth,
                         float* acc, void* stream, void* fixed_ws, size_t fixed_bytes);

}  // namespace nerf

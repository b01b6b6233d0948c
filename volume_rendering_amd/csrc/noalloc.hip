// nerf_render_noalloc: the forward render for callers that cannot allocate
// device memory.  The many-network mode's per-chunk workspace (live-sample
// lists, per-cell buckets, raw outputs) comes from a fixed device array of
// this library instead of cfg.workspace or a stream-ordered allocation; the
// rays are rendered in the largest chunks whose workspace fits it.  The other
// modes allocate nothing in any case.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_util.hpp"
#include "nerf_mi355x.h"

namespace {

constexpr size_t kScratchBytes = (size_t)NERF_NOALLOC_SCRATCH_MB << 20;

// One copy per device, held from module load to process end.  Host code
// never uses this name as an address: the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (NULL on failure, with
// the error recorded).
void* scratch_on_current_device() {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        nerf_fail(NERF_ERR_HIP, "nerf_render_noalloc: hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        nerf_fail(NERF_ERR_UNSUPPORTED, "nerf_render_noalloc: device %d beyond %d", dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s != hipSuccess || !p) {
            nerf_fail(NERF_ERR_HIP, "nerf_render_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(s));
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" nerf_status nerf_render_noalloc(const float* rays_o, const float* rays_d, const float* t_near,
                                           const float* t_far, int64_t n_rays, const nerf_weights* w,
                                           const nerf_render_cfg* cfg, float* rgb, float* depth, float* acc,
                                           void* stream) {
    if (cfg && cfg->mode == NERF_MODE_KILO && n_rays > 0) {
        void* p = scratch_on_current_device();
        if (!p) return NERF_ERR_HIP;
        return nerf::render_entry(rays_o, rays_d, t_near, t_far, n_rays, w, cfg, rgb, depth, acc, stream, p,
                                  kScratchBytes);
    }
    // nothing to allocate: the same validation and launches as nerf_render
    return nerf::render_entry(rays_o, rays_d, t_near, t_far, n_rays, w, cfg, rgb, depth, acc, stream, nullptr, 0);
}

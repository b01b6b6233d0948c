"""Helpers shared by the GPU tests: device transfers and workload setup.
Inputs come from ``seeded_inputs``; expected values only from ``oracle``."""
import sys

import numpy as np

import seeded_inputs as si


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def dev(a, dtype=None):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def empty(shape, dtype=None):
    torch = torch_cuda()
    return torch.empty(shape, dtype=dtype or torch.float32, device="cuda")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def page_rays(H, W, focal, pose):
    """Rays of the oracle for a pinhole camera (the GPU path builds its own
    with nerf_gen_rays)."""
    from oracle import rays
    return rays.get_rays(H, W, focal, focal, 0.5 * W, 0.5 * H, pose)


def gpu_rays(H, W, focal, pose):
    import volume_rendering_amd as v
    ro, rd = empty((H * W, 3)), empty((H * W, 3))
    v.nerf_gen_rays(pose, W, H, focal, focal, 0.5 * W, 0.5 * H, ro, rd)
    return ro, rd


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def in_chunks(fn, n, chunk=1024):
    """Runs fn(slice) over [0, n) in chunks and concatenates the outputs
    (arrays, or dicts of arrays) along the first axis."""
    outs = [fn(slice(i, min(n, i + chunk))) for i in range(0, n, chunk)]
    if isinstance(outs[0], dict):
        return {k: np.concatenate([o[k] for o in outs]) for k in outs[0] if np.ndim(outs[0][k]) > 0}
    return np.concatenate(outs)


def bf16_render_check(what, rgb, depth, acc, raw_def, raw_emu, z, rays_d, white=False, rgb_tol=2e-2, acc_tol=2e-2,
                      depth_tol=0.25, tau=1e-3):
    """Checks a render with bfloat16 networks against the float64 definition
    on every ray.

    The last sample's interval is 1e10 |d| long, so its alpha is a step
    function of relu(sigma_raw) at 0.  Where the bfloat16 model (``raw_emu``,
    the oracle's bfloat16 emulation on the same samples) lies on the other side
    of that step than the definition (``raw_def``), or within ``tau`` of it
    (the GPU accumulates the same bfloat16 products in float32 in another
    order), the GPU may absorb there or not: such rays are compared with the
    nearer of the definition's two composites, last sample opaque or
    transparent.  Every other ray is compared with the definition itself.
    rgb and acc are asserted at their bounds; depth (no bound is stated for
    bfloat16) at a loose sanity bound, with max and p99.9 reported."""
    from oracle import composite as ocomp
    s_def, s_emu = raw_def[:, -1, 3], raw_emu[:, -1, 3]
    # (a sample both oracles leave at exactly 0, such as a skipped empty-space
    # sample, is transparent on every side)
    either = ((s_def > 0) != (s_emu > 0)) | ((np.abs(s_emu) < tau) & ((s_def != 0) | (s_emu != 0)))
    rgb_a, dep_a, acc_a, _ = ocomp.volume_render(raw_def, z, rays_d, white)
    raw_b = np.array(raw_def, dtype=np.float64, copy=True)
    raw_b[:, -1, 3] = np.where(s_def > 0, 0.0, 1.0)  # the other side of the step
    rgb_b, dep_b, acc_b, _ = ocomp.volume_render(raw_b, z, rays_d, white)
    e_a = np.max(np.abs(rgb - rgb_a), axis=1)
    e_b = np.max(np.abs(rgb - rgb_b), axis=1)
    pick_b = either & (e_b < e_a)
    rgb_ref = np.where(pick_b[:, None], rgb_b, rgb_a)
    acc_ref = np.where(pick_b, acc_b, acc_a)
    dep_ref = np.where(pick_b, dep_b, dep_a)
    e_rgb = np.max(np.abs(rgb - rgb_ref), axis=1)
    e_acc = np.abs(acc - acc_ref)
    e_dep = np.abs(depth - dep_ref)
    say(f"  {what}: {len(rgb)} rays, {int(either.sum())} on either side of the last-sample step "
        f"({int(pick_b.sum())} took the other side); rgb max {e_rgb.max():.2e} p99.9 {np.quantile(e_rgb, 0.999):.2e}; "
        f"acc max {e_acc.max():.2e} p99.9 {np.quantile(e_acc, 0.999):.2e}; "
        f"depth max {e_dep.max():.2e} p99.9 {np.quantile(e_dep, 0.999):.2e}")
    assert e_rgb.max() <= rgb_tol
    assert e_acc.max() <= acc_tol
    assert e_dep.max() <= depth_tol
    return dict(either=either, e_rgb=e_rgb, e_acc=e_acc, e_dep=e_dep)

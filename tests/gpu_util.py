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

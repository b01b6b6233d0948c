"""Pinhole ray generation (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Follows "Spatial Intelligence - Part 1: NeRF", Section 2 Code,
2. Ray generation (``get_rays``): for pixel column i and row j the
camera-space direction is ((i - cx)/fx, -(j - cy)/fy, -1) with
cx = W/2, cy = H/2, fx = fy = focal and no half-pixel shift; it is rotated
into the world by the upper-left 3x3 of the camera-to-world matrix and is not
normalised; the origin is the matrix's translation column.  Rays are ordered
row-major: ray index = j*W + i.

Defined as float32 operations with no fused multiply-add, so the rays are
bit-reproducible on any IEEE float32 machine:
  dx = (i - cx) / fx,  dy = -((j - cy) / fy),  dz = -1
  d_k = ((R_k0*dx + R_k1*dy) + R_k2*dz)      (left to right, each op rounded)
"""
from __future__ import annotations

import numpy as np

f32 = np.float32


def get_rays(H: int, W: int, fx: float, fy: float, cx: float, cy: float, c2w: np.ndarray):
    """Returns (rays_o, rays_d), float32 [H*W, 3] each."""
    c2w = np.asarray(c2w, dtype=np.float32)
    j, i = np.meshgrid(np.arange(H, dtype=np.float32), np.arange(W, dtype=np.float32), indexing="ij")
    i = i.reshape(-1)
    j = j.reshape(-1)
    dx = (i - f32(cx)) / f32(fx)
    dy = -((j - f32(cy)) / f32(fy))
    dz = np.full_like(dx, f32(-1.0))
    d = np.empty((H * W, 3), dtype=np.float32)
    for k in range(3):
        d[:, k] = (c2w[k, 0] * dx + c2w[k, 1] * dy) + c2w[k, 2] * dz
    o = np.broadcast_to(c2w[:, 3], (H * W, 3)).astype(np.float32).copy()
    return o, d


def page_intrinsics(H: int, W: int, focal: float):
    """The page's intrinsics: a single focal length, principal point at the
    image centre."""
    return dict(H=H, W=W, fx=focal, fy=focal, cx=0.5 * W, cy=0.5 * H)

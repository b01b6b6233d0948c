"""Alpha compositing by transmittance (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Spatial Intelligence - Part 1: NeRF", Section 1 Theory, 3. Volume rendering
(discrete quadrature) and Section 2 Code, 5. Volume rendering in code
(``volume_render``):
  delta_i = (z_{i+1} - z_i) |d|, with delta_{N-1} = 1e10 |d|
  c_i = sigmoid(rgb_raw_i),  sigma_i = max(sigma_raw_i, 0)
  alpha_i = 1 - exp(-sigma_i delta_i)
  T_0 = 1,  T_{i+1} = T_i (1 - alpha_i + 1e-10)   (exclusive product)
  w_i = T_i alpha_i
  rgb = sum w_i c_i,  depth = sum w_i z_i,  acc = sum w_i
  white background: rgb += 1 - acc
Depth is in ray-parameter units and is not divided by acc.  Float64.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def volume_render(raw, z, rays_d, white_bkgd: bool = False, term_T: float = 0.0):
    """``raw`` [R, N, 4] (rgb_raw, sigma_raw), ``z`` [R, N], ``rays_d`` [R, 3].
    ``term_T`` > 0 applies early termination: sample i and every later sample
    are dropped once T_i < term_T.  Returns (rgb [R,3], depth [R], acc [R],
    weights [R,N]) in float64."""
    raw = np.asarray(raw, dtype=np.float64)
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    dnorm = np.linalg.norm(np.asarray(rays_d, dtype=np.float64), axis=-1, keepdims=True)
    dists = np.concatenate([z[:, 1:] - z[:, :-1], np.full_like(z[:, :1], 1e10)], axis=1) * dnorm
    rgb = sigmoid(raw[..., :3])
    sigma = np.maximum(raw[..., 3], 0.0)
    alpha = 1.0 - np.exp(-sigma * dists)
    surv = np.concatenate([np.ones_like(alpha[:, :1]), 1.0 - alpha + 1e-10], axis=1)
    T = np.cumprod(surv, axis=1)[:, :-1]
    if term_T > 0.0:
        stopped = np.cumsum(T < term_T, axis=1) > 0
        alpha = np.where(stopped, 0.0, alpha)
    w = T * alpha
    rgb_map = np.sum(w[..., None] * rgb, axis=1)
    acc = np.sum(w, axis=1)
    depth = np.sum(w * z, axis=1)
    if white_bkgd:
        rgb_map = rgb_map + (1.0 - acc[:, None])
    return rgb_map, depth, acc, w

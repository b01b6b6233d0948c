"""Samples along rays: stratified samples, sample points, view directions,
inverse-CDF resampling and the merge of coarse and fine samples (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources: "Spatial Intelligence - Part 1: NeRF", Section 1 Theory,
3. Volume rendering (r(t) = o + t d; samples t_1 < ... < t_N) and
4.2 Hierarchical volume sampling; Section 2 Code, 6. Hierarchical sampling
(``sample_pdf``, ``render_rays``).
"""
from __future__ import annotations

import numpy as np

from .philox import STREAM_JITTER, STREAM_PDF, uniforms

f32 = np.float32


def ray_counters(R: int, ray_offset) -> np.ndarray:
    """Global ray index of each of R rays, the Philox counter of its random
    numbers: ray_offset + r for an integer offset, or the given per-ray
    indices for an integer array of length R (rays sampled from a larger
    batch keep their place in it).  Returns uint64 [R, 1]."""
    if np.ndim(ray_offset) == 0:
        return (np.arange(R, dtype=np.uint64) + np.uint64(int(ray_offset)))[:, None]
    ids = np.asarray(ray_offset, dtype=np.int64)
    assert ids.shape == (R,) and (R == 0 or ids.min() >= 0)
    return ids.astype(np.uint64)[:, None]


def stratified(t_near, t_far, n: int, seed: int, jitter: bool = True, ray_offset=0):
    """Stratified samples.  The page calls ``stratified_sample`` without
    defining it; the reading here is n equal strata on [near, far] with one
    uniform draw in each (u = 1/2 without jitter).  As float32 operations:
      step = (far - near) / n;  z_i = near + step * (i + u_i).
    Returns float32 [R, n]."""
    t_near = np.asarray(t_near, dtype=np.float32)
    t_far = np.asarray(t_far, dtype=np.float32)
    R = t_near.shape[0]
    step = (t_far - t_near) / f32(n)
    i = np.arange(n, dtype=np.float32)[None, :]
    if jitter:
        u = uniforms(seed, STREAM_JITTER, ray_counters(R, ray_offset), np.arange(n, dtype=np.uint64)[None, :])
    else:
        u = np.full((R, n), f32(0.5), dtype=np.float32)
    s = i + u
    return t_near[:, None] + step[:, None] * s


def points(rays_o, rays_d, z):
    """Sample points x = o + z d as float32 operations (no fused multiply-add).
    Returns float32 [R, N, 3]."""
    o = np.asarray(rays_o, dtype=np.float32)[:, None, :]
    d = np.asarray(rays_d, dtype=np.float32)[:, None, :]
    return o + np.asarray(z, dtype=np.float32)[:, :, None] * d


def view_dirs(rays_d):
    """Unit viewing direction d/|d| in float64 (the page's ``dirs``; the
    theory gives the direction as a point on the sphere)."""
    d = np.asarray(rays_d, dtype=np.float64)
    return d / np.linalg.norm(d, axis=-1, keepdims=True)


def midpoints(z):
    """Bin edges between consecutive coarse samples, float32:
    b_k = 0.5 * (z_k + z_{k+1})."""
    z = np.asarray(z, dtype=np.float32)
    return f32(0.5) * (z[:, 1:] + z[:, :-1])


def sample_pdf(bins, weights, n_fine: int, seed: int, ray_offset=0):
    """Inverse-CDF resampling ("6. Hierarchical sampling", ``sample_pdf``).

    ``bins`` float32 [R, B+1] are bin edges, ``weights`` float32 [R, B] the
    weight of each bin.  Steps in the page's order:
      1. w' = w + 1e-5 (float32), so no bin has zero probability;
      2. pdf = w' / sum(w'); cdf = running sum with a leading 0 (B+1 entries);
         here the running sum is taken in float64, where it is exact in
         any order: every float32 w' >= 1e-5 > 2^-17 is a multiple of
         2^-40, so partial sums below 2^13 (e.g. weights at most 1 with up
         to 255 bins) need at most 53 bits.  Each cdf entry is then one
         correctly rounded division, so cdf_0 = 0 and cdf_B = 1 exactly;
      3. u uniform in [0,1) (Philox stream 1, one per (ray, fine index));
      4. idx = number of cdf entries <= u (right-sided search);
         below = max(idx-1, 0), above = min(idx, B);
      5. denom = max(cdf[above] - cdf[below], 1e-5);
         t = (u - cdf[below]) / denom;
         z = bins[below] + t * (bins[above] - bins[below]),
         in float64 without fused multiply-add, rounded once to float32.
    Returns (z_fine float32 [R, n_fine], idx int32 [R, n_fine])."""
    bins = np.asarray(bins, dtype=np.float32)
    w = np.asarray(weights, dtype=np.float32) + f32(1e-5)
    R, B = w.shape
    S = np.concatenate([np.zeros((R, 1)), np.cumsum(w.astype(np.float64), axis=1)], axis=1)
    cdf = S / S[:, -1:]
    u = uniforms(seed, STREAM_PDF, ray_counters(R, ray_offset), np.arange(n_fine, dtype=np.uint64)[None, :]
                 ).astype(np.float64)
    idx = np.empty((R, n_fine), dtype=np.int64)
    for r in range(R):
        idx[r] = np.searchsorted(cdf[r], u[r], side="right")
    below = np.maximum(idx - 1, 0)
    above = np.minimum(idx, B)
    cdf_b = np.take_along_axis(cdf, below, 1)
    cdf_a = np.take_along_axis(cdf, above, 1)
    bins64 = bins.astype(np.float64)
    bin_b = np.take_along_axis(bins64, below, 1)
    bin_a = np.take_along_axis(bins64, above, 1)
    denom = np.maximum(cdf_a - cdf_b, 1e-5)
    t = (u - cdf_b) / denom
    z = (bin_b + t * (bin_a - bin_b)).astype(np.float32)
    return z, idx.astype(np.int32)


def hierarchical_fine_samples(z_coarse, w_coarse, n_fine: int, seed: int, ray_offset=0):
    """The page's resampling step of ``render_rays``: bins are the midpoints
    of the coarse samples, weighted by the coarse weights without the two end
    samples; the fine network sees the ascending sort of coarse and fine
    samples together.  Returns (z_fine, idx, z_merged)."""
    z_coarse = np.asarray(z_coarse, dtype=np.float32)
    w = np.asarray(w_coarse, dtype=np.float32)
    z_f, idx = sample_pdf(midpoints(z_coarse), w[:, 1:-1], n_fine, seed, ray_offset)
    z2 = np.sort(np.concatenate([z_coarse, z_f], axis=1), axis=1)
    return z_f, idx, z2

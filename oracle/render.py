"""End-to-end forward renders (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

``render_nerf`` is the page's ``render_rays`` ("Spatial Intelligence - Part
1: NeRF", Section 2 Code, 6. Hierarchical sampling): stratified coarse
samples, coarse network, compositing, inverse-CDF resampling over the
midpoints of the coarse samples with the coarse weights minus the two end
samples, ascending merge of coarse and fine samples, fine network,
compositing.  ``render_hash`` swaps the encoding for the multiresolution hash
grid and the hash-field network.  ``render_kilo`` evaluates many tiny
networks, one per cell of a regular grid, skips samples outside the scene
box or in empty voxels, and stops a ray once its transmittance falls below a
threshold ("KiloNeRF: Speeding up Neural Radiance Fields with Thousands of
Tiny MLPs", abstract: thousands of tiny MLPs plus further optimisations).
"""
from __future__ import annotations

import numpy as np

from . import composite, encoding, mlp, sampling

f32 = np.float32


def _encode_points(x, L_pos, use_pi):
    R, N, _ = x.shape
    return encoding.freq_encode(x.reshape(-1, 3), L_pos, True, use_pi)


def occupied(x, occ, occ_res=128, box=(-1.5, 1.5)):
    """Empty-space test of sample points (the same voxel arithmetic as the
    many-network render): inside the closed box and in an occupied voxel.
    ``occ`` None: every sample is live.  Returns bool [...]."""
    if occ is None:
        return np.ones(np.asarray(x).shape[:-1], dtype=bool)
    live, _, _ = kilo_classify(x, occ, occ_res, 1, box)
    return live


def nerf_pass(params, rays_o, rays_d, z, L_pos=10, L_dir=4, mode="f64", use_pi=True, white_bkgd=False, occ=None,
              occ_res=128, box=(-1.5, 1.5), term_T=0.0):
    """One network pass over given samples ``z`` [R, N] (float32): points,
    encodings, network, compositing.  With an occupancy grid ``occ``, samples
    outside the box or in empty voxels have density 0 (empty-space skipping:
    "Spatial Intelligence - Part 1: NeRF", Section 1 Theory, 4.2, uniform
    samples waste compute on empty space); ``term_T`` > 0 drops sample i and
    later once T_i < term_T.  Returns dict(raw, rgb, depth, acc, w, n_live)."""
    z = np.asarray(z, dtype=np.float32)
    R, N = z.shape
    x = sampling.points(rays_o, rays_d, z)
    live = occupied(x, occ, occ_res, box)
    pe = _encode_points(x, L_pos, use_pi)
    de = encoding.freq_encode(sampling.view_dirs(rays_d), L_dir, True, use_pi)
    de = np.repeat(de, N, axis=0)
    raw = mlp.nerf_forward(params, pe, de, mode).reshape(R, N, 4)
    raw[~live] = 0.0
    rgb, depth, acc, w = composite.volume_render(raw, z, rays_d, white_bkgd, term_T)
    return dict(raw=raw, rgb=rgb, depth=depth, acc=acc, w=w, n_live=int(live.sum()))


def render_nerf(rays_o, rays_d, t_near, t_far, coarse, fine=None, n_coarse=64, n_fine=128, L_pos=10, L_dir=4,
                seed=0, jitter=True, mode="f64", use_pi=True, white_bkgd=False, ray_offset=0, occ=None, occ_res=128,
                box=(-1.5, 1.5), term_T=0.0):
    """Coarse pass, then (if ``fine`` is given and n_fine > 0) resampling and
    the fine pass; both passes skip empty space and stop early as
    ``nerf_pass`` describes.  The coarse weights enter the sampler as float32,
    the precision of the page's tensors."""
    z_c = sampling.stratified(t_near, t_far, n_coarse, seed, jitter, ray_offset)
    c = nerf_pass(coarse, rays_o, rays_d, z_c, L_pos, L_dir, mode, use_pi, white_bkgd, occ, occ_res, box, term_T)
    out = dict(z_c=z_c, coarse=c, rgb=c["rgb"], depth=c["depth"], acc=c["acc"], n_live=c["n_live"])
    if fine is not None and n_fine > 0:
        w32 = c["w"].astype(np.float32)
        z_f, idx, z2 = sampling.hierarchical_fine_samples(z_c, w32, n_fine, seed, ray_offset)
        f = nerf_pass(fine, rays_o, rays_d, z2, L_pos, L_dir, mode, use_pi, white_bkgd, occ, occ_res, box, term_T)
        out.update(z_f=z_f, bin_idx=idx, z2=z2, fine=f, rgb=f["rgb"], depth=f["depth"], acc=f["acc"],
                   n_live=c["n_live"] + f["n_live"])
    return out


def render_hash(rays_o, rays_d, t_near, t_far, grid, tables, field, n_samples=128, seed=0, jitter=True,
                mode="f64", box=(-1.5, 1.5), white_bkgd=False, ray_offset=0, level_mask=None, occ=None, occ_res=128,
                term_T=0.0):
    """Hash-grid field render: stratified samples, world box mapped to the
    unit cube, grid features (times the optional per-level mask), spherical
    harmonics direction encoding, field network, compositing; empty space and
    early termination as ``nerf_pass``."""
    z = sampling.stratified(t_near, t_far, n_samples, seed, jitter, ray_offset)
    R, N = z.shape
    x3 = sampling.points(rays_o, rays_d, z)
    live = occupied(x3, occ, occ_res, box)
    x = x3.reshape(-1, 3)
    feats = grid.encode(encoding.world_to_unit(x, *box), tables, level_mask)
    de = np.repeat(encoding.sh16(sampling.view_dirs(rays_d)), N, axis=0)
    raw = mlp.hash_field_forward(field, feats, de, mode).reshape(R, N, 4)
    raw[~live] = 0.0
    rgb, depth, acc, w = composite.volume_render(raw, z, rays_d, white_bkgd, term_T)
    return dict(z=z, raw=raw, rgb=rgb, depth=depth, acc=acc, w=w, n_live=int(live.sum()))


def kilo_classify(x, occ_dense, occ_res=128, cells=16, box=(-1.5, 1.5)):
    """Per sample point: inside the (closed) box, occupied voxel, cell id.
    Voxel and cell coordinates are clamp(floor((x - lo) * (res/size)), 0,
    res-1) as float32 operations; ids are x-major.  Returns (live bool,
    cell int64, voxel int64)."""
    lo, hi = box
    x = np.asarray(x, dtype=np.float32)
    inside = np.all((x >= f32(lo)) & (x <= f32(hi)), axis=-1)
    t = x - f32(lo)
    vs = f32(occ_res / (hi - lo))
    cs = f32(cells / (hi - lo))
    v = np.clip(np.floor(t * vs), 0, occ_res - 1).astype(np.int64)
    c = np.clip(np.floor(t * cs), 0, cells - 1).astype(np.int64)
    vox = (v[..., 0] * occ_res + v[..., 1]) * occ_res + v[..., 2]
    cell = (c[..., 0] * cells + c[..., 1]) * cells + c[..., 2]
    live = inside & occ_dense[vox]
    return live, cell, vox


def render_kilo(rays_o, rays_d, t_near, t_far, occ_dense, cell_nets, n_samples=192, seed=0, jitter=True,
                term_T=1e-2, L_pos=10, L_dir=4, mode="f64", use_pi=True, occ_res=128, cells=16,
                box=(-1.5, 1.5), ray_offset=0, white_bkgd=False):
    """Many tiny networks.  ``cell_nets(c)`` returns the parameters of cell
    c.  Dead samples (outside the box or in an empty voxel) have density 0;
    compositing stops a ray at the first sample whose transmittance is below
    ``term_T``.  Returns dict(rgb, depth, acc, live, cell, n_live)."""
    z = sampling.stratified(t_near, t_far, n_samples, seed, jitter, ray_offset)
    R, N = z.shape
    x = sampling.points(rays_o, rays_d, z)
    live, cell, _ = kilo_classify(x, occ_dense, occ_res, cells, box)
    raw = np.zeros((R, N, 4))
    vdir = encoding.freq_encode(sampling.view_dirs(rays_d), L_dir, True, use_pi)
    rr, ss = np.nonzero(live)
    cl = cell[rr, ss]
    for c in np.unique(cl):
        sel = cl == c
        r_sel, s_sel = rr[sel], ss[sel]
        pe = encoding.freq_encode(x[r_sel, s_sel], L_pos, True, use_pi)
        raw[r_sel, s_sel] = mlp.nerf_forward(cell_nets(int(c)), pe, vdir[r_sel], mode)
    rgb, depth, acc, w = composite.volume_render(raw, z, rays_d, white_bkgd, term_T)
    return dict(z=z, raw=raw, rgb=rgb, depth=depth, acc=acc, w=w, live=live, cell=cell, n_live=int(live.sum()))

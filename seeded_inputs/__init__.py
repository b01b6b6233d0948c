"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds only input generation: camera poses, network weights,
hash tables, occupancy grids, query points and parity subsets.  It contains
none of the rendering arithmetic (no ray generation, sampling, encoding,
network evaluation or compositing), so the oracle and the GPU path can both
draw their inputs from it without sharing any of the method.

Every generator takes an integer seed and a purpose tag; the stream is
numpy's PCG64 seeded with ``[seed, tag]`` so that independent fixtures never
share random numbers.  Fixtures are produced as float32 (float16 for hash
tables), the precision the renderer consumes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Purpose tags: one independent random stream per kind of fixture.
TAG_POSES = 2
TAG_MLP = 3
TAG_HASH = 4
TAG_OCC = 5
TAG_SUBSET = 6
TAG_QUERY = 7
TAG_TARGET = 8


def rng(seed: int, tag: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), *[int(e) for e in extra]])


# ----------------------------------------------------------------------------
# Camera poses
# ----------------------------------------------------------------------------

def look_at_pose(position: np.ndarray) -> np.ndarray:
    """Camera-to-world 3x4 matrix for a camera at ``position`` looking at the
    origin, with world up = +z.  The camera looks down its own -z axis with +y
    up, the convention the ray generator assumes (its camera-space direction
    has z = -1).  Built in float64, rounded to float32 once."""
    p = np.asarray(position, dtype=np.float64)
    back = p / np.linalg.norm(p)
    right = np.cross(np.array([0.0, 0.0, 1.0]), back)
    if np.linalg.norm(right) < 1e-6:
        right = np.cross(np.array([0.0, 1.0, 0.0]), back)
    right /= np.linalg.norm(right)
    up = np.cross(back, right)
    c2w = np.stack([right, up, back, p], axis=1)  # columns: R | t
    return c2w.astype(np.float32)


def poses(n: int, seed: int = 0, radius: float = 4.0, hemisphere: bool = True) -> np.ndarray:
    """``n`` camera poses on a sphere (or upper hemisphere) of ``radius``
    around the origin, each looking at the origin.  Returns float32 [n,3,4]."""
    g = rng(seed, TAG_POSES)
    out = []
    for _ in range(n):
        u0, u1 = g.random(), g.random()
        az = 2.0 * math.pi * u0
        el = math.asin(u1) if hemisphere else math.asin(2.0 * u1 - 1.0)
        p = radius * np.array([math.cos(el) * math.cos(az), math.cos(el) * math.sin(az), math.sin(el)])
        out.append(look_at_pose(p))
    return np.stack(out).astype(np.float32)


def sweep_poses(n: int, elevation_deg: float = 30.0, radius: float = 4.0) -> np.ndarray:
    """``n`` poses evenly spaced in azimuth around the scene (a 360 degree
    sweep at a fixed elevation and radius), each looking at the origin.
    Deterministic; returns float32 [n,3,4]."""
    el = math.radians(elevation_deg)
    out = []
    for k in range(n):
        az = 2.0 * math.pi * k / n
        p = radius * np.array([math.cos(el) * math.cos(az), math.cos(el) * math.sin(az), math.sin(el)])
        out.append(look_at_pose(p))
    return np.stack(out).astype(np.float32)


# ----------------------------------------------------------------------------
# Network weights (float32, row-major [out, in])
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class NerfNetShape:
    """Shape of a NeRF-family radiance network: ``depth`` ReLU layers of
    ``width`` on the position encoding (``pos_ch`` wide), optional skip
    concatenation of the position encoding after layer ``skip``, a density
    head, a linear feature layer, a direction layer of ``dir_width`` on
    [feature, direction encoding (``dir_ch`` wide)] and an rgb head."""
    depth: int
    width: int
    skip: int  # -1: no skip
    pos_ch: int
    dir_ch: int
    dir_width: int

    def layer_dims(self):
        dims = []
        for i in range(self.depth):
            if i == 0:
                fin = self.pos_ch
            elif self.skip >= 0 and i == self.skip + 1:
                fin = self.width + self.pos_ch
            else:
                fin = self.width
            dims.append((self.width, fin))
        return dims

    def n_params(self) -> int:
        n = sum(o * i + o for o, i in self.layer_dims())
        n += self.width + 1                       # density head
        n += self.width * self.width + self.width  # feature layer
        n += self.dir_width * (self.width + self.dir_ch) + self.dir_width
        n += 3 * self.dir_width + 3                # rgb head
        return n


NERF_8x256 = NerfNetShape(depth=8, width=256, skip=4, pos_ch=63, dir_ch=27, dir_width=128)
NERF_4x64 = NerfNetShape(depth=4, width=64, skip=-1, pos_ch=39, dir_ch=27, dir_width=32)
NERF_CELL_2x32 = NerfNetShape(depth=2, width=32, skip=-1, pos_ch=63, dir_ch=27, dir_width=16)


@dataclass(frozen=True)
class HashFieldShape:
    """Hash-grid radiance field: density net feat_ch -> width -> width (ReLU),
    density head, linear feature layer (width), colour net
    [feature, direction encoding (dir_ch)] -> width -> width (ReLU) -> rgb."""
    feat_ch: int = 32
    width: int = 64
    dir_ch: int = 16

    def n_params(self) -> int:
        w, f, d = self.width, self.feat_ch, self.dir_ch
        return (w * f + w) + (w * w + w) + (w + 1) + (w * w + w) + (w * (w + d) + w) + (w * w + w) + (3 * w + 3)


HASH_FIELD = HashFieldShape()


def _uniform(g: np.random.Generator, shape, bound: float) -> np.ndarray:
    return ((g.random(shape) * 2.0 - 1.0) * bound).astype(np.float32)


def _he_uniform_linear(g, fan_out: int, fan_in: int):
    """He-uniform weights U(+-sqrt(6/fan_in)); bias U(+-1/sqrt(fan_in))."""
    W = _uniform(g, (fan_out, fan_in), math.sqrt(6.0 / fan_in))
    b = _uniform(g, (fan_out,), 1.0 / math.sqrt(fan_in))
    return W, b


def nerf_params(shape: NerfNetShape, seed: int = 0, net_id: int = 0) -> dict:
    """Seeded He-uniform weights for a NeRF-family network.  Keys:
    ``layers`` (list of (W, b)), ``sigma`` (w [1,W], b [1]), ``feature``,
    ``dir``, ``rgb``."""
    g = rng(seed, TAG_MLP, net_id)
    layers = [_he_uniform_linear(g, o, i) for o, i in shape.layer_dims()]
    sigma = _he_uniform_linear(g, 1, shape.width)
    feature = _he_uniform_linear(g, shape.width, shape.width)
    dirl = _he_uniform_linear(g, shape.dir_width, shape.width + shape.dir_ch)
    rgb = _he_uniform_linear(g, 3, shape.dir_width)
    return {"shape": shape, "layers": layers, "sigma": sigma, "feature": feature, "dir": dirl, "rgb": rgb}


def hash_field_params(shape: HashFieldShape = HASH_FIELD, seed: int = 0) -> dict:
    g = rng(seed, TAG_MLP, 1000)
    w = shape.width
    return {
        "shape": shape,
        "density": [_he_uniform_linear(g, w, shape.feat_ch), _he_uniform_linear(g, w, w)],
        "sigma": _he_uniform_linear(g, 1, w),
        "feature": _he_uniform_linear(g, w, w),
        "color": [_he_uniform_linear(g, w, w + shape.dir_ch), _he_uniform_linear(g, w, w)],
        "rgb": _he_uniform_linear(g, 3, w),
    }


def cell_params(n_cells: int, shape: NerfNetShape = NERF_CELL_2x32, seed: int = 0) -> list:
    """One seeded network per cell (net_id = 2000 + cell)."""
    return [nerf_params(shape, seed, 2000 + c) for c in range(n_cells)]


def cell_params_stacked(n_cells: int, shape: NerfNetShape = NERF_CELL_2x32, seed: int = 0) -> dict:
    """All cell networks drawn in one go and stacked along a leading cell
    axis (same He-uniform bounds as :func:`nerf_params`).  Used for the 4096
    cell workload where per-cell generators would be slow."""
    g = rng(seed, TAG_MLP, 4000)

    def lin(fo, fi):
        W = ((g.random((n_cells, fo, fi)) * 2.0 - 1.0) * math.sqrt(6.0 / fi)).astype(np.float32)
        b = ((g.random((n_cells, fo)) * 2.0 - 1.0) / math.sqrt(fi)).astype(np.float32)
        return W, b

    return {
        "shape": shape,
        "layers": [lin(o, i) for o, i in shape.layer_dims()],
        "sigma": lin(1, shape.width),
        "feature": lin(shape.width, shape.width),
        "dir": lin(shape.dir_width, shape.width + shape.dir_ch),
        "rgb": lin(3, shape.dir_width),
    }


def cell_slice(stacked: dict, c: int) -> dict:
    """Parameters of cell ``c`` from :func:`cell_params_stacked`, in the
    layout :func:`nerf_params` returns."""
    return {
        "shape": stacked["shape"],
        "layers": [(W[c], b[c]) for W, b in stacked["layers"]],
        **{k: (stacked[k][0][c], stacked[k][1][c]) for k in ("sigma", "feature", "dir", "rgb")},
    }


# ----------------------------------------------------------------------------
# Hash tables, occupancy, query points
# ----------------------------------------------------------------------------

def hash_tables(sizes, n_feat: int = 2, seed: int = 0, scale: float = 1e-4) -> list:
    """One float16 table [size, n_feat] per level, U(-scale, +scale)."""
    g = rng(seed, TAG_HASH, int(scale * 1e6))
    return [((g.random((int(s), n_feat)) * 2.0 - 1.0) * scale).astype(np.float16) for s in sizes]


def occupancy_bits(res: int = 128, p: float = 0.1, seed: int = 0) -> np.ndarray:
    """Bernoulli(p) occupancy over a res^3 grid, x-major voxel order, packed
    little-endian into uint32 words (bit v%32 of word v/32)."""
    g = rng(seed, TAG_OCC)
    occ = g.random(res ** 3) < p
    return np.packbits(occ.astype(np.uint8), bitorder="little").view(np.uint32).copy()


def occupancy_words(res: int, seed: int = 0) -> np.ndarray:
    """Occupancy of a large res^3 grid as uniformly random uint32 words
    (each voxel occupied with probability 1/2), for grids too large to draw
    one float per voxel.  Same bit order as :func:`occupancy_bits`."""
    n_words = (res ** 3 + 31) // 32
    return rng(seed, TAG_OCC, res).integers(0, 2 ** 32, size=n_words, dtype=np.uint32)


class PackedOccupancy:
    """Read-only view of a packed occupancy bitset that indexes like a dense
    boolean array (``occ[vox]`` for an integer array ``vox``)."""

    def __init__(self, words: np.ndarray):
        self.words = words

    def __getitem__(self, vox):
        vox = np.asarray(vox, dtype=np.int64)
        return ((self.words[vox >> 5] >> (vox & 31).astype(np.uint32)) & 1).astype(bool)


def occupancy_dense(bits: np.ndarray, res: int = 128) -> np.ndarray:
    return np.unpackbits(bits.view(np.uint8), bitorder="little")[: res ** 3].astype(bool)


def query_points(n: int, seed: int = 0) -> np.ndarray:
    """``n`` points uniform in [0,1)^3, float32 [n,3]."""
    return rng(seed, TAG_QUERY).random((n, 3)).astype(np.float32)


def subset(n_total: int, k: int, seed: int = 0) -> np.ndarray:
    """Sorted random subset of ``k`` distinct indices below ``n_total``."""
    if k >= n_total:
        return np.arange(n_total, dtype=np.int64)
    return np.sort(rng(seed, TAG_SUBSET).choice(n_total, size=k, replace=False)).astype(np.int64)


def target_colors(n: int, seed: int = 0) -> np.ndarray:
    """``n`` colours uniform in [0,1)^3, float32 [n,3] (training targets)."""
    return rng(seed, TAG_TARGET).random((n, 3)).astype(np.float32)


def flat_params(params: dict) -> np.ndarray:
    """The weights and biases of a NeRF-family parameter dict back to back,
    float32, in the C ABI's order: each hidden layer (W row-major, then b),
    then the density head, the feature layer, the direction layer and the rgb
    head."""
    seq = list(params["layers"]) + [params[k] for k in ("sigma", "feature", "dir", "rgb")]
    return np.concatenate([np.asarray(a, np.float32).ravel() for Wb in seq for a in Wb])


TAG_INR = 9


def hash_inr_params(sizes, n_levels: int, hidden: int = 32, n_out: int = 1, seed: int = 0):
    """Parameters of a hash-grid INR: one float32 table [size, 2] per level,
    U(-1e-4, 1e-4), and a decoder Linear(2L -> hidden), ReLU, Linear(hidden
    -> n_out) with weights and biases U(+-1/sqrt(fan_in)).  Returns (tables,
    (W1, b1, W2, b2))."""
    g = rng(seed, TAG_INR)
    tables = [_uniform(g, (int(s), 2), 1e-4) for s in sizes]
    f = 2 * n_levels
    W1 = _uniform(g, (hidden, f), 1.0 / math.sqrt(f))
    b1 = _uniform(g, (hidden,), 1.0 / math.sqrt(f))
    W2 = _uniform(g, (n_out, hidden), 1.0 / math.sqrt(hidden))
    b2 = _uniform(g, (n_out,), 1.0 / math.sqrt(hidden))
    return tables, (W1, b1, W2, b2)


def hash_inr_flat(tables, mlp) -> np.ndarray:
    """The C ABI's flat order: tables level by level, then W1, b1, W2, b2."""
    return np.concatenate([np.asarray(t, np.float32).ravel() for t in tables] +
                          [np.asarray(a, np.float32).ravel() for a in mlp])


def inr_target_image(res: int = 96):
    """A grey-level test image on a res x res grid of [0,1]^2 with structure at
    several scales: a smooth product of low-frequency sines, thin vertical
    stripes and a sharp-edged disk, rescaled to [0,1].  Returns (coords
    float32 [res*res, 2] as (x, y), values float32 [res*res, 1])."""
    t = np.linspace(0.0, 1.0, res)
    X, Y = np.meshgrid(t, t)
    img = 0.5 + 0.35 * np.sin(6 * np.pi * X) * np.sin(6 * np.pi * Y)
    img = img + 0.25 * (np.sin(22 * np.pi * X) > 0)
    img = img + 0.4 * (np.hypot(X - 0.5, Y - 0.5) < 0.18)
    img = (img - img.min()) / (img.max() - img.min())
    coords = np.stack([X.ravel(), Y.ravel()], axis=1).astype(np.float32)
    return coords, img.ravel()[:, None].astype(np.float32)

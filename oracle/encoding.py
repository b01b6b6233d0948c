"""Input encodings (oracle): frequency (positional) encoding, the
multiresolution hash grid in 3D (and the 2D grid it generalises), and the
16-term spherical-harmonics direction encoding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).
"""
from __future__ import annotations

import math

import numpy as np

f32 = np.float32

# ----------------------------------------------------------------------------
# Frequency encoding
# ----------------------------------------------------------------------------


def freq_encode(x, L: int, include_input: bool = True, use_pi: bool = True) -> np.ndarray:
    """gamma(p) = (p, sin(2^0 pi p), cos(2^0 pi p), ..., sin(2^{L-1} pi p),
    cos(2^{L-1} pi p)) applied to each coordinate of p
    ("Spatial Intelligence - Part 1: NeRF", Section 1 Theory, 4.1 Positional
    encoding): width d + 2 d L for a d-vector (63 for L=10, 27 for L=4).

    Layout follows the theory formula, frequency-major: the input, then for
    each k the d sines followed by the d cosines.  ``use_pi=False`` drops the
    factor pi, as the page's code snippet (Section 2 Code, 3. Positional
    encoding) does.  The argument a = 2^k p is exact for float32 p; sin(pi a)
    is evaluated in float64.  Returns float64 [..., d + 2 d L]."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    parts = [x] if include_input else []
    for k in range(L):
        a = x * (2.0 ** k)
        arg = math.pi * a if use_pi else a
        parts.append(np.sin(arg))
        parts.append(np.cos(arg))
    return np.concatenate(parts, axis=-1)


# ----------------------------------------------------------------------------
# Multiresolution hash grid
# ----------------------------------------------------------------------------

PRIMES_3D = (1, 2654435761, 805459861)


def grid_resolutions(n_levels: int, n_min: int, n_max: int):
    """N_l = round(N_min * b^l), b = exp((ln N_max - ln N_min)/(L-1))
    ("Instant-NGP - Visual Experiments", shared toolkit, ``HashGrid2D``)."""
    b = math.exp((math.log(n_max) - math.log(n_min)) / (n_levels - 1))
    return [int(round(n_min * b ** l)) for l in range(n_levels)]


def level_layout(res, table_size: int, dim: int):
    """Per level: (direct?, table entries).  A level indexes directly when its
    (N+1)^dim vertices fit the table; its table then holds exactly that many
    entries, otherwise ``table_size`` (same toolkit)."""
    out = []
    for N in res:
        verts = (N + 1) ** dim
        out.append((verts <= table_size, min(table_size, verts)))
    return out


def hash_index(coords, table_size: int, primes=PRIMES_3D) -> np.ndarray:
    """Spatial hash: xor over axes of coordinate * prime, modulo the table
    size (the toolkit's ``_idx``, extended to 3D with the primes 1,
    2654435761, 805459861).  Computed in exact integer arithmetic."""
    coords = [np.asarray(c, dtype=np.int64) for c in coords]
    h = None
    for c, p in zip(coords, primes):
        # exact in int64 while coordinate * prime < 2^63
        assert c.size == 0 or (int(c.max()) < 2 ** 31 and int(c.min()) >= 0)
        term = c * np.int64(p)
        h = term if h is None else (h ^ term)
    return h % np.int64(table_size)


def direct_index(coords, N: int) -> np.ndarray:
    """Direct index of a vertex, x-major: ((ix*(N+1)) + iy)*(N+1) + iz
    (the toolkit's 2D form ix*(N+1) + iy, extended to 3D)."""
    idx = np.zeros_like(np.asarray(coords[0], dtype=np.int64))
    for c in coords:
        idx = idx * (N + 1) + np.asarray(c, dtype=np.int64)
    return idx


class HashGrid:
    """Multiresolution grid over [0,1]^dim with one feature table per level."""

    def __init__(self, dim: int, n_levels: int, table_size: int, n_min: int, n_max: int):
        self.dim = dim
        self.L = n_levels
        self.T = table_size
        self.res = grid_resolutions(n_levels, n_min, n_max)
        lay = level_layout(self.res, table_size, dim)
        self.direct = [d for d, _ in lay]
        self.sizes = [s for _, s in lay]

    def level_indices(self, x, l: int):
        """Integer part of the lookup for level l: for each point and each of
        the 2^dim corners (corner bits in lexicographic order, first axis
        most significant) the table index, plus the interpolation fractions.
        c = x * N_l and w = c - floor(c) are float32 operations so that the
        cell and the index are bit-exact; corners are clamped to [0, N_l].
        Returns (idx int64 [P, 2^dim], frac float32 [P, dim])."""
        N = self.res[l]
        x = np.asarray(x, dtype=np.float32)
        c = x * f32(N)
        c0 = np.floor(c)
        w = c - c0
        c0 = c0.astype(np.int64)
        P = x.shape[0]
        idx = np.empty((P, 2 ** self.dim), dtype=np.int64)
        for corner in range(2 ** self.dim):
            bits = [(corner >> (self.dim - 1 - a)) & 1 for a in range(self.dim)]
            cc = [np.clip(c0[:, a] + bits[a], 0, N) for a in range(self.dim)]
            idx[:, corner] = direct_index(cc, N) if self.direct[l] else hash_index(cc, self.T)
        return idx, w

    def encode(self, x, tables, level_mask=None) -> np.ndarray:
        """Interpolated features, levels concatenated (level-major, then
        feature): multilinear weights prod over axes of (w or 1-w), summed
        over the 2^dim corners.  Float64 [P, L*F]."""
        feats = []
        for l in range(self.L):
            idx, w = self.level_indices(x, l)
            w = w.astype(np.float64)
            tab = np.asarray(tables[l]).astype(np.float64)
            acc = np.zeros((idx.shape[0], tab.shape[1]))
            for corner in range(2 ** self.dim):
                bits = [(corner >> (self.dim - 1 - a)) & 1 for a in range(self.dim)]
                wt = np.ones(idx.shape[0])
                for a in range(self.dim):
                    wt = wt * (w[:, a] if bits[a] else (1.0 - w[:, a]))
                acc += wt[:, None] * tab[idx[:, corner]]
            if level_mask is not None:
                acc = acc * level_mask[l]
            feats.append(acc)
        return np.concatenate(feats, axis=1)


def hashgrid_3d(table_size: int = 2 ** 19, n_levels: int = 16, n_min: int = 16, n_max: int = 2048) -> HashGrid:
    return HashGrid(3, n_levels, table_size, n_min, n_max)


def world_to_unit(x, lo: float = -1.5, hi: float = 1.5):
    """Maps the world box [lo, hi]^3 onto the unit cube as float32 operations:
    (x - lo) / (hi - lo)."""
    x = np.asarray(x, dtype=np.float32)
    return (x - f32(lo)) / f32(hi - lo)


# ----------------------------------------------------------------------------
# Spherical harmonics (16 terms, degrees 0..3)
# ----------------------------------------------------------------------------

_SH_C = {
    "c0": 0.5 * math.sqrt(1.0 / math.pi),
    "c1": math.sqrt(3.0 / (4.0 * math.pi)),
    "c2a": 0.5 * math.sqrt(15.0 / math.pi),
    "c2b": 0.25 * math.sqrt(5.0 / math.pi),
    "c2c": 0.25 * math.sqrt(15.0 / math.pi),
    "c3a": 0.25 * math.sqrt(35.0 / (2.0 * math.pi)),
    "c3b": 0.5 * math.sqrt(105.0 / math.pi),
    "c3c": 0.25 * math.sqrt(21.0 / (2.0 * math.pi)),
    "c3d": 0.25 * math.sqrt(7.0 / math.pi),
    "c3e": 0.25 * math.sqrt(105.0 / math.pi),
}


def sh16(v) -> np.ndarray:
    """Real orthonormal spherical harmonics of a unit vector (x, y, z), degrees
    0 to 3, ordered by degree l then order m = -l..l, with the normalisation
    sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) (times sqrt 2 for m != 0) and no
    Condon-Shortley phase.  Float64 [..., 16]."""
    v = np.asarray(v, dtype=np.float64)
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    c = _SH_C
    xx, yy, zz = x * x, y * y, z * z
    out = [
        np.full_like(x, c["c0"]),
        c["c1"] * y, c["c1"] * z, c["c1"] * x,
        c["c2a"] * x * y, c["c2a"] * y * z, c["c2b"] * (3.0 * zz - 1.0), c["c2a"] * x * z, c["c2c"] * (xx - yy),
        c["c3a"] * y * (3.0 * xx - yy), c["c3b"] * x * y * z, c["c3c"] * y * (5.0 * zz - 1.0),
        c["c3d"] * z * (5.0 * zz - 3.0), c["c3c"] * x * (5.0 * zz - 1.0), c["c3e"] * z * (xx - yy),
        c["c3a"] * x * (xx - 3.0 * yy),
    ]
    return np.stack(out, axis=-1)

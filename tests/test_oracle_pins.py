"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties a part of ``oracle/`` to something other than itself: values
the pages print (``tests/golden/``), closed forms, invariants, library
routines for special cases, or brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import seeded_inputs as si
from oracle import composite, encoding, mlp, philox, rays, render, sampling


def _read_rows(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------
# Philox (random numbers the method draws)
# ----------------------------------------------------------------------------

def test_philox_known_answers(golden_dir):
    for row in _read_rows(os.path.join(golden_dir, "philox4x32_10_kat.txt")):
        v = [int(t, 16) for t in row]
        out = philox.philox4x32_10(tuple(v[0:4]), tuple(v[4:6]))
        assert [int(o) for o in out] == v[6:10]


def test_philox_uniform_statistics():
    n = 1 << 20
    u = philox.uniforms(0, philox.STREAM_JITTER, np.arange(n) // 64, np.arange(n) % 64).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    hist, _ = np.histogram(u, bins=256, range=(0.0, 1.0))
    chi2 = ((hist - n / 256) ** 2 / (n / 256)).sum()
    assert scipy.stats.chi2.sf(chi2, 255) > 1e-4
    lag1 = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(lag1) < 5.0 / math.sqrt(n)
    # distinct streams and seeds give unrelated sequences
    u1 = philox.uniforms(0, philox.STREAM_PDF, np.arange(n) // 64, np.arange(n) % 64).astype(np.float64)
    u2 = philox.uniforms(1, philox.STREAM_JITTER, np.arange(n) // 64, np.arange(n) % 64).astype(np.float64)
    assert abs(np.corrcoef(u, u1)[0, 1]) < 5.0 / math.sqrt(n)
    assert abs(np.corrcoef(u, u2)[0, 1]) < 5.0 / math.sqrt(n)


def test_philox_uniform_is_24bit_grid():
    u = philox.uniforms(7, 0, np.arange(4096), 3).astype(np.float64)
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))


# ----------------------------------------------------------------------------
# Rays
# ----------------------------------------------------------------------------

def test_rays_identity_pose_closed_form():
    H, W, f = 6, 8, 40.0
    c2w = np.eye(3, 4, dtype=np.float32)
    o, d = rays.get_rays(H, W, f, f, 0.5 * W, 0.5 * H, c2w)
    for j in range(H):
        for i in range(W):
            r = j * W + i  # row-major pixel order
            assert d[r, 0] == np.float32((i - W / 2) / f)
            assert d[r, 1] == np.float32(-(j - H / 2) / f)
            assert d[r, 2] == -1.0
    assert np.all(o == 0)


def test_rays_centre_pixel_points_at_origin():
    P = si.poses(4, seed=0, hemisphere=True)
    for c2w in P:
        H = W = 32
        o, d = rays.get_rays(H, W, 40.0, 40.0, 16.0, 16.0, c2w)
        centre = 16 * W + 16  # (i - W/2) = (j - H/2) = 0
        assert np.allclose(np.linalg.norm(d[centre]), 1.0, atol=1e-6)
        assert np.allclose(o[centre] + 4.0 * d[centre].astype(np.float64), 0.0, atol=1e-5)
        # every ray has z_cam = -1 before rotation, so |d| >= 1
        assert np.all(np.linalg.norm(d.astype(np.float64), axis=1) >= 1.0 - 1e-6)


def test_poses_on_sphere_and_hemisphere():
    hemi = si.poses(16, seed=0, hemisphere=True)
    sph = si.poses(64, seed=0, hemisphere=False)
    assert np.allclose(np.linalg.norm(hemi[:, :, 3], axis=1), 4.0, atol=1e-5)
    assert np.all(hemi[:, 2, 3] >= 0)
    assert np.any(sph[:, 2, 3] < 0)
    for c2w in hemi:
        R = c2w[:, :3].astype(np.float64)
        assert np.allclose(R.T @ R, np.eye(3), atol=1e-6)


# ----------------------------------------------------------------------------
# Stratified samples, points
# ----------------------------------------------------------------------------

def test_stratified_without_jitter_closed_form():
    near = np.full(5, 2.0, np.float32)
    far = np.full(5, 6.0, np.float32)
    z = sampling.stratified(near, far, 16, seed=0, jitter=False)
    assert np.allclose(z, 2.0 + (np.arange(16) + 0.5) * 0.25, atol=0)


def test_stratified_each_sample_in_its_stratum_and_uniform():
    R, N = 2048, 64
    near = np.full(R, 2.0, np.float32)
    far = np.full(R, 6.0, np.float32)
    z = sampling.stratified(near, far, N, seed=0, jitter=True).astype(np.float64)
    step = 4.0 / N
    lo = 2.0 + np.arange(N) * step
    assert np.all(z >= lo - 1e-6) and np.all(z <= lo + step + 1e-6)
    assert np.all(np.diff(z, axis=1) >= 0)
    frac = ((z - lo) / step).ravel()
    assert scipy.stats.kstest(frac, "uniform").pvalue > 1e-4


def test_points_on_the_ray():
    o = np.array([[1.0, 2.0, 3.0]], np.float32)
    d = np.array([[0.5, -0.25, 2.0]], np.float32)
    z = np.array([[0.0, 1.0, 4.0]], np.float32)
    x = sampling.points(o, d, z)
    assert np.array_equal(x[0], np.array([[1, 2, 3], [1.5, 1.75, 5.0], [3.0, 1.0, 11.0]], np.float32))


# ----------------------------------------------------------------------------
# Frequency encoding
# ----------------------------------------------------------------------------

def test_freq_encoding_widths():
    for L, w in ((10, 63), (4, 27), (6, 39)):
        assert encoding.freq_encode(np.zeros((1, 3), np.float32), L).shape == (1, w)


def test_freq_encoding_closed_forms_at_dyadic_points():
    x = np.array([[0.5, 0.25, -1.0]], np.float32)
    g = encoding.freq_encode(x, 10)[0]
    assert np.array_equal(g[:3], x[0].astype(np.float64))
    for k in range(10):
        s = g[3 + 6 * k: 6 + 6 * k]
        c = g[6 + 6 * k: 9 + 6 * k]
        # x = 1/2: sin(pi/2)=1, cos=0 at k=0; sin=0, cos=+-1 afterwards
        if k == 0:
            assert abs(s[0] - 1.0) < 1e-15 and abs(c[0]) < 1e-15
        else:
            assert abs(s[0]) < 1e-12 and abs(abs(c[0]) - 1.0) < 1e-15
        # x = 1/4 at k=0: sqrt(2)/2 both; k=1: sin=1, cos=0
        if k == 0:
            assert abs(s[1] - math.sqrt(0.5)) < 1e-15 and abs(c[1] - math.sqrt(0.5)) < 1e-15
        if k == 1:
            assert abs(s[1] - 1.0) < 1e-15 and abs(c[1]) < 1e-15
        # x = -1: sin(pi 2^k (-1)) = 0; cos = -1 at k=0, +1 later
        assert abs(s[2]) < 1e-12
        assert abs(c[2] - (-1.0 if k == 0 else 1.0)) < 1e-15


def test_freq_encoding_without_pi_is_plain_sin():
    x = np.array([[0.3, -1.7, 2.2]], np.float32)
    g = encoding.freq_encode(x, 4, use_pi=False)[0]
    for k in range(4):
        assert np.allclose(g[3 + 6 * k: 6 + 6 * k], np.sin(x[0].astype(np.float64) * 2 ** k), atol=0, rtol=1e-15)
        assert np.allclose(g[6 + 6 * k: 9 + 6 * k], np.cos(x[0].astype(np.float64) * 2 ** k), atol=0, rtol=1e-15)


# ----------------------------------------------------------------------------
# Hash grid
# ----------------------------------------------------------------------------

def test_hashgrid2d_experiment1_table(golden_dir):
    rows = _read_rows(os.path.join(golden_dir, "hashgrid2d_experiment1.txt"))
    g = encoding.HashGrid(2, 8, 2 ** 12, 8, 160)
    assert g.res == [int(r[1]) for r in rows]
    assert [(N + 1) ** 2 for N in g.res] == [int(r[2]) for r in rows]
    assert g.direct == [r[3] == "direct" for r in rows]


def test_hashgrid2d_experiment4_hashed_levels(golden_dir):
    for T, n_hash, L in (map(int, r) for r in _read_rows(os.path.join(golden_dir, "hashgrid2d_experiment4.txt"))):
        g = encoding.HashGrid(2, L, T, 8, 160)
        assert sum(not d for d in g.direct) == n_hash


def test_hashgrid3d_layout():
    g = encoding.hashgrid_3d()
    assert g.res == [16, 22, 31, 42, 58, 81, 111, 154, 213, 294, 406, 562, 776, 1072, 1482, 2048]
    assert g.direct == [True] * 5 + [False] * 11
    assert g.sizes[:5] == [(N + 1) ** 3 for N in g.res[:5]]
    assert all(s == 2 ** 19 for s in g.sizes[5:])


def test_hash_reduces_to_2d_toolkit_form():
    # with z = 0 the 3D hash is the toolkit's 2D form ix ^ iy*2654435761 mod T
    ix = np.arange(0, 3000, 7)
    iy = (ix * 13) % 2049
    h3 = encoding.hash_index([ix, iy, np.zeros_like(ix)], 2 ** 19)
    ref = [(int(a) ^ (int(b) * 2654435761)) % 2 ** 19 for a, b in zip(ix, iy)]
    assert h3.tolist() == ref


def test_hash_low_bits_equal_uint32_wraparound():
    g = np.random.default_rng(0)
    c = g.integers(0, 2049, size=(3, 200000))
    h = encoding.hash_index(list(c), 2 ** 19)
    c32 = c.astype(np.uint32)
    with np.errstate(over="ignore"):
        h32 = (c32[0] * np.uint32(1)) ^ (c32[1] * np.uint32(2654435761)) ^ (c32[2] * np.uint32(805459861))
    assert np.array_equal(h, (h32 & np.uint32(2 ** 19 - 1)).astype(np.int64))


def test_direct_levels_are_bijections():
    g = encoding.hashgrid_3d()
    for l in range(5):
        N = g.res[l]
        ax = np.arange(N + 1)
        X, Y, Z = np.meshgrid(ax, ax, ax, indexing="ij")
        idx = encoding.direct_index([X.ravel(), Y.ravel(), Z.ravel()], N)
        assert np.array_equal(np.sort(idx), np.arange((N + 1) ** 3))


def test_hashgrid_interpolation_reproduces_linear_field():
    # On a direct level, a table holding a linear function of the vertex
    # coordinates is reproduced exactly by multilinear interpolation.
    g = encoding.HashGrid(3, 2, 2 ** 19, 16, 22)
    x = si.query_points(500, seed=3)
    tables = []
    for l, N in enumerate(g.res):
        ax = np.arange(N + 1, dtype=np.float64)
        X, Y, Z = np.meshgrid(ax, ax, ax, indexing="ij")
        idx = encoding.direct_index([X.ravel().astype(int), Y.ravel().astype(int), Z.ravel().astype(int)], N)
        t = np.zeros((g.sizes[l], 2))
        t[idx, 0] = 0.5 * X.ravel() - 2.0 * Y.ravel() + 0.25 * Z.ravel()
        t[idx, 1] = 1.0 + Z.ravel()
        tables.append(t)
    out = g.encode(x, tables)
    for l, N in enumerate(g.res):
        c = (x * np.float32(N)).astype(np.float64)
        assert np.allclose(out[:, 2 * l], 0.5 * c[:, 0] - 2.0 * c[:, 1] + 0.25 * c[:, 2], atol=1e-9)
        assert np.allclose(out[:, 2 * l + 1], 1.0 + c[:, 2], atol=1e-9)


def test_hashgrid_vertex_and_partition_of_unity():
    g = encoding.hashgrid_3d()
    tabs = si.hash_tables(g.sizes, seed=0, scale=1.0)
    # partition of unity: a constant table gives that constant
    const = [np.full((s, 2), 0.75, np.float16) for s in g.sizes]
    x = si.query_points(256, seed=1)
    assert np.allclose(g.encode(x, const), 0.75, atol=1e-12)
    # at a vertex the output is that vertex's table entry
    N = g.res[7]
    v = np.array([[3, 100, 47]])
    xv = (v / N).astype(np.float32)
    idx, w = g.level_indices(xv, 7)
    if np.all(w == 0):
        out = g.encode(xv, tabs)[0, 14:16]
        h = encoding.hash_index([v[:, 0], v[:, 1], v[:, 2]], 2 ** 19)[0]
        assert np.allclose(out, tabs[7][h].astype(np.float64), atol=0)


def test_hashgrid_brute_force_single_point():
    g = encoding.hashgrid_3d()
    tabs = si.hash_tables(g.sizes, seed=0, scale=1.0)
    p = np.array([[0.3141, 0.5926, 0.5358]], np.float32)
    out = g.encode(p, tabs)[0]
    for l, N in enumerate(g.res):
        c = [float(np.float32(p[0, a]) * np.float32(N)) for a in range(3)]
        c0 = [math.floor(t) for t in c]
        fr = [t - math.floor(t) for t in c]
        acc = [0.0, 0.0]
        for dx in (0, 1):
            for dy in (0, 1):
                for dz in (0, 1):
                    ix, iy, iz = (min(max(c0[0] + dx, 0), N), min(max(c0[1] + dy, 0), N), min(max(c0[2] + dz, 0), N))
                    if (N + 1) ** 3 <= 2 ** 19:
                        idx = (ix * (N + 1) + iy) * (N + 1) + iz
                    else:
                        idx = (ix ^ (iy * 2654435761) ^ (iz * 805459861)) % (2 ** 19)
                    wt = (fr[0] if dx else 1 - fr[0]) * (fr[1] if dy else 1 - fr[1]) * (fr[2] if dz else 1 - fr[2])
                    acc[0] += wt * float(tabs[l][idx, 0])
                    acc[1] += wt * float(tabs[l][idx, 1])
        assert np.allclose(out[2 * l: 2 * l + 2], acc, atol=1e-12)


# ----------------------------------------------------------------------------
# Spherical harmonics
# ----------------------------------------------------------------------------

def test_sh16_matches_scipy_real_harmonics():
    g = np.random.default_rng(1)
    v = g.normal(size=(300, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    polar = np.arccos(np.clip(v[:, 2], -1, 1))
    azim = np.arctan2(v[:, 1], v[:, 0])
    ours = encoding.sh16(v)
    col = 0
    for l in range(4):
        for m in range(-l, l + 1):
            Y = scipy.special.sph_harm_y(l, abs(m), polar, azim)
            if m == 0:
                ref = Y.real
            elif m > 0:
                ref = math.sqrt(2) * (-1) ** m * Y.real
            else:
                ref = math.sqrt(2) * (-1) ** m * Y.imag
            assert np.allclose(ours[:, col], ref, atol=1e-12), (l, m)
            col += 1


def test_sh16_orthonormal_by_quadrature():
    n = 100000
    k = np.arange(n) + 0.5
    z = 1 - 2 * k / n
    r = np.sqrt(1 - z * z)
    phi = math.pi * (1 + 5 ** 0.5) * k
    v = np.stack([r * np.cos(phi), r * np.sin(phi), z], 1)
    Y = encoding.sh16(v)
    G = Y.T @ Y * (4 * math.pi / n)
    assert np.allclose(G, np.eye(16), atol=1e-3)
    assert abs(Y[0, 0] - 1 / (2 * math.sqrt(math.pi))) < 1e-15


# ----------------------------------------------------------------------------
# Networks
# ----------------------------------------------------------------------------

def test_parameter_count_convention(golden_dir):
    for name, dims, count in _read_rows(os.path.join(golden_dir, "mlp_param_counts.txt")):
        layers = [tuple(map(int, d.split(":"))) for d in dims.split(",")]
        assert sum(i * o + o for i, o in layers) == int(count)
    for shape, expect in ((si.NERF_8x256, 595844), (si.NERF_4x64, 22308), (si.NERF_CELL_2x32, 5204)):
        p = si.nerf_params(shape, seed=0)
        n = sum(W.size + b.size for W, b in p["layers"])
        n += sum(p[k][0].size + p[k][1].size for k in ("sigma", "feature", "dir", "rgb"))
        assert n == shape.n_params() == expect


@pytest.mark.parametrize("shape", [si.NERF_4x64, si.NERF_8x256, si.NERF_CELL_2x32])
def test_nerf_forward_matches_naive_loops(shape):
    p = si.nerf_params(shape, seed=5)
    g = np.random.default_rng(2)
    pe = g.normal(size=(3, shape.pos_ch))
    de = g.normal(size=(3, shape.dir_ch))
    assert np.allclose(mlp.nerf_forward(p, pe, de), mlp.nerf_forward_naive(p, pe, de), atol=1e-10, rtol=1e-12)


def test_nerf_zero_weights_give_biases():
    p = si.nerf_params(si.NERF_8x256, seed=0)
    z = {k: (np.zeros_like(p[k][0]), p[k][1]) for k in ("sigma", "feature", "dir", "rgb")}
    q = dict(p, layers=[(np.zeros_like(W), b) for W, b in p["layers"]], **z)
    out = mlp.nerf_forward(q, np.ones((2, 63)), np.ones((2, 27)))
    assert np.allclose(out[:, :3], p["rgb"][1]) and np.allclose(out[:, 3], p["sigma"][1][0])


def test_nerf_skip_concatenates_encoding_after_hidden_state():
    # All layers zero except the position-encoding columns of the layer after
    # the skip, identity layers after it: sigma = w . relu(A gamma).
    s = si.NERF_8x256
    p = si.nerf_params(s, seed=1)
    W = s.width
    layers = []
    for i, (Wl, bl) in enumerate(p["layers"]):
        Wz = np.zeros_like(Wl)
        if i == s.skip + 1:
            Wz[:, W:] = Wl[:, W:]
        elif i > s.skip + 1:
            Wz = np.eye(W, dtype=np.float32)
        layers.append((Wz, np.zeros_like(bl)))
    q = dict(p, layers=layers, sigma=(p["sigma"][0], np.zeros(1, np.float32)))
    g = np.random.default_rng(3)
    pe = g.normal(size=(4, 63))
    out = mlp.nerf_forward(q, pe, np.zeros((4, 27)))
    A = p["layers"][s.skip + 1][0][:, W:].astype(np.float64)
    expect = np.maximum(pe @ A.T, 0) @ p["sigma"][0][0].astype(np.float64)
    assert np.allclose(out[:, 3], expect, atol=1e-9)
    assert np.abs(expect).max() > 0.1


def test_hash_field_forward_matches_naive_loops():
    p = si.hash_field_params(seed=4)
    g = np.random.default_rng(8)
    feats = g.normal(size=(4, 32))
    de = g.normal(size=(4, 16))
    assert np.allclose(mlp.hash_field_forward(p, feats, de), mlp.hash_field_forward_naive(p, feats, de), atol=1e-10,
                       rtol=1e-12)


def test_hash_field_zero_weights_give_biases():
    p = si.hash_field_params(seed=0)
    zero = lambda Wb: (np.zeros_like(Wb[0]), Wb[1])  # noqa: E731
    q = dict(p, density=[zero(x) for x in p["density"]], color=[zero(x) for x in p["color"]],
             **{k: zero(p[k]) for k in ("sigma", "feature", "rgb")})
    out = mlp.hash_field_forward(q, np.ones((3, 32)), np.ones((3, 16)))
    assert np.allclose(out[:, :3], p["rgb"][1]) and np.allclose(out[:, 3], p["sigma"][1][0])


def test_hash_field_density_ignores_direction_and_colour_reads_features_through_the_feature_layer():
    p = si.hash_field_params(seed=2)
    g = np.random.default_rng(9)
    feats = np.repeat(g.normal(size=(1, 32)), 5, axis=0)
    de = g.normal(size=(5, 16))
    out = mlp.hash_field_forward(p, feats, de)
    assert np.all(out[:, 3] == out[0, 3])            # density: grid features only
    assert np.ptp(out[:, 0]) > 1e-3                  # colour: depends on the direction
    # with a zero feature layer the colour no longer depends on the grid features
    q = dict(p, feature=(np.zeros_like(p["feature"][0]), p["feature"][1]))
    f2 = g.normal(size=(5, 32))
    de2 = np.repeat(de[:1], 5, axis=0)
    o2 = mlp.hash_field_forward(q, f2, de2)
    assert np.allclose(o2[:, :3], o2[0, :3], atol=1e-14) and np.ptp(o2[:, 3]) > 1e-3


def test_round_bf16_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, -2.5, 1e-3], np.float32)
    r = mlp.round_bf16(vals)
    assert r[0] == 1.0
    assert r[1] == 1.0 + 2 ** -7 or r[1] == 1.0  # tie 1+2^-8: even mantissa -> 1.0
    assert r[1] == 1.0
    assert r[2] == 1.0
    assert r[3] == 1.0 + 2 ** -7
    assert r[4] == -2.5
    assert abs(r[5] - 1e-3) <= 1e-3 * 2 ** -8


# ----------------------------------------------------------------------------
# Compositing
# ----------------------------------------------------------------------------

def _const_raw(R, N, rgb_raw, sigma):
    raw = np.zeros((R, N, 4))
    raw[..., :3] = rgb_raw
    raw[..., 3] = sigma
    return raw


def test_constant_density_transmittance_closed_form():
    R, N = 3, 64
    z = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), N, seed=0)
    d = np.array([[0.0, 0.0, -1.0], [0.6, 0.0, 0.8], [1.0, 1.0, 1.0]], np.float32)
    sigma = 0.7
    rgb, depth, acc, w = composite.volume_render(_const_raw(R, N, 0.3, sigma), z, d)
    dn = np.linalg.norm(d.astype(np.float64), axis=1)
    z64 = z.astype(np.float64)
    # 1 - sum_{j<i} w_j equals T_i up to the 1e-10 term (at most 64e-10)
    T = np.concatenate([np.ones((R, 1)), 1 - np.cumsum(w, 1)[:, :-1]], 1)
    T_closed = np.exp(-sigma * (z64 - z64[:, :1]) * dn[:, None])
    assert np.allclose(T, T_closed, rtol=1e-7, atol=1e-8)
    # colour is constant, so rgb = sigmoid(0.3) * acc
    assert np.allclose(rgb, (1 / (1 + math.exp(-0.3))) * acc[:, None], atol=1e-14)


def test_weights_telescope_exactly():
    g = np.random.default_rng(4)
    R, N = 8, 64
    raw = g.normal(size=(R, N, 4)) * 3
    z = np.sort(g.uniform(2, 6, size=(R, N)), axis=1).astype(np.float32)
    d = g.normal(size=(R, 3)).astype(np.float32)
    _, _, acc, w = composite.volume_render(raw, z, d)
    dn = np.linalg.norm(d.astype(np.float64), axis=1, keepdims=True)
    dist = np.concatenate([np.diff(z.astype(np.float64), axis=1), np.full((R, 1), 1e10)], 1) * dn
    alpha = 1 - np.exp(-np.maximum(raw[..., 3], 0) * dist)
    T = np.ones(R)
    Tsum = np.zeros(R)
    for i in range(N):
        Tsum += T
        T = T * (1 - alpha[:, i] + 1e-10)
    assert np.allclose(acc, 1 - T + 1e-10 * Tsum, atol=1e-13)


def test_composite_special_cases():
    R, N = 2, 16
    z = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), N, 0, jitter=False)
    d = np.array([[0, 0, -1], [0, 1, 0]], np.float32)
    rgb, depth, acc, w = composite.volume_render(_const_raw(R, N, 1.0, 0.0), z, d)
    assert np.all(rgb == 0) and np.all(depth == 0) and np.all(acc == 0)
    rgbw, _, _, _ = composite.volume_render(_const_raw(R, N, 1.0, 0.0), z, d, white_bkgd=True)
    assert np.allclose(rgbw, 1.0)
    raw = _const_raw(R, N, 0.0, 0.0)
    raw[:, 5, 3] = 1e6  # one opaque sample
    raw[:, 5, :3] = 2.0
    rgb, depth, acc, w = composite.volume_render(raw, z, d)
    assert np.allclose(w[:, 5], 1.0) and np.allclose(acc, 1.0)
    assert np.allclose(depth, z[:, 5]) and np.allclose(rgb, 1 / (1 + math.exp(-2.0)))
    # the last sample absorbs everything that is left (delta = 1e10)
    raw = _const_raw(R, N, 0.0, 0.0)
    raw[:, -1, 3] = 1e-3
    _, _, acc, _ = composite.volume_render(raw, z, d)
    assert np.allclose(acc, 1.0)


def test_early_termination_drops_samples_after_threshold():
    R, N = 4, 64
    z = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), N, 0, jitter=False)
    d = np.tile(np.array([[0, 0, -1]], np.float32), (R, 1))
    raw = _const_raw(R, N, 0.5, 2.0)
    rgb0, _, acc0, w0 = composite.volume_render(raw, z, d)
    rgb1, _, acc1, w1 = composite.volume_render(raw, z, d, term_T=1e-2)
    T = np.cumprod(np.concatenate([np.ones((R, 1)), 1 - (1 - np.exp(-2.0 * 0.0625)) + 1e-10 + np.zeros((R, N))], 1), 1)[:, :N]
    first = np.argmax(T < 1e-2, axis=1)
    for r in range(R):
        assert np.all(w1[r, first[r]:] == 0)
        assert np.allclose(w1[r, :first[r]], w0[r, :first[r]])
    assert np.all(acc1 < acc0) and np.all(acc1 > 0.99 - 1e-9)


# ----------------------------------------------------------------------------
# Inverse-CDF resampling
# ----------------------------------------------------------------------------

def test_sample_pdf_bins_match_linear_scan():
    g = np.random.default_rng(5)
    R, Nc = 64, 64
    zc = np.sort(g.uniform(2, 6, size=(R, Nc)), axis=1).astype(np.float32)
    w = (g.random((R, Nc)) ** 4).astype(np.float32)
    bins = sampling.midpoints(zc)
    wm = w[:, 1:-1]
    zf, idx = sampling.sample_pdf(bins, wm, 128, seed=3)
    u = philox.uniforms(3, philox.STREAM_PDF, np.arange(R)[:, None], np.arange(128)[None, :])
    for r in range(R):
        wp = [float(np.float32(v) + np.float32(1e-5)) for v in wm[r]]
        tot = math.fsum(wp)
        cdf = [0.0] + [math.fsum(wp[: k + 1]) / tot for k in range(len(wp))]
        for m in range(128):
            cnt = sum(1 for c in cdf if c <= float(u[r, m]))
            assert idx[r, m] == cnt
            assert bins[r, cnt - 1] <= zf[r, m] <= bins[r, cnt]


def test_sample_pdf_uniform_pdf_gives_uniform_samples():
    R, Nc = 16, 64
    near = np.full(R, 2.0, np.float32)
    zc = sampling.stratified(near, np.full(R, 6.0, np.float32), Nc, 0, jitter=False)
    bins = sampling.midpoints(zc)
    zf, _ = sampling.sample_pdf(bins, np.full((R, Nc - 2), 0.5, np.float32), 128, seed=9)
    u = philox.uniforms(9, philox.STREAM_PDF, np.arange(R)[:, None], np.arange(128)[None, :]).astype(np.float64)
    lin = bins[:, :1].astype(np.float64) + u * (bins[:, -1:].astype(np.float64) - bins[:, :1])
    assert np.allclose(zf, lin, atol=2e-6)


def test_sample_pdf_spike_mass():
    R, Nc, Nf = 256, 64, 128
    zc = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), Nc, 0, jitter=False)
    w = np.zeros((R, Nc - 2), np.float32)
    w[:, 20] = 1.0
    _, idx = sampling.sample_pdf(sampling.midpoints(zc), w, Nf, seed=1)
    p_spike = (1.0 + 1e-5) / (1.0 + 62 * 1e-5)
    frac = np.mean(idx == 21)
    n = R * Nf
    assert abs(frac - p_spike) < 5 * math.sqrt(p_spike * (1 - p_spike) / n) + 1e-4


def test_midpoints_lie_between_consecutive_samples():
    R, N = 4, 64
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    zc = sampling.stratified(near, far, N, 0, jitter=False)  # z_i = 2 + (i + 1/2) / 16
    b = sampling.midpoints(zc)
    assert b.shape == (R, N - 1)
    k = np.arange(N - 1, dtype=np.float64)
    assert np.array_equal(b.astype(np.float64), np.broadcast_to(2.0 + (k + 1.0) / 16.0, (R, N - 1)))
    zj = sampling.stratified(near, far, N, 5)
    bj = sampling.midpoints(zj)
    assert np.all((bj > zj[:, :-1]) & (bj < zj[:, 1:]))


@pytest.mark.parametrize("k", [1, 2, 31, 61, 62])
def test_hierarchical_spike_goes_to_the_bin_around_its_coarse_sample(k):
    """One coarse weight spike at sample k (Section 2 Code, 6. Hierarchical
    sampling: bins are midpoints of the coarse samples, weights drop the two
    end samples): a fraction (1 + 1e-5) / (1 + 62e-5) of the fine samples lands
    in [b_{k-1}, b_k], the bin that contains coarse sample k."""
    R, Nc, Nf = 256, 64, 128
    zc = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), Nc, 4)
    w = np.zeros((R, Nc), np.float32)
    w[:, k] = 1.0
    zf, idx, _ = sampling.hierarchical_fine_samples(zc, w, Nf, seed=7)
    b = sampling.midpoints(zc)
    assert np.all((b[:, k - 1] < zc[:, k]) & (zc[:, k] < b[:, k]))
    inside = (zf >= b[:, k - 1:k]) & (zf <= b[:, k:k + 1])
    p = (1.0 + 1e-5) / (1.0 + 62 * 1e-5)
    n = R * Nf
    assert abs(inside.mean() - p) < 5 * math.sqrt(p * (1 - p) / n) + 1e-4
    assert np.all(inside == (idx == k))


@pytest.mark.parametrize("k", [0, 63])
def test_hierarchical_end_sample_weights_are_ignored(k):
    """A spike on an end sample (excluded by the page's weights[1:-1]) leaves a
    uniform pdf over the 62 bins."""
    R, Nc, Nf = 512, 64, 128
    zc = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), Nc, 0, jitter=False)
    w = np.zeros((R, Nc), np.float32)
    w[:, k] = 1.0
    _, idx, _ = sampling.hierarchical_fine_samples(zc, w, Nf, seed=8)
    counts = np.bincount(idx.reshape(-1) - 1, minlength=62)
    chi2 = scipy.stats.chisquare(counts)
    assert counts.size == 62 and chi2.pvalue > 1e-4


def test_hierarchical_uniform_weights_map_u_linearly():
    """Equal weights on evenly spaced coarse samples z_i = near + (i + 1/2) s:
    the fine samples are near + s + u * 62 s, the linear map of the uniforms
    onto [b_0, b_62]."""
    R, Nc, Nf = 32, 64, 128
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    zc = sampling.stratified(near, far, Nc, 0, jitter=False)
    zf, _, _ = sampling.hierarchical_fine_samples(zc, np.full((R, Nc), 0.25, np.float32), Nf, seed=13,
                                                  ray_offset=77)
    u = philox.uniforms(13, philox.STREAM_PDF, (77 + np.arange(R))[:, None], np.arange(Nf)[None, :])
    s = 4.0 / 64
    assert np.allclose(zf, 2.0 + s + u.astype(np.float64) * 62 * s, atol=2e-6, rtol=0)


def test_hierarchical_merge_is_sorted_union():
    g = np.random.default_rng(6)
    R = 8
    zc = sampling.stratified(np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32), 64, 0)
    w = g.random((R, 64)).astype(np.float32)
    zf, idx, z2 = sampling.hierarchical_fine_samples(zc, w, 128, seed=2)
    assert z2.shape == (R, 192)
    assert np.all(np.diff(z2, axis=1) >= 0)
    for r in range(R):
        assert sorted(np.concatenate([zc[r], zf[r]]).tolist()) == z2[r].tolist()
    assert idx.min() >= 1 and idx.max() <= 62


# ----------------------------------------------------------------------------
# End-to-end renders on fields with closed forms
# ----------------------------------------------------------------------------

def _constant_field(shape, rgb_raw, sigma_raw):
    p = si.nerf_params(shape, seed=0)
    q = dict(p)
    q["layers"] = [(np.zeros_like(W), np.zeros_like(b)) for W, b in p["layers"]]
    q["sigma"] = (np.zeros_like(p["sigma"][0]), np.full(1, sigma_raw, np.float32))
    q["feature"] = (np.zeros_like(p["feature"][0]), np.zeros_like(p["feature"][1]))
    q["dir"] = (np.zeros_like(p["dir"][0]), np.zeros_like(p["dir"][1]))
    q["rgb"] = (np.zeros_like(p["rgb"][0]), np.array(rgb_raw, np.float32))
    return q


def test_render_constant_field_closed_form():
    R = 32
    c2w = si.poses(1, seed=0)[0]
    o, d = rays.get_rays(4, 8, 40.0, 40.0, 4.0, 2.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    q = _constant_field(si.NERF_4x64, [0.2, -0.4, 1.0], 0.5)
    out = render.render_nerf(o, d, near, far, q, q, n_coarse=16, n_fine=32, L_pos=6, L_dir=4, seed=0)
    dn = np.linalg.norm(d.astype(np.float64), axis=1)
    z2 = out["z2"].astype(np.float64)
    T_last = np.exp(-0.5 * (z2[:, -1] - z2[:, 0]) * dn)
    acc = 1.0 - T_last  # last sample's delta is 1e10: everything left is absorbed
    assert np.allclose(out["acc"], 1.0, atol=1e-6)
    sig = 1 / (1 + np.exp(-np.array([0.2, -0.4, 1.0])))
    assert np.allclose(out["rgb"], sig[None, :] * out["acc"][:, None], atol=1e-12)
    assert np.all(T_last > 0)


def _zero_hash_field(rgb_raw, sigma_raw):
    p = si.hash_field_params(seed=0)
    zero = lambda Wb: (np.zeros_like(Wb[0]), np.zeros_like(Wb[1]))  # noqa: E731
    q = dict(p, density=[zero(x) for x in p["density"]], color=[zero(x) for x in p["color"]],
             feature=zero(p["feature"]))
    q["sigma"] = (np.zeros_like(p["sigma"][0]), np.full(1, sigma_raw, np.float32))
    q["rgb"] = (np.zeros_like(p["rgb"][0]), np.array(rgb_raw, np.float32))
    return q


def test_render_hash_constant_field_closed_form():
    R = 32
    c2w = si.poses(1, seed=1)[0]
    o, d = rays.get_rays(4, 8, 40.0, 40.0, 4.0, 2.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    grid = encoding.hashgrid_3d()
    tabs = si.hash_tables(grid.sizes, seed=0, scale=1.0)
    q = _zero_hash_field([0.3, -1.0, 0.6], 0.4)
    out = render.render_hash(o, d, near, far, grid, tabs, q, n_samples=48, seed=0)
    dn = np.linalg.norm(d.astype(np.float64), axis=1)
    z = out["z"].astype(np.float64)
    # 1 - sum_{j<i} w_j = T_i = exp(-sigma (z_i - z_0) |d|) up to the 1e-10 term
    T = np.concatenate([np.ones((R, 1)), 1 - np.cumsum(out["w"], 1)[:, :-1]], 1)
    assert np.allclose(T, np.exp(-0.4 * (z - z[:, :1]) * dn[:, None]), rtol=1e-7, atol=1e-8)
    assert np.allclose(out["acc"], 1.0, atol=1e-9)
    sig = 1 / (1 + np.exp(-np.array([0.3, -1.0, 0.6])))
    assert np.allclose(out["rgb"], sig[None, :] * out["acc"][:, None], atol=1e-12)


def test_render_hash_density_from_a_linear_coarsest_level():
    """Level 0 (direct) holds the linear function a . v / N + c of its vertex
    v; trilinear interpolation reproduces it, so with the density path reading
    only that feature, sigma_raw at a sample is relu(a . u + c) with u the
    sample point mapped from the box [-1.5, 1.5]^3 to the unit cube."""
    R = 24
    c2w = si.poses(1, seed=2)[0]
    o, d = rays.get_rays(4, 6, 30.0, 30.0, 3.0, 2.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    grid = encoding.hashgrid_3d()
    tabs = [np.zeros((s, 2), np.float64) for s in grid.sizes]
    N = grid.res[0]
    a, c = np.array([0.9, -0.6, 0.75]), -0.2
    v = np.stack(np.meshgrid(*[np.arange(N + 1)] * 3, indexing="ij"), -1).reshape(-1, 3)
    tabs[0][encoding.direct_index([v[:, 0], v[:, 1], v[:, 2]], N), 0] = v @ a / N + c
    q = _zero_hash_field([0.0, 0.0, 0.0], 0.0)
    W0 = np.zeros_like(q["density"][0][0])
    W0[0, 0] = 1.0  # level 0, feature 0
    W1 = np.zeros_like(q["density"][1][0])
    W1[0, 0] = 1.0
    q["density"] = [(W0, q["density"][0][1]), (W1, q["density"][1][1])]
    ws = np.zeros_like(q["sigma"][0])
    ws[0, 0] = 1.0
    q["sigma"] = (ws, q["sigma"][1])
    out = render.render_hash(o, d, near, far, grid, tabs, q, n_samples=40, seed=3)
    x = sampling.points(o, d, out["z"]).astype(np.float64)
    u = (x + 1.5) / 3.0
    expect = np.maximum(u @ a + c, 0.0)
    inside = np.all((u >= 0) & (u <= 1), axis=-1)
    assert inside.mean() > 0.3
    assert np.allclose(out["raw"][..., 3][inside], expect[inside], atol=1e-6)


def test_empty_space_skipping_full_and_empty_occupancy():
    """Full occupancy with every sample inside the box reproduces the render
    without skipping; empty occupancy renders nothing (white background: 1)."""
    R = 24
    c2w = si.poses(1, seed=3)[0]
    o, d = rays.get_rays(4, 6, 20.0, 20.0, 3.0, 2.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    pc, pf = si.nerf_params(si.NERF_4x64, seed=2, net_id=0), si.nerf_params(si.NERF_4x64, seed=2, net_id=1)
    base = render.render_nerf(o, d, near, far, pc, pf, 16, 32, 6, 4, seed=1)
    full = render.render_nerf(o, d, near, far, pc, pf, 16, 32, 6, 4, seed=1, occ=np.ones(32 ** 3, bool), occ_res=32,
                              box=(-10.0, 10.0))
    for k in ("rgb", "acc", "depth", "z2"):
        assert np.array_equal(base[k], full[k]), k
    assert full["n_live"] == R * (16 + 48)
    empty = render.render_nerf(o, d, near, far, pc, pf, 16, 32, 6, 4, seed=1, occ=np.zeros(32 ** 3, bool),
                               occ_res=32, white_bkgd=True)
    assert np.all(empty["acc"] == 0) and np.all(empty["depth"] == 0) and np.all(empty["rgb"] == 1.0)
    assert empty["n_live"] == 0
    grid = encoding.hashgrid_3d()
    tabs = si.hash_tables(grid.sizes, seed=0, scale=1.0)
    field = si.hash_field_params(seed=0)
    hb = render.render_hash(o, d, near, far, grid, tabs, field, 24, seed=0)
    hf = render.render_hash(o, d, near, far, grid, tabs, field, 24, seed=0, occ=np.ones(16 ** 3, bool), occ_res=16,
                            box=(-1.5, 1.5))
    inside = np.all(np.abs(sampling.points(o, d, hb["z"])) <= 1.5, axis=-1)
    assert hf["n_live"] == int(inside.sum())
    # the hash render's box also maps to the unit cube, so only the dead samples change
    assert np.array_equal(hf["raw"][inside], hb["raw"][inside]) and np.all(hf["raw"][~inside] == 0)


def test_skipped_samples_are_transparent():
    """A skipped sample has alpha 0: the render equals compositing the
    network outputs with those samples' densities set to 0 by hand."""
    R = 16
    c2w = si.poses(1, seed=4)[0]
    o, d = rays.get_rays(4, 4, 12.0, 12.0, 2.0, 2.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    p = si.nerf_params(si.NERF_4x64, seed=3)
    occ = np.random.default_rng(1).random(8 ** 3) < 0.4
    out = render.render_nerf(o, d, near, far, p, None, 32, 0, 6, 4, seed=2, occ=occ, occ_res=8, term_T=1e-2)
    z = out["z_c"]
    x = sampling.points(o, d, z)
    ref = render.nerf_pass(p, o, d, z, 6, 4)
    raw = ref["raw"].copy()
    t = (x - np.float32(-1.5)) * np.float32(8 / 3.0)
    v = np.clip(np.floor(t), 0, 7).astype(np.int64)
    inside = np.all((x >= np.float32(-1.5)) & (x <= np.float32(1.5)), axis=-1)
    live = inside & occ[(v[..., 0] * 8 + v[..., 1]) * 8 + v[..., 2]]
    raw[~live] = 0.0
    rgb, depth, acc, _ = composite.volume_render(raw, z, d, False, 1e-2)
    assert np.allclose(out["rgb"], rgb, atol=1e-12) and np.allclose(out["acc"], acc, atol=1e-12)
    assert out["n_live"] == int(live.sum()) and 0 < out["n_live"] < R * 32


def test_kilo_reduces_to_single_network_with_full_occupancy():
    R = 64
    c2w = si.poses(1, seed=0)[0]
    o, d = rays.get_rays(8, 8, 10.0, 10.0, 4.0, 4.0, c2w)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    net = si.nerf_params(si.NERF_CELL_2x32, seed=3)
    full = np.ones(128 ** 3, bool)
    k = render.render_kilo(o, d, near, far, full, lambda c: net, n_samples=48, seed=0, term_T=1e-2)
    # the same single network with the box test applied by hand
    z = sampling.stratified(near, far, 48, 0)
    x = sampling.points(o, d, z)
    inside = np.all(np.abs(x) <= 1.5, axis=-1)
    pe = encoding.freq_encode(x.reshape(-1, 3), 10)
    de = np.repeat(encoding.freq_encode(sampling.view_dirs(d), 4), 48, axis=0)
    raw = mlp.nerf_forward(net, pe, de).reshape(R, 48, 4)
    raw[~inside] = 0.0
    rgb, depth, acc, _ = composite.volume_render(raw, z, d, term_T=1e-2)
    assert np.allclose(k["rgb"], rgb, atol=1e-12) and np.allclose(k["acc"], acc, atol=1e-12)
    empty = render.render_kilo(o, d, near, far, np.zeros(128 ** 3, bool), lambda c: net, n_samples=48)
    assert np.all(empty["rgb"] == 0) and np.all(empty["acc"] == 0) and empty["n_live"] == 0


def test_kilo_voxel_and_cell_ids_brute_force():
    g = np.random.default_rng(7)
    x = g.uniform(-1.6, 1.6, size=(2000, 3)).astype(np.float32)
    x[:10] = np.float32(1.5)
    x[10:20] = np.float32(-1.5)
    occ = g.random(128 ** 3) < 0.5
    live, cell, vox = render.kilo_classify(x, occ)
    for p in range(len(x)):
        v = []
        c = []
        for a in range(3):
            t = np.float32(x[p, a]) - np.float32(-1.5)
            v.append(min(max(int(math.floor(np.float32(t * np.float32(128 / 3.0)))), 0), 127))
            c.append(min(max(int(math.floor(np.float32(t * np.float32(16 / 3.0)))), 0), 15))
        assert vox[p] == (v[0] * 128 + v[1]) * 128 + v[2]
        assert cell[p] == (c[0] * 16 + c[1]) * 16 + c[2]
        ins = all(-1.5 <= float(x[p, a]) <= 1.5 for a in range(3))
        assert live[p] == (ins and occ[vox[p]])

"""Hash-grid variants through the C ABI ("Instant-NGP - Visual Experiments"):
the 2D grid of the notebook's experiments (indices bit-exact against the
oracle at the printed configurations), level masks (coarse-to-fine
evaluation) in 2D and 3D, and a field render with a level mask."""
import ctypes

import numpy as np
import pytest

import seeded_inputs as si
from oracle import encoding as oenc
from oracle import render as oren
from tests.gpu_util import dev, empty, host, max_abs, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def v():
    torch_cuda()
    import volume_rendering_amd as v
    return v


def _points(n, dim, seed):
    x = np.random.default_rng(seed).random((n, dim)).astype(np.float32)
    edge = np.array([[0.0] * dim, [1.0] * dim, [0.5] * dim, [1.2] + [-0.1] * (dim - 1), [1e-7] + [0.9999999] * (dim - 1)],
                    np.float32)
    x[:5] = edge
    return x


def _encode(v, g, tabs, x, dim, mask=None):
    torch = torch_cuda()
    L = g.n_levels
    tdev = dev(np.concatenate(tabs, 0))
    g.tables = tdev.data_ptr()
    if mask is not None:
        for l in range(L):
            g.level_mask[l] = float(mask[l])
    n = x.shape[0]
    out = empty((n, 2 * L))
    idx = torch.full((n, L, 2 ** dim), -1, dtype=torch.int32, device="cuda")
    v.nerf_encode_hashgrid(dev(x), g, out, idx)
    return host(out), host(idx).view(np.uint32)


@pytest.mark.parametrize("T", [2 ** 12, 2 ** 8, 2 ** 14])
def test_hashgrid2d_experiment_configs(v, T):
    """8 levels from 8 to 160 in 2D: Experiment 1 (T = 2^12, 5 direct
    levels) and Experiment 4 (T = 2^8 and 2^14)."""
    say(f"2D grid T={T}")
    g = v.nerf_hashgrid_init(8, T, 8, 160, dim=2)
    og = oenc.HashGrid(2, 8, T, 8, 160)
    tabs = si.hash_tables(og.sizes, seed=5, scale=1.0)
    x = _points(4099, 2, seed=T)
    out, idx = _encode(v, g, tabs, x, 2)
    for l in range(8):
        ref_idx, _ = og.level_indices(x, l)
        assert np.array_equal(idx[:, l, :].astype(np.int64), ref_idx), l
    err = max_abs(out, og.encode(x, tabs))
    say(f"  features err {err:.2e}")
    assert err <= 8e-6


@pytest.mark.parametrize("dim", [2, 3])
def test_hashgrid_level_mask(v, dim):
    """Coarse-to-fine masks: levels with mask 0 are zero and not looked up
    (their debug indices stay untouched), others scale by the mask."""
    say(f"level mask dim={dim}")
    if dim == 2:
        g = v.nerf_hashgrid_init(8, 2 ** 12, 8, 160, dim=2)
        og = oenc.HashGrid(2, 8, 2 ** 12, 8, 160)
        mask = [1, 1, 1, 0.5, 0, 0, 0, 0]
    else:
        g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
        og = oenc.hashgrid_3d()
        mask = [1] * 6 + [0.25, 0] + [1, 0] * 4
    tabs = si.hash_tables(og.sizes, seed=6, scale=1.0)
    x = _points(3001, dim, seed=dim)
    out, idx = _encode(v, g, tabs, x, dim, mask)
    ref = og.encode(x, tabs, np.asarray(mask, np.float64))
    err = max_abs(out, ref)
    say(f"  features err {err:.2e}")
    assert err <= 8e-6
    for l, m in enumerate(mask):
        if m == 0:
            assert np.all(out[:, 2 * l:2 * l + 2] == 0.0)
            assert np.all(idx[:, l, :] == 0xFFFFFFFF)
        else:
            ref_idx, _ = og.level_indices(x, l)
            assert np.array_equal(idx[:, l, :].astype(np.int64), ref_idx)


def test_render_hash_coarse_levels_only(v):
    """A field rendered from its 6 coarsest levels (the notebook's
    coarse-to-fine evaluation), float32, against the oracle."""
    import volume_rendering_amd._binding as B
    say("hash render with a level mask")
    og = oenc.hashgrid_3d()
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    mask = [1.0] * 6 + [0.0] * 10
    for l in range(16):
        g.level_mask[l] = mask[l]
    tabs = si.hash_tables(og.sizes, seed=7, scale=1.0)
    tdev = dev(np.concatenate(tabs, 0))
    g.tables = tdev.data_ptr()
    o, d = page_rays(256, 256, 355.2, si.poses(1, seed=9)[0])
    sel = si.subset(256 * 256, 150, seed=18)
    o, d = o[sel], d[sel]
    R = len(sel)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    field = si.hash_field_params(seed=3)
    net = v.weights.pack_to_device(4, 0, field)
    w = B.nerf_weights(net=B.nerf_mlp_desc(4, 0), coarse=net.data_ptr())
    w.grid = ctypes.pointer(g)
    cfg = B.nerf_render_cfg(mode=1, n_coarse=128, use_pi=1, jitter=1, seed=5, box_lo=-1.5, box_hi=1.5)
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    v.nerf_render(dev(o), dev(d), dev(near), dev(far), w, cfg, rgb, depth, acc)
    ref = oren.render_hash(o, d, near, far, og, tabs, field, 128, seed=5, level_mask=np.asarray(mask))
    say(f"  rgb err {max_abs(host(rgb), ref['rgb']):.2e}")
    assert max_abs(host(rgb), ref["rgb"]) <= 1e-4
    assert max_abs(host(acc), ref["acc"]) <= 1e-4
    assert max_abs(host(depth), ref["depth"]) <= 1e-3

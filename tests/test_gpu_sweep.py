"""Pose sweeps and white backgrounds through the C ABI ("Spatial Intelligence
- Part 1: NeRF", Section 2 Code, 1. Overview: render_image and the video of a
pose sweep; 5. Volume rendering in code: white_bkgd), against the oracle."""
import ctypes

import numpy as np
import pytest

import seeded_inputs as si
from oracle import encoding as oenc
from oracle import rays as orays
from oracle import render as oren
from tests.gpu_util import dev, empty, host, max_abs, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu

RGB_TOL, ACC_TOL, DEPTH_TOL = 1e-4, 1e-4, 1e-3


@pytest.fixture(scope="module")
def v():
    torch_cuda()
    import volume_rendering_amd as v
    return v


def _sweep_setup(v, dtype=0):
    import volume_rendering_amd._binding as B
    pc, pf = si.nerf_params(si.NERF_4x64, seed=8, net_id=0), si.nerf_params(si.NERF_4x64, seed=8, net_id=1)
    nets = [v.weights.pack_to_device(2, dtype, pc), v.weights.pack_to_device(2, dtype, pf)]
    w = B.nerf_weights(net=B.nerf_mlp_desc(2, dtype), coarse=nets[0].data_ptr(), fine=nets[1].data_ptr())
    return pc, pf, nets, w


def test_pose_sweep_white_background(v):
    """Three frames of a 360 degree sweep, 24x20 pixels (ragged), 48 samples,
    float32 4x64 network, white background: every frame equals the oracle's
    render of that pose with the frame's ray counters."""
    import volume_rendering_amd._binding as B
    say("pose sweep, white background")
    torch = torch_cuda()
    W, H, f, n = 24, 20, 30.0, 3
    P = si.sweep_poses(n, elevation_deg=30.0)
    pc, pf, nets, w = _sweep_setup(v)
    cfg = B.nerf_render_cfg(mode=0, n_coarse=48, n_fine=0, use_pi=1, white_bkgd=1, jitter=1, seed=4, ray_offset=5)
    R = W * H
    rgb, depth, acc = empty((n, R, 3)), empty((n, R)), empty((n, R))
    v.nerf_render_poses(P, W, H, f, f, 0.5 * W, 0.5 * H, 2.0, 6.0, w, cfg, rgb, depth, acc)
    g_rgb, g_dep, g_acc = host(rgb), host(depth), host(acc)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    for k in range(n):
        o, d = orays.get_rays(H, W, f, f, 0.5 * W, 0.5 * H, P[k])
        ref = oren.render_nerf(o, d, near, far, pc, None, 48, 0, 6, 4, seed=4, white_bkgd=True, ray_offset=5 + k * R)
        say(f"  frame {k}: rgb err {max_abs(g_rgb[k], ref['rgb']):.2e}")
        assert max_abs(g_rgb[k], ref["rgb"]) <= RGB_TOL
        assert max_abs(g_acc[k], ref["acc"]) <= ACC_TOL
        assert max_abs(g_dep[k], ref["depth"]) <= DEPTH_TOL
    assert np.all(g_rgb >= 0.0) and np.all(g_rgb <= 1.0 + 1e-6)
    # a caller workspace gives the same frames; too small a one is refused
    ws = torch.empty(32 * R, dtype=torch.uint8, device="cuda")
    rgb2, depth2, acc2 = empty((n, R, 3)), empty((n, R)), empty((n, R))
    v.nerf_render_poses(P, W, H, f, f, 0.5 * W, 0.5 * H, 2.0, 6.0, w, cfg, rgb2, depth2, acc2, workspace=ws)
    assert np.array_equal(host(rgb2), g_rgb) and np.array_equal(host(acc2), g_acc)
    with pytest.raises(v.NerfError, match="NERF_ERR_WORKSPACE"):
        v.nerf_render_poses(P, W, H, f, f, 0.5 * W, 0.5 * H, 2.0, 6.0, w, cfg, rgb2, depth2, acc2,
                            workspace=ws[: 32 * R - 16])


@pytest.mark.parametrize("dtype", [0, 1])
def test_pose_sweep_hierarchical_equals_single_renders(v, dtype):
    """A hierarchical sweep (32 + 64 samples) is, frame for frame and bit for
    bit, nerf_render of that pose's rays with the frame's ray offset."""
    import volume_rendering_amd._binding as B
    say(f"hierarchical pose sweep dtype={dtype}")
    W, H, f, n = 17, 13, 20.0, 4
    P = si.sweep_poses(n, elevation_deg=20.0, radius=3.5)
    _, _, nets, w = _sweep_setup(v, dtype)
    cfg = B.nerf_render_cfg(mode=0, n_coarse=32, n_fine=64, use_pi=1, white_bkgd=1, jitter=1, seed=11, ray_offset=3)
    R = W * H
    rgb, depth, acc = empty((n, R, 3)), empty((n, R)), empty((n, R))
    v.nerf_render_poses(P, W, H, f, f, 0.5 * W, 0.5 * H, 2.0, 6.0, w, cfg, rgb, depth, acc)
    torch = torch_cuda()
    near, far = torch.full((R,), 2.0, device="cuda"), torch.full((R,), 6.0, device="cuda")
    for k in range(n):
        ro, rd = empty((R, 3)), empty((R, 3))
        v.nerf_gen_rays(P[k], W, H, f, f, 0.5 * W, 0.5 * H, ro, rd)
        c = B.nerf_render_cfg(mode=0, n_coarse=32, n_fine=64, use_pi=1, white_bkgd=1, jitter=1, seed=11,
                              ray_offset=3 + k * R)
        r1, d1, a1 = empty((R, 3)), empty(R), empty(R)
        v.nerf_render(ro, rd, near, far, w, c, r1, d1, a1)
        assert np.array_equal(host(rgb)[k], host(r1)) and np.array_equal(host(acc)[k], host(a1))
        assert np.array_equal(host(depth)[k], host(d1))


def test_hash_render_white_background(v):
    import volume_rendering_amd._binding as B
    say("hash render, white background")
    og = oenc.hashgrid_3d()
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    tabs = si.hash_tables(og.sizes, seed=1, scale=1.0)
    tdev = dev(np.concatenate(tabs, 0))
    g.tables = tdev.data_ptr()
    o, d = page_rays(256, 256, 355.2, si.poses(1, seed=6)[0])
    sel = si.subset(256 * 256, 200, seed=16)
    o, d = o[sel], d[sel]
    R = len(sel)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    field = si.hash_field_params(seed=2)
    net = v.weights.pack_to_device(4, 0, field)
    w = B.nerf_weights(net=B.nerf_mlp_desc(4, 0), coarse=net.data_ptr())
    w.grid = ctypes.pointer(g)
    cfg = B.nerf_render_cfg(mode=1, n_coarse=128, use_pi=1, white_bkgd=1, jitter=1, seed=2, box_lo=-1.5, box_hi=1.5)
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    v.nerf_render(dev(o), dev(d), dev(near), dev(far), w, cfg, rgb, depth, acc)
    ref = oren.render_hash(o, d, near, far, og, tabs, field, 128, seed=2, white_bkgd=True)
    say(f"  rgb err {max_abs(host(rgb), ref['rgb']):.2e}")
    assert max_abs(host(rgb), ref["rgb"]) <= RGB_TOL
    assert max_abs(host(acc), ref["acc"]) <= ACC_TOL
    assert max_abs(host(depth), ref["depth"]) <= DEPTH_TOL


def test_kilo_render_white_background(v):
    import volume_rendering_amd._binding as B
    say("many-network render, white background")
    torch = torch_cuda()
    stacked = si.cell_params_stacked(4096, seed=0)
    cells = [si.cell_slice(stacked, c) for c in range(4096)]
    cdev = v.weights.pack_many_to_device(3, 0, cells)
    bits = si.occupancy_bits(128, 0.1, seed=0)
    odev = dev(bits.view(np.int32))
    o, d = page_rays(800, 800, 1110.0, si.poses(1, seed=0)[0])
    sel = si.subset(800 * 800, 300, seed=17)
    o, d = o[sel], d[sel]
    R = len(sel)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    cfg = B.nerf_render_cfg(mode=2, n_coarse=192, use_pi=1, white_bkgd=1, jitter=1, seed=0, term_T=1e-2,
                            box_lo=-1.5, box_hi=1.5, occ_res=128, cell_res=16, occ=odev.data_ptr())
    w = B.nerf_weights(net=B.nerf_mlp_desc(3, 0), cells=cdev.data_ptr(), n_cells=4096)
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    v.nerf_render(dev(o), dev(d), dev(near), dev(far), w, cfg, rgb, depth, acc)
    ref = oren.render_kilo(o, d, near, far, si.occupancy_dense(bits), lambda c: cells[c], 192, seed=0,
                           term_T=1e-2, white_bkgd=True)
    say(f"  rgb err {max_abs(host(rgb), ref['rgb']):.2e}")
    assert max_abs(host(rgb), ref["rgb"]) <= RGB_TOL
    assert max_abs(host(acc), ref["acc"]) <= ACC_TOL
    assert np.all(host(rgb) >= 1.0 - host(acc)[:, None] - 1e-6)

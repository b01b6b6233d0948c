"""Empty-space skipping and early termination in the NeRF and hash-grid
renders ("Spatial Intelligence - Part 1: NeRF", Section 1 Theory, 4.2:
uniform samples waste compute on empty space), through the C ABI against the
oracle.  Rays whose transmittance comes within 1e-5 (relative) of the
threshold may stop one sample apart and are left out of the colour checks."""
import ctypes

import numpy as np
import pytest

import seeded_inputs as si
from oracle import encoding as oenc
from oracle import render as oren
from oracle import sampling as osamp
from tests.gpu_util import bf16_render_check, dev, empty, host, max_abs, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu

RGB_TOL, ACC_TOL, DEPTH_TOL = 1e-4, 1e-4, 1e-3


@pytest.fixture(scope="module")
def v():
    torch_cuda()
    import volume_rendering_amd as v
    return v


def _near_threshold(w, term_T):
    """Rays with a transmittance (before some sample) within 1e-5 of term_T."""
    T = 1.0 - np.concatenate([np.zeros((w.shape[0], 1)), np.cumsum(w, 1)[:, :-1]], 1)
    return np.any(np.abs(T / term_T - 1.0) < 1e-5, axis=1)


def _dense(params, shift):
    return dict(params, sigma=(params["sigma"][0], params["sigma"][1] + np.float32(shift)))


def _render(v, mode, kind, dtype, o, d, nets, nc, nf, occ_bits, occ_res, term_T, seed=0, white=False, grid=None,
            box=(-1.5, 1.5)):
    import volume_rendering_amd._binding as B
    torch = torch_cuda()
    R = o.shape[0]
    occ = dev(occ_bits.view(np.int32)) if occ_bits is not None else None
    nlive = torch.zeros(1, dtype=torch.int64, device="cuda")
    cfg = B.nerf_render_cfg(mode=mode, n_coarse=nc, n_fine=nf, use_pi=1, white_bkgd=int(white), jitter=1, seed=seed,
                            term_T=term_T, box_lo=box[0], box_hi=box[1], occ_res=occ_res,
                            occ=occ.data_ptr() if occ is not None else None, dbg_n_live=nlive.data_ptr())
    dz, dw = empty((R, nc + nf)), empty((R, nc))
    cfg.dbg_z, cfg.dbg_w_coarse = dz.data_ptr(), dw.data_ptr()
    w = B.nerf_weights(net=B.nerf_mlp_desc(kind, dtype), coarse=nets[0].data_ptr(),
                       fine=nets[1].data_ptr() if len(nets) > 1 else None)
    if grid is not None:
        w.grid = ctypes.pointer(grid)
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    v.nerf_render(dev(o), dev(d), dev(near), dev(far), w, cfg, rgb, depth, acc)
    return host(rgb), host(depth), host(acc), host(dz), host(dw), int(host(nlive)[0]), near, far


def test_full_occupancy_equals_no_skipping(v):
    """Every sample live (full grid, a box holding them all), no termination:
    the same outputs, bit for bit, as the render without a grid."""
    say("skipping: full occupancy")
    pose = si.poses(1, seed=3)[0]
    o, d = page_rays(24, 24, 30.0, pose)
    pc, pf = si.nerf_params(si.NERF_4x64, seed=5, net_id=0), si.nerf_params(si.NERF_4x64, seed=5, net_id=1)
    for dtype in (0, 1):
        nets = [v.weights.pack_to_device(2, dtype, pc), v.weights.pack_to_device(2, dtype, pf)]
        a = _render(v, 0, 2, dtype, o, d, nets, 64, 128, None, 1, 0.0, seed=9)
        b = _render(v, 0, 2, dtype, o, d, nets, 64, 128, si.occupancy_bits(8, 1.0, seed=0), 8, 0.0, seed=9,
                    box=(-100.0, 100.0))
        for x, y in zip(a[:5], b[:5]):
            assert np.array_equal(x, y)
        assert b[5] == 576 * (64 + 192)


@pytest.mark.parametrize("term_T", [0.0, 1e-2])
def test_nerf_skipping_hierarchical_stage_isolated(v, term_T):
    """32^3 occupancy at 50%, 64 + 128 samples, float32 4x64 networks with a
    dense field (density bias +8): coarse weights and the live count against
    the oracle, resampling bit-exact from the GPU's own coarse weights, fine
    colour from the GPU's merged samples."""
    say(f"skipping: hierarchical, term_T={term_T}")
    pose = si.poses(1, seed=7)[0]
    o, d = page_rays(24, 20, 30.0, pose)
    pc = _dense(si.nerf_params(si.NERF_4x64, seed=6, net_id=0), 8.0)
    pf = _dense(si.nerf_params(si.NERF_4x64, seed=6, net_id=1), 8.0)
    nets = [v.weights.pack_to_device(2, 0, pc), v.weights.pack_to_device(2, 0, pf)]
    bits = si.occupancy_bits(32, 0.5, seed=2)
    occ = si.occupancy_dense(bits, 32)
    rgb, depth, acc, dz, dw, n_live, near, far = _render(v, 0, 2, 0, o, d, nets, 64, 128, bits, 32, term_T, seed=4)
    ref_c = oren.render_nerf(o, d, near, far, pc, None, 64, 0, 6, 4, seed=4, occ=occ, occ_res=32, term_T=term_T)
    keep = ~_near_threshold(ref_c["coarse"]["w"], term_T) if term_T else np.ones(len(o), bool)
    assert max_abs(dw[keep], ref_c["coarse"]["w"][keep]) <= 1e-5
    _, _, z2 = osamp.hierarchical_fine_samples(ref_c["z_c"], dw, 128, 4)
    assert np.array_equal(dz, z2)
    fine = oren.nerf_pass(pf, o, d, dz, 6, 4, occ=occ, occ_res=32, term_T=term_T)
    assert n_live == ref_c["n_live"] + fine["n_live"]
    if term_T:
        keep &= ~_near_threshold(fine["w"], term_T)
        T_end = 1.0 - np.sum(fine["w"], 1)
        n_stop = int(np.sum(T_end < term_T))
        say(f"  live samples {n_live}; rays that stop early: {n_stop} of {len(o)}")
        assert n_stop > 0.3 * len(o)
    say(f"  rgb err {max_abs(rgb[keep], fine['rgb'][keep]):.2e} ({int(keep.sum())} rays)")
    assert keep.mean() > 0.9
    assert max_abs(rgb[keep], fine["rgb"][keep]) <= RGB_TOL
    assert max_abs(acc[keep], fine["acc"][keep]) <= ACC_TOL
    assert max_abs(depth[keep], fine["depth"][keep]) <= DEPTH_TOL


def test_nerf_skipping_empty_grid(v):
    say("skipping: empty grid")
    o, d = page_rays(16, 16, 20.0, si.poses(1, seed=1)[0])
    p = si.nerf_params(si.NERF_4x64, seed=1)
    nets = [v.weights.pack_to_device(2, 1, p), v.weights.pack_to_device(2, 1, p)]
    rgb, depth, acc, _, _, n_live, _, _ = _render(v, 0, 2, 1, o, d, nets, 32, 64, si.occupancy_bits(16, 0.0),
                                                   16, 1e-2, white=True)
    assert n_live == 0 and np.all(acc == 0) and np.all(depth == 0) and np.all(rgb == 1.0)


def test_hash_skipping(v):
    """Hash field, 64^3 occupancy at 40%, stop at T < 1e-2, float32."""
    say("skipping: hash field")
    og = oenc.hashgrid_3d()
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    tabs = si.hash_tables(og.sizes, seed=3, scale=1.0)
    tdev = dev(np.concatenate(tabs, 0))
    g.tables = tdev.data_ptr()
    o, d = page_rays(256, 256, 355.2, si.poses(1, seed=5)[0])
    sel = si.subset(256 * 256, 300, seed=19)
    o, d = o[sel], d[sel]
    field = si.hash_field_params(seed=4)
    field = dict(field, sigma=(field["sigma"][0], field["sigma"][1] + np.float32(4.0)))
    net = v.weights.pack_to_device(4, 0, field)
    bits = si.occupancy_bits(64, 0.4, seed=4)
    occ = si.occupancy_dense(bits, 64)
    rgb, depth, acc, dz, _, n_live, near, far = _render(v, 1, 4, 0, o, d, [net], 128, 0, bits, 64, 1e-2, seed=6,
                                                         grid=g)
    ref = oren.render_hash(o, d, near, far, og, tabs, field, 128, seed=6, occ=occ, occ_res=64, term_T=1e-2)
    assert np.array_equal(dz, ref["z"]) and n_live == ref["n_live"]
    n_stop = int(np.sum(1.0 - np.sum(ref["w"], 1) < 1e-2))
    say(f"  rays that stop early: {n_stop} of {len(o)}")
    assert n_stop > 0.2 * len(o)
    keep = ~_near_threshold(ref["w"], 1e-2)
    say(f"  live {n_live}, rgb err {max_abs(rgb[keep], ref['rgb'][keep]):.2e} ({int(keep.sum())} rays)")
    assert keep.mean() > 0.9
    assert max_abs(rgb[keep], ref["rgb"][keep]) <= RGB_TOL
    assert max_abs(acc[keep], ref["acc"][keep]) <= ACC_TOL
    assert max_abs(depth[keep], ref["depth"][keep]) <= DEPTH_TOL


def test_nerf_skipping_8x256_bf16(v):
    """800x800 camera, 8x256 bfloat16 networks, 128^3 occupancy at 10%, 64 +
    128 samples, no termination: live count exact; resampling bit-exact from
    the GPU's coarse weights; fine colour against the float64 definition on
    every ray."""
    say("skipping: 8x256 bf16 hierarchical")
    o, d = page_rays(800, 800, 1110.0, si.poses(4, seed=0)[1])
    sel = si.subset(800 * 800, 400, seed=20)
    o, d = o[sel], d[sel]
    pc, pf = si.nerf_params(si.NERF_8x256, seed=0, net_id=0), si.nerf_params(si.NERF_8x256, seed=0, net_id=1)
    nets = [v.weights.pack_to_device(1, 1, pc), v.weights.pack_to_device(1, 1, pf)]
    bits = si.occupancy_bits(128, 0.1, seed=0)
    occ = si.occupancy_dense(bits)
    rgb, depth, acc, dz, dw, n_live, near, far = _render(v, 0, 1, 1, o, d, nets, 64, 128, bits, 128, 0.0, seed=0)
    ref_c = oren.render_nerf(o, d, near, far, pc, None, 64, 0, 10, 4, seed=0, mode="bf16", occ=occ)
    assert max_abs(dw, ref_c["coarse"]["w"]) <= 2e-2
    _, _, z2 = osamp.hierarchical_fine_samples(ref_c["z_c"], dw, 128, 0)
    assert np.array_equal(dz, z2)
    fine = oren.nerf_pass(pf, o, d, dz, 10, 4, "f64", occ=occ)
    emu = oren.nerf_pass(pf, o, d, dz, 10, 4, "bf16", occ=occ)
    assert n_live == ref_c["n_live"] + fine["n_live"]
    say(f"  live samples {n_live} of {len(o) * 256}")
    bf16_render_check("fine pass", rgb, depth, acc, fine["raw"], emu["raw"], dz, d)

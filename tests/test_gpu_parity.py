"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs.  Bars: bit-exact for rays, samples, bins and indices; for
float32 networks rgb/acc within 1e-4 and depth within 1e-3; for bfloat16
networks rgb and acc within 2e-2 of the float64 definition on every ray
(``bf16_render_check``)."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import composite as ocomp
from oracle import encoding as oenc
from oracle import mlp as omlp
from oracle import render as oren
from oracle import sampling as osamp
from tests.gpu_util import bf16_render_check, dev, empty, gpu_rays, host, max_abs, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu

RGB_TOL, ACC_TOL, DEPTH_TOL = 1e-4, 1e-4, 1e-3


@pytest.fixture(scope="module")
def v():
    torch_cuda()
    import volume_rendering_amd as v
    return v


def _near_far(R, near=2.0, far=6.0):
    return np.full(R, near, np.float32), np.full(R, far, np.float32)


# ----------------------------------------------------------------------------
# Rays and samples: bit-exact
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("H,W,f,hemi", [(32, 32, 40.0, False), (400, 400, 555.0, True), (37, 53, 71.5, True)])
def test_gen_rays_bit_exact(v, H, W, f, hemi):
    say(f"gen_rays {H}x{W} f={f}")
    pose = si.poses(1, seed=0, hemisphere=hemi)[0]
    ro, rd = gpu_rays(H, W, f, pose)
    o, d = page_rays(H, W, f, pose)
    assert np.array_equal(host(ro), o) and np.array_equal(host(rd), d)


@pytest.mark.parametrize("n,jitter,offset", [(16, True, 0), (64, True, 12345), (192, False, 0), (1, True, 7),
                                             (64, True, 2 ** 32 - 500), (16, True, 2 ** 40 + 3)])
def test_stratified_bit_exact(v, n, jitter, offset):
    say(f"stratified n={n} jitter={jitter}")
    R = 1000
    near, far = _near_far(R)
    far[::3] = 4.5
    z = empty((R, n))
    v.nerf_sample_stratified(dev(near), dev(far), n, 42, offset, jitter, z)
    assert np.array_equal(host(z), osamp.stratified(near, far, n, 42, jitter, offset))


# ----------------------------------------------------------------------------
# Encoders
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L,use_pi", [(10, True), (4, True), (6, False)])
def test_encode_freq(v, L, use_pi):
    say(f"encode_freq L={L} pi={use_pi}")
    g = np.random.default_rng(1)
    x = g.uniform(-6, 6, size=(5003, 3)).astype(np.float32)
    out = empty((5003, 3 + 6 * L))
    v.nerf_encode_freq(dev(x), L, True, use_pi, 0, out)
    ref = oenc.freq_encode(x, L, True, use_pi)
    tol = 2.4e-7 if use_pi else 5e-7
    assert max_abs(host(out), ref) <= tol
    torch = torch_cuda()
    ob = empty((5003, 3 + 6 * L), torch.bfloat16)
    v.nerf_encode_freq(dev(x), L, True, use_pi, 1, ob)
    hb = host(ob.float())
    # bf16 output is the float32 value rounded to nearest even: within half a bf16 ulp of the exact value
    assert np.all(np.abs(hb - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)
    # an output that is not 16-byte aligned takes the scalar stores: same values
    big = empty(5003 * (3 + 6 * L) + 1)
    om = big[1:].view(5003, 3 + 6 * L)
    v.nerf_encode_freq(dev(x), L, True, use_pi, 0, om)
    assert np.array_equal(host(om), host(out))


def test_encode_sh16(v):
    g = np.random.default_rng(2)
    d = g.normal(size=(4000, 3)).astype(np.float32)
    out = empty((4000, 16))
    v.nerf_encode_sh16(dev(d), out)
    assert max_abs(host(out), oenc.sh16(osamp.view_dirs(d))) <= 2e-6


@pytest.mark.parametrize("scale", [1.0, 1e-4])
def test_encode_hashgrid(v, scale):
    say(f"hashgrid scale={scale}")
    torch = torch_cuda()
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    og = oenc.hashgrid_3d()
    tabs = si.hash_tables(og.sizes, seed=0, scale=scale)
    flat = np.concatenate(tabs, axis=0)
    tdev = dev(flat)
    g.tables = tdev.data_ptr()
    x = si.query_points(3001, seed=4)
    x[:5] = [[0, 0, 0], [1, 1, 1], [0.5, 0.5, 0.5], [1.2, -0.1, 0.3], [1e-7, 0.9999999, 0.25]]
    out = empty((3001, 32))
    idx = torch.empty((3001, 16, 8), dtype=torch.int32, device="cuda")
    v.nerf_encode_hashgrid(dev(x), g, out, idx)
    hidx = host(idx).view(np.uint32)
    for l in range(16):
        ref_idx, _ = og.level_indices(x, l)
        assert np.array_equal(hidx[:, l, :].astype(np.int64), ref_idx), l
    ref = og.encode(x, tabs)
    assert max_abs(host(out), ref) <= 1e-6 * scale * 8


# ----------------------------------------------------------------------------
# Networks
# ----------------------------------------------------------------------------

NETS = {
    1: (si.NERF_8x256, 10, 4),
    2: (si.NERF_4x64, 6, 4),
    3: (si.NERF_CELL_2x32, 10, 4),
}


@pytest.mark.parametrize("kind", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", [0, 1])
def test_mlp_standalone(v, kind, dtype):
    say(f"mlp kind={kind} dtype={dtype}")
    g = np.random.default_rng(kind * 10 + dtype)
    S, spr = 997, 50  # ragged: 997 samples leave a partial last wave
    if kind == 4:
        params = si.hash_field_params(seed=1)
        ex = g.uniform(-1, 1, size=(S, 32)).astype(np.float32)
        ev = oenc.sh16(osamp.view_dirs(g.normal(size=((S + spr - 1) // spr, 3)))).astype(np.float32)
    else:
        shape, Lp, Ld = NETS[kind]
        params = si.nerf_params(shape, seed=1)
        ex = oenc.freq_encode(g.uniform(-2, 2, size=(S, 3)).astype(np.float32), Lp).astype(np.float32)
        ev = oenc.freq_encode(osamp.view_dirs(g.normal(size=((S + spr - 1) // spr, 3))).astype(np.float32),
                              Ld).astype(np.float32)
    packed = v.weights.pack_to_device(kind, dtype, params)
    raw = empty((S, 4))
    v.nerf_mlp(kind, dtype, packed, dev(ex), dev(ev), spr, raw)
    evs = np.repeat(ev, spr, axis=0)[:S]
    fwd = omlp.hash_field_forward if kind == 4 else omlp.nerf_forward
    ref = fwd(params, ex, evs, "f64")
    got = host(raw)
    scale = max(1.0, float(np.abs(ref).max()))
    if dtype == 0:
        assert max_abs(got, ref) <= 1e-5 * scale
    else:
        emu = fwd(params, ex, evs, "bf16")
        say(f"  bf16: vs emulation {max_abs(got, emu):.3e}, vs f64 {max_abs(got, ref):.3e}, scale {scale:.2f}")
        assert max_abs(got, emu) <= 2e-2 * scale
        assert max_abs(got, ref) <= 6e-2 * scale


# ----------------------------------------------------------------------------
# Compositing and resampling
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,white", [(64, False), (192, True), (16, False), (100, False), (1, False), (3, True),
                                     (257, False)])
def test_composite(v, N, white):
    say(f"composite N={N}")
    R = 777
    g = np.random.default_rng(N)
    near, far = _near_far(R)
    z = osamp.stratified(near, far, N, 3)
    raw = (g.normal(size=(R, N, 4)) * 2).astype(np.float32)
    pose = si.poses(1, seed=1)[0]
    _, d = page_rays(1, R, 300.0, pose)
    rgb, depth, acc, w = empty((R, 3)), empty(R), empty(R), empty((R, N))
    v.nerf_composite(dev(raw), dev(z), dev(d), white, rgb, depth, acc, w)
    rr, rd_, ra, rw = ocomp.volume_render(raw, z, d, white)
    assert max_abs(host(rgb), rr) <= RGB_TOL
    assert max_abs(host(acc), ra) <= ACC_TOL
    assert max_abs(host(depth), rd_) <= DEPTH_TOL
    assert max_abs(host(w), rw) <= 1e-5
    # without the weights output the other outputs are unchanged
    rgb2, depth2, acc2 = empty((R, 3)), empty(R), empty(R)
    v.nerf_composite(dev(raw), dev(z), dev(d), white, rgb2, depth2, acc2)
    assert np.array_equal(host(rgb2), host(rgb)) and np.array_equal(host(acc2), host(acc))


@pytest.mark.parametrize("nc,nf", [(64, 128), (16, 32), (130, 126), (3, 1), (64, 192)])
def test_sample_pdf_bit_exact(v, nc, nf):
    say(f"sample_pdf nc={nc} nf={nf}")
    torch = torch_cuda()
    R = 513
    g = np.random.default_rng(nc)
    near, far = _near_far(R)
    zc = osamp.stratified(near, far, nc, 5, True, 1000)
    _, d = page_rays(1, R, 300.0, si.poses(1, seed=2)[0])
    raw = (g.normal(size=(R, nc, 4)) * 3).astype(np.float32)
    w = ocomp.volume_render(raw, zc, d)[3].astype(np.float32)
    w[:10] = 0.0  # all-empty rays: uniform pdf
    w[10:20, :] = 0.0
    w[10:20, nc // 2] = 1.0  # spikes
    zf, bins, z2 = empty((R, nf)), torch.empty((R, nf), dtype=torch.int32, device="cuda"), empty((R, nc + nf))
    v.nerf_sample_pdf(dev(zc), dev(w), nf, 11, 1000, zf, bins, z2)
    rzf, ridx, rz2 = osamp.hierarchical_fine_samples(zc, w, nf, 11, 1000)
    assert np.array_equal(host(bins), ridx)
    assert np.array_equal(host(zf), rzf)
    assert np.array_equal(host(z2), rz2)


def test_sample_pdf_unordered_coarse(v):
    """Coarse samples given in descending or shuffled order (the merged output
    is still the ascending union): exercises the merge's sorting of the first
    set, which stratified samples never need."""
    say("sample_pdf with unordered coarse samples")
    R, nc, nf = 200, 64, 128
    g = np.random.default_rng(7)
    near, far = _near_far(R)
    zc = osamp.stratified(near, far, nc, 5, True, 0)
    zc[0::3] = zc[0::3, ::-1]
    for i in range(1, R, 3):
        zc[i] = zc[i, g.permutation(nc)]
    w = g.random((R, nc)).astype(np.float32)
    zf, bins, z2 = empty((R, nf)), torch_cuda().empty((R, nf), dtype=torch_cuda().int32, device="cuda"), empty((R, nc + nf))
    v.nerf_sample_pdf(dev(zc), dev(w), nf, 3, 0, zf, bins, z2)
    rzf, ridx, rz2 = osamp.hierarchical_fine_samples(zc, w, nf, 3, 0)
    assert np.array_equal(host(zf), rzf)
    assert np.array_equal(host(z2), rz2)


# ----------------------------------------------------------------------------
# Fused renders
# ----------------------------------------------------------------------------

def _render(v, mode, kind, dtype, ro, rd, near, far, nets, nc, nf=0, seed=0, jitter=True, chunk=0, grid=None,
            white=False, use_pi=True, ray_offset=0):
    import volume_rendering_amd._binding as B
    R = ro.shape[0]
    cfg = B.nerf_render_cfg(mode=mode, n_coarse=nc, n_fine=nf, use_pi=int(use_pi), white_bkgd=int(white),
                            jitter=int(jitter), seed=seed, ray_offset=ray_offset, chunk=chunk, box_lo=-1.5, box_hi=1.5)
    dz, dw = empty((R, nc + nf)), empty((R, nc))
    cfg.dbg_z, cfg.dbg_w_coarse = dz.data_ptr(), dw.data_ptr()
    w = B.nerf_weights(net=B.nerf_mlp_desc(kind, dtype), coarse=nets[0].data_ptr(),
                       fine=nets[1].data_ptr() if len(nets) > 1 else None)
    if grid is not None:
        import ctypes
        w.grid = ctypes.pointer(grid)
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    v.nerf_render(ro, rd, dev(near), dev(far), w, cfg, rgb, depth, acc)
    return host(rgb), host(depth), host(acc), host(dz), host(dw)


@pytest.mark.parametrize("use_pi,ray_offset", [(True, 0), (False, 0), (True, 2 ** 32 - 300)])
def test_render_tiny_coarse_fp32(v, use_pi, ray_offset):
    """32x32 rays, focal 40, a sphere pose; 16 jittered samples; PE 6/4;
    float32 4x64 network; both encodings, and ray counters that cross 2^32
    inside the image."""
    say(f"render tiny use_pi={use_pi} ray_offset={ray_offset}")
    pose = si.poses(1, seed=0, hemisphere=False)[0]
    ro, rd = gpu_rays(32, 32, 40.0, pose)
    o, d = page_rays(32, 32, 40.0, pose)
    near, far = _near_far(1024)
    params = si.nerf_params(si.NERF_4x64, seed=0)
    net = v.weights.pack_to_device(2, 0, params)
    rgb, depth, acc, dz, dw = _render(v, 0, 2, 0, ro, rd, near, far, [net], 16, use_pi=use_pi, ray_offset=ray_offset)
    ref = oren.render_nerf(o, d, near, far, params, None, 16, 0, 6, 4, seed=0, use_pi=use_pi, ray_offset=ray_offset)
    assert np.array_equal(dz, ref["z_c"])
    assert max_abs(rgb, ref["rgb"]) <= RGB_TOL
    assert max_abs(acc, ref["acc"]) <= ACC_TOL
    assert max_abs(depth, ref["depth"]) <= DEPTH_TOL
    assert max_abs(dw, ref["coarse"]["w"]) <= 1e-5


@pytest.mark.parametrize("dtype,white", [(0, False), (1, False), (0, True)])
def test_render_hierarchical_stage_isolated(v, dtype, white):
    """Coarse 64 + fine 128 with 4x64 networks: coarse weights against the
    oracle, bins and merged samples bit-exact from the GPU's own coarse
    weights, fine colour from the GPU's own merged samples (also on a white
    background)."""
    say(f"render hierarchical 4x64 dtype={dtype} white={white}")
    pose = si.poses(1, seed=3)[0]
    H = W = 24
    ro, rd = gpu_rays(H, W, 30.0, pose)
    o, d = page_rays(H, W, 30.0, pose)
    R = H * W
    near, far = _near_far(R)
    pc, pf = si.nerf_params(si.NERF_4x64, seed=5, net_id=0), si.nerf_params(si.NERF_4x64, seed=5, net_id=1)
    nets = [v.weights.pack_to_device(2, dtype, pc), v.weights.pack_to_device(2, dtype, pf)]
    rgb, depth, acc, dz, dw = _render(v, 0, 2, dtype, ro, rd, near, far, nets, 64, 128, seed=9, white=white)
    mode = "f64" if dtype == 0 else "bf16"
    ref_c = oren.render_nerf(o, d, near, far, pc, None, 64, 0, 6, 4, seed=9, mode=mode)
    assert max_abs(dw, ref_c["coarse"]["w"]) <= (1e-5 if dtype == 0 else 2e-2)
    _, _, z2 = osamp.hierarchical_fine_samples(ref_c["z_c"], dw, 128, 9)
    assert np.array_equal(dz, z2)
    fine = oren.nerf_pass(pf, o, d, dz, 6, 4, "f64", white_bkgd=white)
    if dtype == 0:
        assert max_abs(rgb, fine["rgb"]) <= RGB_TOL
        assert max_abs(acc, fine["acc"]) <= ACC_TOL
        assert max_abs(depth, fine["depth"]) <= DEPTH_TOL
    else:
        emu = oren.nerf_pass(pf, o, d, dz, 6, 4, "bf16")
        bf16_render_check("fine pass", rgb, depth, acc, fine["raw"], emu["raw"], dz, d)


def test_render_8x256_bf16_hierarchical(v):
    """800x800 camera (focal 1110), 8x256 coarse and fine networks in
    bfloat16, 64 + 128 samples; a ragged subset of rays."""
    say("render 8x256 bf16 hierarchical")
    pose = si.poses(4, seed=0)[2]
    o, d = page_rays(800, 800, 1110.0, pose)
    sel = si.subset(800 * 800, 150, seed=1)
    o, d = o[sel], d[sel]
    R = len(sel)
    near, far = _near_far(R)
    pc, pf = si.nerf_params(si.NERF_8x256, seed=0, net_id=0), si.nerf_params(si.NERF_8x256, seed=0, net_id=1)
    nets = [v.weights.pack_to_device(1, 1, pc), v.weights.pack_to_device(1, 1, pf)]
    rgb, depth, acc, dz, dw = _render(v, 0, 1, 1, dev(o), dev(d), near, far, nets, 64, 128, seed=0)
    ref_c = oren.render_nerf(o, d, near, far, pc, None, 64, 0, 10, 4, seed=0, mode="bf16")
    e_w = max_abs(dw, ref_c["coarse"]["w"])
    say(f"  coarse weights vs bf16 emulation: {e_w:.3e}")
    assert e_w <= 2e-2
    _, _, z2 = osamp.hierarchical_fine_samples(ref_c["z_c"], dw, 128, 0)
    assert np.array_equal(dz, z2)
    # end to end (the oracle's own coarse weights): rays whose resampled depths differ
    _, _, z2_e2e = osamp.hierarchical_fine_samples(ref_c["z_c"], ref_c["coarse"]["w"].astype(np.float32), 128, 0)
    say(f"  end-to-end resampling: {100 * np.mean(np.any(z2_e2e != dz, axis=1)):.1f}% of rays differ in a bin")
    fine = oren.nerf_pass(pf, o, d, dz, 10, 4, "f64")
    emu = oren.nerf_pass(pf, o, d, dz, 10, 4, "bf16")
    bf16_render_check("fine pass", rgb, depth, acc, fine["raw"], emu["raw"], dz, d)


def test_render_8x256_fp32_coarse(v):
    """400x400 camera (focal 555), 64 samples, float32 8x256 network."""
    say("render 8x256 fp32 coarse")
    pose = si.poses(8, seed=0)[5]
    o, d = page_rays(400, 400, 555.0, pose)
    sel = si.subset(400 * 400, 70, seed=2)
    o, d = o[sel], d[sel]
    near, far = _near_far(len(sel))
    pc = si.nerf_params(si.NERF_8x256, seed=0, net_id=0)
    net = v.weights.pack_to_device(1, 0, pc)
    rgb, depth, acc, dz, _ = _render(v, 0, 1, 0, dev(o), dev(d), near, far, [net], 64, seed=0)
    ref = oren.render_nerf(o, d, near, far, pc, None, 64, 0, 10, 4, seed=0)
    assert np.array_equal(dz[:, :64], ref["z_c"])
    assert max_abs(rgb, ref["rgb"]) <= RGB_TOL
    assert max_abs(acc, ref["acc"]) <= ACC_TOL
    assert max_abs(depth, ref["depth"]) <= DEPTH_TOL


@pytest.mark.parametrize("scale,dtype", [(1.0, 0), (1e-4, 0), (1.0, 1)])
def test_render_hash(v, scale, dtype):
    """256x256 camera (focal 355.2), 128 samples, scene box [-1.5,1.5]^3
    mapped to the unit cube, 16-level grid, hash-field network."""
    say(f"render hash scale={scale} dtype={dtype}")
    og = oenc.hashgrid_3d()
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    tabs = si.hash_tables(og.sizes, seed=0, scale=scale)
    tdev = dev(np.concatenate(tabs, 0))
    g.tables = tdev.data_ptr()
    pose = si.poses(1, seed=4)[0]
    o, d = page_rays(256, 256, 355.2, pose)
    sel = si.subset(256 * 256, 100, seed=3)
    o, d = o[sel], d[sel]
    near, far = _near_far(len(sel))
    field = si.hash_field_params(seed=0)
    net = v.weights.pack_to_device(4, dtype, field)
    rgb, depth, acc, dz, _ = _render(v, 1, 4, dtype, dev(o), dev(d), near, far, [net], 128, seed=0, grid=g)
    ref = oren.render_hash(o, d, near, far, og, tabs, field, 128, seed=0)
    assert np.array_equal(dz[:, :128], ref["z"])
    say(f"  rgb err {max_abs(rgb, ref['rgb']):.3e}")
    if dtype == 0:
        assert max_abs(rgb, ref["rgb"]) <= RGB_TOL
        assert max_abs(acc, ref["acc"]) <= ACC_TOL
        assert max_abs(depth, ref["depth"]) <= DEPTH_TOL
    else:
        emu = oren.render_hash(o, d, near, far, og, tabs, field, 128, seed=0, mode="bf16")
        bf16_render_check("hash field", rgb, depth, acc, ref["raw"], emu["raw"], ref["z"], d)


def test_render_chunk_invariance_and_determinism(v):
    say("chunk invariance")
    pose = si.poses(1, seed=3)[0]
    ro, rd = gpu_rays(20, 20, 25.0, pose)
    near, far = _near_far(400)
    pc, pf = si.nerf_params(si.NERF_4x64, seed=5, net_id=0), si.nerf_params(si.NERF_4x64, seed=5, net_id=1)
    nets = [v.weights.pack_to_device(2, 1, pc), v.weights.pack_to_device(2, 1, pf)]
    a = _render(v, 0, 2, 1, ro, rd, near, far, nets, 64, 128, seed=3)
    b = _render(v, 0, 2, 1, ro, rd, near, far, nets, 64, 128, seed=3, chunk=37)
    c = _render(v, 0, 2, 1, ro, rd, near, far, nets, 64, 128, seed=3)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


@pytest.mark.parametrize("use_pi", [True, False])
def test_fused_encoding_accuracy(v, use_pi):
    """The frequency encoding computed inside the fused render, measured
    directly.  One sample per ray (its interval is 1e10 |d| long, so its
    weight is exactly 1 and rgb = sigmoid(rgb_raw)) and a float32 4x64
    network that carries three encoding columns unchanged to rgb_raw
    (unit weights, a +2 bias that keeps them through the ReLUs, and -2 in the
    rgb head: the only rounding is of gamma + 2, at most 1.2e-7).  gamma is
    recovered from rgb by the logit and compared with the encoding of the
    same points in float64."""
    say(f"fused encoding accuracy use_pi={use_pi}")
    from oracle import encoding as oenc
    from oracle import sampling as osamp2
    shape = si.NERF_4x64
    W, D, DW = shape.width, shape.depth, shape.dir_width
    cols = [3 + 6 * 5 + 0, 3 + 6 * 5 + 3 + 1, 3 + 6 * 2 + 2]  # sin(2^5 pi x), cos(2^5 pi y), sin(4 pi z)
    z32 = lambda *s: np.zeros(s, np.float32)
    layers = []
    for l in range(D):
        Wl = z32(W, shape.pos_ch if l == 0 else W)
        bl = z32(W)
        for k, c in enumerate(cols):
            Wl[k, c if l == 0 else k] = 1.0
        if l == 0:
            bl[:3] = 2.0
        layers.append((Wl, bl))
    feat = (z32(W, W), z32(W))
    dirl = (z32(DW, W + shape.dir_ch), z32(DW))
    rgbl = (z32(3, DW), np.full(3, -2.0, np.float32))
    for k in range(3):
        feat[0][k, k] = 1.0
        dirl[0][k, k] = 1.0
        rgbl[0][k, k] = 1.0
    params = {"shape": shape, "layers": layers, "sigma": (z32(1, W), np.full(1, 10.0, np.float32)), "feature": feat,
              "dir": dirl, "rgb": rgbl}
    net = v.weights.pack_to_device(2, 0, params)
    H = Wd = 64
    pose = si.poses(1, seed=5)[0]
    ro, rd = gpu_rays(H, Wd, 60.0, pose)
    o, d = page_rays(H, Wd, 60.0, pose)
    near, far = _near_far(H * Wd, 1.0, 7.0)
    rgb, _, acc, dz, _ = _render(v, 0, 2, 0, ro, rd, near, far, [net], 1, seed=9, use_pi=use_pi)
    assert np.all(acc == 1.0)
    x = osamp2.points(o, d, dz)  # the render's own sample depths (bit-exact with the oracle's)
    gamma = oenc.freq_encode(x.reshape(-1, 3), 6, True, use_pi)[:, cols]
    p = rgb.astype(np.float64)
    got = np.log(p / (1.0 - p))
    err = np.abs(got - gamma)
    say(f"  max |gamma error| {err.max():.2e} (p99.9 {np.quantile(err, 0.999):.2e}) over {err.size} values")
    # the route itself (gamma + 2 in float32, a float32 sigmoid, the logit)
    # is good to about 4e-7, which the library sincosf (use_pi=0) shows
    assert err.max() <= 1e-6

"""The training step of a NeRF-family network on the GPU (through the C ABI)
against the oracle (``oracle.backward``) on the same seeded inputs.

Bars.  Float32 networks: loss within 1e-5 relative and rendered rgb within
1e-4 absolute of the float64 definition; each parameter tensor's gradient
within ``GRAD_TOL_F32`` of that tensor's largest gradient (float32
accumulation over at most 319 products per layer and over every sample of
the batch, through the 12 layers of the 8x256 network, plus the rare ReLU
whose pre-activation lies within float32 rounding of 0 and so may take the
other branch).  Bfloat16 networks: against the oracle's bfloat16 emulation
(the same operands rounded to bfloat16, float64 accumulation), each tensor
within ``GRAD_TOL_BF16`` of its largest gradient (a stored activation or
gradient may round to the neighbouring bfloat16 value, 2^-8 relative, where
the float32 and float64 sums straddle a rounding boundary).  Adam: the
float32 update against the float64 formula on the GPU's own gradient.
Training as a whole: the loss against a teacher network's renders falls."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import backward as obwd
from oracle import render as oren
from tests.gpu_util import dev, empty, gpu_rays, host, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu

GRAD_TOL_F32 = 1e-4
GRAD_TOL_BF16 = 2e-2
KIND = {si.NERF_8x256: 1, si.NERF_4x64: 2, si.NERF_CELL_2x32: 3}
LPOS = {si.NERF_8x256: 10, si.NERF_4x64: 6, si.NERF_CELL_2x32: 10}


@pytest.fixture(scope="module")
def v():
    torch_cuda()
    import volume_rendering_amd as v
    return v


def _batch(R, H=None, W=None, seed=0, pose_seed=0):
    """R rays of one camera (the first R pixels of an H x W image), near 2,
    far 6, seeded target colours."""
    W = W or 32
    H = H or (R + W - 1) // W
    pose = si.poses(1, seed=pose_seed)[0]
    o, d = page_rays(H, W, 0.9 * W, pose)
    ro, rd = gpu_rays(H, W, 0.9 * W, pose)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    tgt = si.target_colors(R, seed)
    return dict(o=o[:R], d=d[:R], ro=ro[:R].contiguous(), rd=rd[:R].contiguous(), near=near, far=far, tgt=tgt)


def _cfg(v, shape, dtype, N, seed=7, use_pi=1, white=0, jitter=1, lr=1e-3):
    from volume_rendering_amd import _binding as B
    return B.nerf_train_cfg(net=B.nerf_mlp_desc(KIND[shape], dtype), n_samples=N, use_pi=use_pi, white_bkgd=white,
                            jitter=jitter, seed=seed, ray_offset=0, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8)


def _gpu_step(v, b, cfg, flat, adam=None, step=0, workspace=None):
    torch = torch_cuda()
    params = dev(flat)
    grad = empty(flat.size)
    loss = empty(1)
    rgb = empty((len(b["near"]), 3))
    m = vv = None
    if adam is not None:
        m, vv = dev(adam[0]), dev(adam[1])
    v.nerf_train_step(b["ro"], b["rd"], dev(b["near"]), dev(b["far"]), dev(b["tgt"]), cfg, params, loss, m, vv, step,
                      grad, rgb, workspace)
    torch.cuda.synchronize()
    out = dict(params=host(params), grad=host(grad), loss=float(host(loss)[0]), rgb=host(rgb))
    if adam is not None:
        out.update(m=host(m), v=host(vv))
    return out


def _tensors(flat, params):
    """Splits a flat vector into (name, array) pairs in the ABI order."""
    out, pos = [], 0
    seq = [(f"layer{i}", Wb) for i, Wb in enumerate(params["layers"])] + \
          [(k, params[k]) for k in ("sigma", "feature", "dir", "rgb")]
    for name, (W, b) in seq:
        for suffix, a in (("W", W), ("b", b)):
            n = np.asarray(a).size
            out.append((f"{name}.{suffix}", flat[pos:pos + n]))
            pos += n
    assert pos == flat.size
    return out


def _compare_grads(what, g_gpu, g_ref, params, tol):
    worst = 0.0
    for (name, a), (_, r) in zip(_tensors(g_gpu, params), _tensors(g_ref, params)):
        scale = np.max(np.abs(r))
        assert scale > 0, name
        e = np.max(np.abs(a - r)) / scale
        worst = max(worst, e)
        assert e <= tol, f"{what}: {name}: max error {e:.2e} of the tensor's largest gradient"
    say(f"  {what}: worst tensor error {worst:.2e} of its largest gradient (bar {tol:.0e})")


CASES = [
    # shape, rays, samples, use_pi, white: ragged sample counts and tiles,
    # two 64-sample chunks of the compositor, several split-K partial sums
    (si.NERF_4x64, 61, 23, 1, 0),
    (si.NERF_8x256, 40, 80, 0, 1),
    (si.NERF_CELL_2x32, 300, 32, 1, 0),
]


@pytest.mark.parametrize("shape,R,N,use_pi,white", CASES)
def test_train_grads_f32_match_oracle(v, shape, R, N, use_pi, white):
    say(f"train f32 {shape.depth}x{shape.width} R={R} N={N} use_pi={use_pi} white={white}")
    b = _batch(R, seed=R)
    p = si.nerf_params(shape, seed=11)
    cfg = _cfg(v, shape, 0, N, use_pi=use_pi, white=white)
    out = _gpu_step(v, b, cfg, si.flat_params(p))
    loss, rgb, grads = obwd.train_loss_and_grads(p, b["o"], b["d"], b["near"], b["far"], b["tgt"], N, LPOS[shape], 4,
                                                 seed=7, jitter=True, mode="f64", use_pi=bool(use_pi),
                                                 white_bkgd=bool(white))
    say(f"  loss gpu {out['loss']:.8e} oracle {loss:.8e}")
    assert abs(out["loss"] - loss) <= 1e-5 * loss
    assert np.max(np.abs(out["rgb"] - rgb)) <= 1e-4
    _compare_grads("f32 vs float64 definition", out["grad"], obwd.flatten(grads), p, GRAD_TOL_F32)
    # without Adam moments the parameters are left as they were
    assert np.array_equal(out["params"], si.flat_params(p))


@pytest.mark.parametrize("shape,R,N", [(si.NERF_8x256, 64, 64), (si.NERF_4x64, 100, 48)])
def test_train_grads_bf16_match_emulation(v, shape, R, N):
    say(f"train bf16 {shape.depth}x{shape.width} R={R} N={N}")
    b = _batch(R, seed=R + 1)
    p = si.nerf_params(shape, seed=12)
    out = _gpu_step(v, b, _cfg(v, shape, 1, N), si.flat_params(p))
    kw = dict(seed=7, jitter=True, use_pi=True)
    loss_e, rgb_e, g_e = obwd.train_loss_and_grads(p, b["o"], b["d"], b["near"], b["far"], b["tgt"], N, LPOS[shape],
                                                   4, mode="bf16", **kw)
    loss_d, rgb_d, g_d = obwd.train_loss_and_grads(p, b["o"], b["d"], b["near"], b["far"], b["tgt"], N, LPOS[shape],
                                                   4, mode="f64", **kw)
    say(f"  loss gpu {out['loss']:.6e} emulation {loss_e:.6e} definition {loss_d:.6e}")
    assert abs(out["loss"] - loss_e) <= 1e-2 * loss_e
    assert np.max(np.abs(out["rgb"] - rgb_d)) <= 2e-2  # the forward bar of bfloat16 networks
    _compare_grads("bf16 vs bfloat16 emulation", out["grad"], obwd.flatten(g_e), p, GRAD_TOL_BF16)
    # and the direction of the whole gradient against the float64 definition
    gd, gg = obwd.flatten(g_d), out["grad"].astype(np.float64)
    cos = gd @ gg / (np.linalg.norm(gd) * np.linalg.norm(gg))
    say(f"  cosine with the float64 gradient {cos:.6f}")
    assert cos > 0.99


def test_adam_step_matches_oracle(v):
    say("train adam 4x64")
    shape = si.NERF_4x64
    b = _batch(64, seed=3)
    p = si.nerf_params(shape, seed=13)
    flat = si.flat_params(p)
    g = si.rng(5, 99)
    m0 = (g.normal(size=flat.size) * 1e-3).astype(np.float32)
    v0 = (g.random(flat.size) * 1e-5).astype(np.float32)
    cfg = _cfg(v, shape, 0, 32, lr=5e-4)
    t = 5
    out = _gpu_step(v, b, cfg, flat, adam=(m0, v0), step=t)
    # the oracle's Adam on the GPU's own gradient (stage isolation)
    p1, m1, v1 = obwd.adam(flat.astype(np.float64), out["grad"].astype(np.float64), m0.astype(np.float64),
                           v0.astype(np.float64), t, 5e-4, 0.9, 0.999, 1e-8)
    gg = np.abs(out["grad"].astype(np.float64))
    assert np.all(np.abs(out["m"] - m1) <= 4e-7 * (np.abs(m0) + gg) + 1e-30)
    assert np.all(np.abs(out["v"] - v1) <= 4e-7 * (np.abs(v0) + gg * gg) + 1e-36)
    u = np.abs(p1 - flat)
    err = np.abs(out["params"] - p1)
    assert np.all(err <= 1.2e-7 * np.abs(p1) + 1e-5 * u + 1e-12)
    assert np.count_nonzero(out["params"] != flat) > 0.9 * flat.size


def test_train_step_is_deterministic_and_workspace_equivalent(v):
    say("train determinism 8x256 bf16")
    torch = torch_cuda()
    shape = si.NERF_8x256
    b = _batch(96, seed=4)
    flat = si.flat_params(si.nerf_params(shape, seed=14))
    cfg = _cfg(v, shape, 1, 64)
    a = _gpu_step(v, b, cfg, flat)
    ws = torch.empty(v.nerf_train_workspace_size(cfg, 96), dtype=torch.uint8, device="cuda")
    c = _gpu_step(v, b, cfg, flat, workspace=ws)
    assert np.array_equal(a["grad"], c["grad"]) and a["loss"] == c["loss"]
    assert np.array_equal(a["rgb"], c["rgb"])


@pytest.mark.parametrize("dtype", [0, 1])
def test_training_fits_a_teacher(v, dtype):
    """A 4x64 student trained with Adam on the renders of a 4x64 teacher
    (the oracle's forward render, float64): the loss falls."""
    say(f"train teacher fit dtype={dtype}")
    torch = torch_cuda()
    shape = si.NERF_4x64
    R, N, steps = 512, 32, 200
    pose = si.poses(1, seed=2)[0]
    o, d = page_rays(16, 32, 30.0, pose)
    near, far = np.full(R, 2.0, np.float32), np.full(R, 6.0, np.float32)
    teacher = si.nerf_params(shape, seed=21)
    teacher = dict(teacher, sigma=(teacher["sigma"][0], teacher["sigma"][1] + np.float32(1.0)))
    tgt = oren.render_nerf(o, d, near, far, teacher, None, n_coarse=N, n_fine=0, L_pos=6, L_dir=4, seed=3,
                           jitter=False)["rgb"].astype(np.float32)
    ro, rd = gpu_rays(16, 32, 30.0, pose)
    flat = si.flat_params(si.nerf_params(shape, seed=22))
    params, m, vv = dev(flat), dev(np.zeros_like(flat)), dev(np.zeros_like(flat))
    loss = empty(1)
    tn, tf, tg = dev(near), dev(far), dev(tgt)
    losses = []
    for t in range(1, steps + 1):
        cfg = _cfg(v, shape, dtype, N, seed=100 + t, lr=5e-3)
        v.nerf_train_step(ro, rd, tn, tf, tg, cfg, params, loss, m, vv, t)
        if t == 1 or t % 50 == 0:
            losses.append(float(host(loss)[0]))
    torch.cuda.synchronize()
    say(f"  losses {['%.3e' % x for x in losses]}")
    assert np.all(np.isfinite(losses))
    assert losses[-1] < 0.05 * losses[0]


@pytest.mark.parametrize("dtype", [0, 1])
def test_hierarchical_train_step(v, dtype):
    """The page's two-network step as two calls and the sampler: the coarse
    pass (stratified, weights out), nerf_sample_pdf on its weights, the fine
    pass on the merged depths (cfg.z).  Each pass is checked against the
    oracle's pass on the same depths; the merged depths against the oracle's
    chain (bins may flip where float32 and float64 weights straddle a CDF
    step)."""
    say(f"train hierarchical dtype={dtype}")
    torch = torch_cuda()
    shape = si.NERF_4x64
    R, NC, NF = 60, 16, 32
    b = _batch(R, seed=9)
    pc, pf = si.nerf_params(shape, seed=31), si.nerf_params(shape, seed=32)
    mode = "bf16" if dtype else "f64"
    ref = obwd.hierarchical_train_step(pc, pf, b["o"], b["d"], b["near"], b["far"], b["tgt"], n_coarse=NC, n_fine=NF,
                                       L_pos=6, L_dir=4, seed=7, mode=mode)
    tol = GRAD_TOL_BF16 if dtype else GRAD_TOL_F32
    # coarse pass with its weights
    w = empty((R, NC))
    cfg = _cfg(v, shape, dtype, NC)
    cfg.weights = w.data_ptr()
    out_c = _gpu_step(v, b, cfg, si.flat_params(pc))
    w_h = host(w)
    say(f"  coarse loss gpu {out_c['loss']:.6e} oracle {ref['loss_c']:.6e}; weights max err "
        f"{np.max(np.abs(w_h - ref['w_c'])):.2e}")
    assert abs(out_c["loss"] - ref["loss_c"]) <= (1e-2 if dtype else 1e-5) * ref["loss_c"]
    assert np.max(np.abs(w_h - ref["w_c"])) <= (2e-2 if dtype else 1e-5)
    _compare_grads("coarse pass", out_c["grad"], obwd.flatten(ref["grads_c"]), pc, tol)
    # the sampler on the GPU's weights, end to end
    zc = empty((R, NC))
    v.nerf_sample_stratified(dev(b["near"]), dev(b["far"]), NC, 7, 0, True, zc)
    assert np.array_equal(host(zc), ref["z_c"])
    z2 = empty((R, NC + NF))
    bins = empty((R, NF), dtype=torch.int32)
    v.nerf_sample_pdf(zc, w, NF, 7, 0, bin_idx=bins, z_merged=z2)
    z2_h = host(z2)
    # the chosen bins are integers; the depths inside a bin move with the
    # weights' last bits, so they are compared within a tolerance
    same = np.all(host(bins) == ref["bins"], axis=1)
    dz = np.max(np.abs(z2_h - ref["z2"]), axis=1)
    say(f"  chosen bins identical on {same.mean():.1%} of rays; merged depths on those within {dz[same].max():.2e}")
    assert same.mean() >= (0.8 if dtype else 0.95)
    if not dtype:
        assert dz[same].max() <= 1e-4
    # fine pass on the oracle's merged depths
    cfg_f = _cfg(v, shape, dtype, NC + NF)
    z_in = dev(ref["z2"].astype(np.float32))
    cfg_f.z = z_in.data_ptr()
    out_f = _gpu_step(v, b, cfg_f, si.flat_params(pf))
    say(f"  fine loss gpu {out_f['loss']:.6e} oracle {ref['loss_f']:.6e}")
    assert abs(out_f["loss"] - ref["loss_f"]) <= (1e-2 if dtype else 1e-5) * ref["loss_f"]
    _compare_grads("fine pass", out_f["grad"], obwd.flatten(ref["grads_f"]), pf, tol)
    torch.cuda.synchronize()

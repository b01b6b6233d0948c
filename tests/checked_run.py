"""Runs a representative set of calls through the checked library
(libnerf_mi355x_checked.so: the kernels built with -DNERF_CHECK record failed
index-range checks instead of faulting) and requires that no check fails.
A positive control then feeds NaN coarse weights to the inverse-CDF sampler,
outside its documented precondition (finite weights in [0, 100]; the kernel
runs on and keeps every index in range), and requires that the precondition
check records it and nothing else.

Run by tests/test_gpu_zchecked.py in a process of its own, because the
binding loads one library per process.  Exit status 0 when both hold."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import seeded_inputs as si  # noqa: E402
import volume_rendering_amd._binding as B  # noqa: E402

B._LIB_PATH = os.path.join(ROOT, "volume_rendering_amd", "libnerf_mi355x_checked.so")
import volume_rendering_amd as v  # noqa: E402

dev = torch.device("cuda:0")


def t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev) if dtype is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype)


def empty(*shape):
    return torch.empty(shape, device=dev)


def rays(n_poses, H, W, f, sel_n, seed):
    P = si.poses(n_poses, seed=0)
    ro = empty(n_poses * H * W, 3)
    rd = empty(n_poses * H * W, 3)
    for p in range(n_poses):
        v.nerf_gen_rays(P[p], W, H, f, f, 0.5 * W, 0.5 * H, ro[p * H * W:(p + 1) * H * W], rd[p * H * W:(p + 1) * H * W])
    sel = torch.from_numpy(si.subset(n_poses * H * W, sel_n, seed=seed)).to(dev)
    ro, rd = ro[sel].contiguous(), rd[sel].contiguous()
    return ro, rd, torch.full((sel_n,), 2.0, device=dev), torch.full((sel_n,), 6.0, device=dev)


def check(what):
    torch.cuda.synchronize()
    f = B.nerf_check_flags()
    print(f"{what}: flags {f:#x}", flush=True)
    return f


def main():
    if B.nerf_check_flags() != 0:
        print("not the checked library, or flags set before any call")
        return 1
    bad = 0
    R = 512
    ro, rd, near, far = rays(2, 400, 400, 555.0, R, 1)
    rgb, depth, acc = empty(R, 3), empty(R), empty(R)
    # NeRF renders: hierarchical 8x256 (bf16, fp32), tiny 4x64, with occupancy and termination
    for kind, shape, dt in ((1, si.NERF_8x256, 1), (1, si.NERF_8x256, 0), (2, si.NERF_4x64, 0)):
        nc_ = v.weights.pack_to_device(kind, dt, si.nerf_params(shape, seed=0, net_id=0))
        nf_ = v.weights.pack_to_device(kind, dt, si.nerf_params(shape, seed=0, net_id=1))
        w = B.nerf_weights(net=B.nerf_mlp_desc(kind, dt), coarse=nc_.data_ptr(), fine=nf_.data_ptr())
        cfg = B.nerf_render_cfg(mode=0, n_coarse=64, n_fine=128, use_pi=1, jitter=1, seed=3)
        v.nerf_render(ro, rd, near, far, w, cfg, rgb, depth, acc)
        bad |= check(f"nerf render kind {kind} dtype {dt}")
        occ = t(si.occupancy_bits(128, 0.3, seed=1).view(np.int32))
        cfg = B.nerf_render_cfg(mode=0, n_coarse=64, n_fine=128, use_pi=1, jitter=1, seed=3, term_T=1e-2,
                                box_lo=-1.5, box_hi=1.5, occ_res=128, occ=occ.data_ptr())
        v.nerf_render(ro, rd, near, far, w, cfg, rgb, depth, acc)
        bad |= check(f"nerf render kind {kind} dtype {dt}, occupancy and termination")
    # hash-grid field render (3D, 16 levels) and standalone encoders (3D, 2D with a level mask)
    g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
    tab = (torch.rand(((g.total_entries + 1) // 2 * 2, 2), device=dev) * 2 - 1).to(torch.float16)
    g.tables = tab.data_ptr()
    for dt in (1, 0):
        net = v.weights.pack_to_device(4, dt, si.hash_field_params(seed=3))
        w = B.nerf_weights(net=B.nerf_mlp_desc(4, dt), coarse=net.data_ptr())
        w.grid = B.C.pointer(g)
        cfg = B.nerf_render_cfg(mode=1, n_coarse=128, use_pi=1, jitter=1, seed=5, box_lo=-1.5, box_hi=1.5)
        v.nerf_render(ro, rd, near, far, w, cfg, rgb, depth, acc)
        bad |= check(f"hash render dtype {dt}")
    x = t(si.query_points(1 << 16, seed=2))
    out = empty(1 << 16, 32)
    v.nerf_encode_hashgrid(x, g, out)
    bad |= check("hash-grid encoder 3D")
    g2 = v.nerf_hashgrid_init(8, 2 ** 12, 8, 160, dim=2)
    g2.level_mask[3] = 0.0
    tab2 = (torch.rand(((g2.total_entries + 1) // 2 * 2, 2), device=dev) * 2 - 1).to(torch.float16)
    g2.tables = tab2.data_ptr()
    x2 = torch.rand((5001, 2), device=dev)
    v.nerf_encode_hashgrid(x2, g2, empty(5001, 16))
    bad |= check("hash-grid encoder 2D, level mask")
    # samplers and compositor
    z = empty(R, 64)
    v.nerf_sample_stratified(near, far, 64, 7, 0, True, z)
    wts = torch.rand((R, 64), device=dev)
    zm = empty(R, 192)
    v.nerf_sample_pdf(z, wts, 128, 7, 0, z_merged=zm)
    raw = torch.randn((R, 192, 4), device=dev)
    v.nerf_composite(raw, zm, rd, 0, rgb, depth, acc)
    bad |= check("stratified, inverse CDF and merge, compositing")
    # many tiny networks (16^3 cells, 128^3 occupancy) and the entry point that allocates nothing
    Rk = 4096
    ko, kd, kn, kf = rays(1, 800, 800, 1110.0, Rk, 2)
    stacked = si.cell_params_stacked(4096, seed=0)
    cells = v.weights.pack_many_to_device(3, 1, [si.cell_slice(stacked, c) for c in range(4096)])
    occ = t(si.occupancy_bits(128, 0.1, seed=0).view(np.int32))
    w = B.nerf_weights(net=B.nerf_mlp_desc(3, 1), cells=cells.data_ptr(), n_cells=4096)
    cfg = B.nerf_render_cfg(mode=2, n_coarse=192, use_pi=1, jitter=1, seed=0, term_T=1e-2, box_lo=-1.5, box_hi=1.5,
                            occ_res=128, cell_res=16, occ=occ.data_ptr())
    krgb, kdep, kacc = empty(Rk, 3), empty(Rk), empty(Rk)
    v.nerf_render(ko, kd, kn, kf, w, cfg, krgb, kdep, kacc)
    v.nerf_render_noalloc(ko, kd, kn, kf, w, cfg, krgb, kdep, kacc)
    bad |= check("many-network render (and without allocation)")
    # training step (8x256 bf16) and the hash-grid INR step
    Rt = 256
    to, td, tn, tf = rays(2, 400, 400, 555.0, Rt, 3)
    ph = si.nerf_params(si.NERF_8x256, seed=0, net_id=0)
    params = t(si.flat_params(ph))
    tcfg = B.nerf_train_cfg(net=B.nerf_mlp_desc(1, 1), n_samples=64, use_pi=1, white_bkgd=0, jitter=1, seed=1,
                            ray_offset=0, lr=5e-4, beta1=0.9, beta2=0.999, eps=1e-8)
    v.nerf_train_step(to, td, tn, tf, t(si.target_colors(Rt, seed=0)), tcfg, params, empty(1),
                      torch.zeros_like(params), torch.zeros_like(params), 1)
    bad |= check("training step")
    gi = v.nerf_hashgrid_init(8, 2 ** 12, 8, 160, dim=2)
    icfg = B.nerf_hash_inr_cfg(hidden=32, n_out=1, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8)
    n_par = v.nerf_hash_inr_param_count(gi, icfg)
    ip = (torch.rand(n_par, device=dev) - 0.5) * 0.1
    xi = torch.rand((3000, 2), device=dev)
    v.nerf_hash_inr_train_step(xi, torch.rand((3000, 1), device=dev), gi, icfg, ip, empty(1),
                               torch.zeros_like(ip), torch.zeros_like(ip), 1)
    bad |= check("hash-grid INR step")
    # full-size workloads: the largest indices each path forms
    Rf = 800 * 800
    fo, fd, fn, ff = rays(1, 800, 800, 1110.0, Rf, 4)
    frgb, fdep, facc = empty(Rf, 3), empty(Rf), empty(Rf)
    w = B.nerf_weights(net=B.nerf_mlp_desc(3, 1), cells=cells.data_ptr(), n_cells=4096)
    v.nerf_render(fo, fd, fn, ff, w, cfg, frgb, fdep, facc)
    bad |= check("many-network render, 640,000 rays")
    nc_ = v.weights.pack_to_device(1, 1, si.nerf_params(si.NERF_8x256, seed=0, net_id=0))
    nf_ = v.weights.pack_to_device(1, 1, si.nerf_params(si.NERF_8x256, seed=0, net_id=1))
    w = B.nerf_weights(net=B.nerf_mlp_desc(1, 1), coarse=nc_.data_ptr(), fine=nf_.data_ptr())
    hcfg = B.nerf_render_cfg(mode=0, n_coarse=64, n_fine=128, use_pi=1, jitter=1, seed=0)
    v.nerf_render(fo, fd, fn, ff, w, hcfg, frgb, fdep, facc)
    bad |= check("hierarchical render, one 800 x 800 pose")
    Rh = 256 * 256
    ho, hd, hn, hf = rays(1, 256, 256, 355.2, Rh, 5)
    net = v.weights.pack_to_device(4, 1, si.hash_field_params(seed=3))
    w = B.nerf_weights(net=B.nerf_mlp_desc(4, 1), coarse=net.data_ptr())
    w.grid = B.C.pointer(g)
    cfg_h = B.nerf_render_cfg(mode=1, n_coarse=128, use_pi=1, jitter=1, seed=5, box_lo=-1.5, box_hi=1.5)
    v.nerf_render(ho, hd, hn, hf, w, cfg_h, empty(Rh, 3), empty(Rh), empty(Rh))
    bad |= check("hash render, 256 x 256 rays")
    xq = t(si.query_points(1 << 22, seed=0))
    v.nerf_encode_hashgrid(xq, g, empty(1 << 22, 32))
    bad |= check("hash-grid encoder, 2^22 points")
    if bad:
        print(f"FAILED: index checks recorded {bad:#x}")
        return 1
    # positive control: NaN weights break the sampler's precondition (bit 8)
    wn = torch.full((R, 64), float("nan"), device=dev)
    v.nerf_sample_pdf(z, wn, 128, 7, 0, z_merged=zm)
    f = check("positive control (NaN coarse weights)")
    if f != (1 << 8):
        print(f"FAILED: the control should set bit 8 alone, got {f:#x}")
        return 1
    if B.nerf_check_flags() != 0:
        print("FAILED: flags not cleared")
        return 1
    print("checked library: no failed index check; the control was recorded")
    return 0


if __name__ == "__main__":
    sys.exit(main())

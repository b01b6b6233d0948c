"""Throughput of the NeRF forward-render hot path on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload hierarchical|coarse|tiny|hash|kilo|encode|composite|hashgrid|mlp|train|
                                train_hierarchical]
                    [--dtype bf16|f32] [--no-cpu-baseline]

A step is one ``nerf_render`` over the whole workload with rays, weights
and tables already resident in HBM.  Default workload: the hierarchical
render, 4 poses x 800x800 rays (focal 1110), 64 stratified + 128
inverse-CDF samples per ray, 8x256 coarse and fine networks in bfloat16.

The standalone workloads time one call of a single step against the HBM
roofline: ``encode`` the frequency encoding (L = 10, with the input) of the
coarse workload's 81.92M sample points, ``composite`` the compositing of its
1.28M rays x 64 samples, ``hashgrid`` the 16-level hash-grid encoding of
2^22 points (all against the HBM roofline), ``mlp`` the 8x256 network in
bfloat16 on 2^23 encoded samples read from HBM (against the MFMA roofline),
``train`` one training step (nerf_train_step: forward, loss, every gradient,
Adam) on 4096 random rays x 64 samples of the 8x256 network, its algorithmic
products against the MFMA roofline over the whole step's time;
``train_hierarchical`` the page's two-network step (coarse 64 samples,
inverse-CDF resampling, fine network on the 192 merged samples).

Prints one JSON line: rays/s (``value``), samples/s, the dominant kernel's
achieved throughput against its roofline (timed live with HIP events on
the launch stream), and the CPU oracle's throughput on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA TFLOP/s, MI355X
MACS_8x256 = 593408
MACS_4x64 = 21952
MACS_HASH_FIELD = 19712
MACS_CELL_2x32 = 5088
# multiply-adds per sample of the products that carry a gradient back to a
# layer's input: every layer but the first, without the columns of the
# position encoding (skip layer) and of the direction encoding
MACS_8x256_DINPUT = MACS_8x256 - 256 * 63 - 256 * 63 - 128 * 27

# Memory-side bytes per launch of the dominant kernel(s), from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes scaled by a 1 GiB copy (x2.0 and x1.0),
# keyed by (workload, dtype), with the digest of the files holding the
# kernels' device code and launch shapes at the time the counters were taken
# (host-only declarations and workspace layouts are left out).  A figure whose
# files have changed since is stale and reported as null.
_INR_SOURCES = ["hash_train.hip", "inr_plan.hpp", "optim.hpp", "raysteps.hpp", "common.hpp"]
KERNEL_SOURCES = {
    "hierarchical": ["render_common.hpp", "render_nerf_bf16.hip", "mlp.hpp", "nets.hpp", "raysteps.hpp",
                     "common.hpp"],
    "encode": ["kernels.hip", "common.hpp"],
    "composite": ["kernels.hip", "common.hpp"],
    "hashgrid": ["kernels.hip", "raysteps.hpp", "common.hpp"],
    "hash": ["render_common.hpp", "render_hash.hip", "mlp.hpp", "nets.hpp", "raysteps.hpp", "common.hpp"],
    "kilo": ["kilo.hip", "mlp.hpp", "nets.hpp", "raysteps.hpp", "common.hpp"],
    "train": ["train.hip", "train_plan.hpp", "optim.hpp", "mlp.hpp", "nets.hpp", "common.hpp"],
    "hash_inr": _INR_SOURCES,
    "hash_inr_4m": _INR_SOURCES,
}
MEASURED_TRAFFIC = {
    ("hierarchical", "bf16"): (5.1258e8, "f034620437ea85cf"),   # k_render_nerf per launch
    ("kilo", "bf16"): (1.5026e9, "2b3cdabff501d0ed"),          # every kernel of one render
    ("hashgrid", "f32"): (6.4819e9, "148a965141f8efaa"),       # both encoder kernels
    ("train", "bf16"): (9.2043e9, "d4e1de2ca3da3bcb"),       # every kernel of one step
    ("hash", "bf16"): (1.9769e10, "b9fa053d5b66c96c"),       # k_render_hash per launch (gathers missing L2)
    ("hash_inr", "f32"): (6.48e6, "2ab8671f0bf90ff6"),         # every kernel of one step, 96 x 96
    ("hash_inr_4m", "f32"): (7.64e8, "2ab8671f0bf90ff6"),     # every kernel of one step, 2048 x 2048
}


def source_digest(workload):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(workload, []):
        with open(os.path.join(ROOT, "volume_rendering_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, dtype):
    rec = MEASURED_TRAFFIC.get((workload, dtype))
    if rec is None or workload not in KERNEL_SOURCES or source_digest(workload) != rec[1]:
        return None
    return rec[0]

WORKLOADS = {
    # name: (poses, hemisphere, H, W, focal, n_coarse, n_fine, net kind, chunk)
    "hierarchical": dict(poses=4, hemi=True, H=800, W=800, focal=1110.0, nc=64, nf=128, kind=1, chunk=0),
    # the same with empty-space skipping (128^3 occupancy at 10%) and termination at T < 1e-2
    "hierarchical_occ": dict(poses=4, hemi=True, H=800, W=800, focal=1110.0, nc=64, nf=128, kind=1, chunk=0,
                             occ=True),
    "coarse": dict(poses=8, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=0, kind=1, chunk=65536),
    "tiny": dict(poses=1, hemi=False, H=32, W=32, focal=40.0, nc=16, nf=0, kind=2, chunk=0),
    "hash": dict(poses=1, hemi=True, H=256, W=256, focal=355.2, nc=128, nf=0, kind=4, chunk=0),
    "kilo": dict(poses=1, hemi=True, H=800, W=800, focal=1110.0, nc=192, nf=0, kind=3, chunk=0),
    # standalone steps (kind 0): coarse workload's rays and samples, or 2^22 grid queries
    "encode": dict(poses=8, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=0, kind=0, chunk=0),
    "composite": dict(poses=8, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=0, kind=0, chunk=0),
    "hashgrid": dict(points=1 << 22, kind=0),
    "mlp": dict(poses=1, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=0, kind=0, chunk=0, rays=1 << 17),
    # one training step: 4096 random rays of the coarse workload's images, 64 stratified samples, 8x256
    "train": dict(poses=8, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=0, kind=0, chunk=0, rays=4096),
    # the page's two-network step: coarse 64 + fine 128 (192 merged), two 8x256 networks
    "train_hierarchical": dict(poses=8, hemi=True, H=400, W=400, focal=555.0, nc=64, nf=128, kind=0, chunk=0,
                               rays=4096),
    # one full-batch Adam step of the 2D hash-grid INR of "Instant-NGP - Visual Experiments", Experiment 2
    # (8 levels, T = 2^12, N 8..160, decoder 16 -> 32 -> 1, lr 1e-2) on its 96 x 96 image; the same model
    # on a 2048 x 2048 image (4.19M points per step)
    # the page's video: a 24-frame 360 degree pose sweep (30 degrees elevation, radius 4), white background,
    # coarse 64 + fine 128 on the two 8x256 networks, through nerf_render_poses
    "sweep": dict(kind=0, frames=24, H=400, W=400, focal=555.0, nc=64, nf=128),
    "hash_inr": dict(kind=0, res=96, L=8, T=2 ** 12, nmin=8, nmax=160, hidden=32, lr=1e-2),
    "hash_inr_4m": dict(kind=0, res=2048, L=8, T=2 ** 12, nmin=8, nmax=160, hidden=32, lr=1e-2),
}
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="hierarchical", choices=sorted(WORKLOADS))
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle CPU time (all threads)")
    ap.add_argument("--poses", type=int, default=0, help="override the workload's pose count")
    ap.add_argument("--n-fine", type=int, default=-1, help="override the workload's inverse-CDF samples")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device copy of MIB mebibytes (counter calibration)")
    return ap.parse_args()


def host_threads():
    """(BLAS threads the oracle uses, nproc, CPUs in this process's affinity mask)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    return int(threads), os.cpu_count() or 1, len(os.sched_getaffinity(0))


def with_single_thread(measure, record):
    """Adds the oracle's rate on one thread (BLAS limited to 1) and the host
    core counts to a cpu_baseline record measured on all threads."""
    _, nproc, affinity = host_threads()
    record["nproc"], record["affinity_cpus"] = nproc, affinity
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = measure()
        record["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
    except Exception as e:  # pragma: no cover
        record["single_thread"] = {"error": str(e)}
    return record


def cpu_baseline(wl, kind, rays_o, rays_d, near, far, coarse, fine, target_s, occ=None):
    """The oracle (float64 definition) timed on a bounded sample of rays."""
    from oracle import render as oren
    threads = host_threads()[0]
    Lp = 6 if kind == 2 else 10
    if kind == 3:
        target_s = min(target_s, 6.0)

    def run(n):
        sel = np.linspace(0, rays_o.shape[0] - 1, n).astype(np.int64)
        t = time.perf_counter()
        if kind == 3:
            cells, occ_k = coarse
            oren.render_kilo(rays_o[sel], rays_d[sel], near[sel], far[sel], occ_k, lambda c: cells[c], wl["nc"],
                             seed=0, term_T=1e-2, ray_offset=sel)
        elif kind == 4:
            grid, tabs, field = coarse
            oren.render_hash(rays_o[sel], rays_d[sel], near[sel], far[sel], grid, tabs, field, wl["nc"], seed=0,
                             ray_offset=sel)
        else:
            extra = dict(occ=occ, term_T=1e-2) if occ is not None else {}
            oren.render_nerf(rays_o[sel], rays_d[sel], near[sel], far[sel], coarse, fine if wl["nf"] else None,
                             wl["nc"], wl["nf"], Lp, 4, seed=0, ray_offset=sel, **extra)
        return time.perf_counter() - t

    def measure(t_s):
        n = 8
        dt = run(n)
        n2 = int(min(rays_o.shape[0], max(n, n * t_s / max(dt, 1e-3))))
        dt2 = run(n2)
        return {"value": n2 / dt2, "unit": "rays/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{n2} rays evenly spaced over the workload, float64 oracle, {dt2:.1f} s"}

    rec = measure(target_s)
    return with_single_thread(lambda: dict(measure(target_s / 2), cores=1), rec)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path.  Rays are independent, so the "
              "render would shard by contiguous pixel blocks per GPU (same counters, replicated networks) "
              "and gather rgb/depth/acc at the end.", file=sys.stderr)
        sys.exit(2)

    import torch
    import seeded_inputs as si
    import volume_rendering_amd as v
    from volume_rendering_amd import _binding as B

    wl = dict(WORKLOADS[args.workload])
    if wl["kind"] == 0:
        return standalone(args, wl)
    if args.poses > 0:
        wl["poses"] = args.poses
    if args.n_fine >= 0:
        wl["nf"] = args.n_fine
    dtype = 1 if args.dtype == "bf16" else 0
    kind = wl["kind"]
    if kind == 2 and args.dtype == "bf16" and args.workload == "tiny":
        dtype = 0  # the tiny workload is defined in float32
    dt_name = "bf16" if dtype else "f32"
    dev = torch.device("cuda")

    # rays on the device
    P = si.poses(wl["poses"], seed=0, hemisphere=wl["hemi"])
    H, W, f = wl["H"], wl["W"], wl["focal"]
    R = wl["poses"] * H * W
    ro = torch.empty((R, 3), device=dev)
    rd = torch.empty((R, 3), device=dev)
    for p in range(wl["poses"]):
        v.nerf_gen_rays(P[p], W, H, f, f, 0.5 * W, 0.5 * H, ro[p * H * W:(p + 1) * H * W],
                        rd[p * H * W:(p + 1) * H * W])
    near = torch.full((R,), 2.0, device=dev)
    far = torch.full((R,), 6.0, device=dev)

    grid_keep = None
    kilo_keep = None
    if kind == 3:
        stacked = si.cell_params_stacked(4096, seed=0)
        cell_list = [si.cell_slice(stacked, c) for c in range(4096)]
        cells_dev = v.weights.pack_many_to_device(3, dtype, cell_list)
        occ_bits = si.occupancy_bits(128, 0.1, seed=0)
        occ_dev = torch.from_numpy(occ_bits.view(np.int32)).to(dev)
        nlive = torch.zeros(1, dtype=torch.int64, device=dev)
        kilo_keep = (cells_dev, occ_dev, nlive)
        coarse_p, fine_p = (cell_list, si.occupancy_dense(occ_bits)), None
        nets = []
        mode = B.NERF_MODE_KILO
    elif kind == 4:
        g = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
        tabs = si.hash_tables(list(g.size)[:16], seed=0, scale=1.0)
        tdev = torch.from_numpy(np.concatenate(tabs, 0)).to(dev)
        g.tables = tdev.data_ptr()
        field = si.hash_field_params(seed=0)
        nets = [v.weights.pack_to_device(4, dtype, field)]
        grid_keep = (g, tdev)
        coarse_p, fine_p = field, None
        mode = B.NERF_MODE_HASH
    else:
        shape = si.NERF_8x256 if kind == 1 else si.NERF_4x64
        coarse_p = si.nerf_params(shape, seed=0, net_id=0)
        fine_p = si.nerf_params(shape, seed=0, net_id=1)
        nets = [v.weights.pack_to_device(kind, dtype, coarse_p), v.weights.pack_to_device(kind, dtype, fine_p)]
        mode = B.NERF_MODE_NERF
    skipping = kind == 3 or wl.get("occ", False)
    cfg = B.nerf_render_cfg(mode=mode, n_coarse=wl["nc"], n_fine=wl["nf"], use_pi=1, jitter=1, seed=0,
                            chunk=wl["chunk"], box_lo=-1.5, box_hi=1.5, term_T=1e-2 if skipping else 0.0,
                            occ_res=128, cell_res=16)
    occ_keep = None
    if wl.get("occ", False):
        occ_bits = si.occupancy_bits(128, 0.1, seed=0)
        occ_keep = (torch.from_numpy(occ_bits.view(np.int32)).to(dev), torch.zeros(1, dtype=torch.int64, device=dev))
        cfg.occ = occ_keep[0].data_ptr()
        cfg.dbg_n_live = occ_keep[1].data_ptr()
    if kilo_keep is not None:
        w = B.nerf_weights(net=B.nerf_mlp_desc(kind, dtype), cells=kilo_keep[0].data_ptr(), n_cells=4096)
        cfg.occ = kilo_keep[1].data_ptr()
        cfg.dbg_n_live = kilo_keep[2].data_ptr()
        ws_bytes = B.nerf_render_workspace_size(cfg, R)
        kilo_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        cfg.workspace, cfg.workspace_bytes = kilo_ws.data_ptr(), ws_bytes
    else:
        w = B.nerf_weights(net=B.nerf_mlp_desc(kind, dtype), coarse=nets[0].data_ptr(),
                           fine=nets[1].data_ptr() if len(nets) > 1 else None)
    if grid_keep is not None:
        import ctypes
        w.grid = ctypes.pointer(grid_keep[0])
    rgb = torch.empty((R, 3), device=dev)
    depth = torch.empty((R,), device=dev)
    acc = torch.empty((R,), device=dev)

    def step():
        v.nerf_render(ro, rd, near, far, w, cfg, rgb, depth, acc)

    _calibration_copy(args, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_kernel = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

    if kind == 3:
        n_mlp_samples = int(kilo_keep[2].item())  # live samples the cell networks evaluated
    elif occ_keep is not None:
        n_mlp_samples = int(occ_keep[1].item())  # live samples (inside the box, occupied), both passes
    else:
        n_mlp_samples = R * (wl["nc"] + (wl["nc"] + wl["nf"] if wl["nf"] else 0))
    macs = {1: MACS_8x256, 2: MACS_4x64, 3: MACS_CELL_2x32, 4: MACS_HASH_FIELD}[kind]
    flops = 2.0 * macs * n_mlp_samples  # algorithmic network FLOPs per launch (all chunks of one step)
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    peak = PEAK[dt_name]
    out = {
        "metric": "rays/sec & samples/sec (coarse64+fine128, 8x256 MLP); MFMA util %, HBM GB/s %",
        "value": R / (ms_step * 1e-3),
        "unit": "rays/s",
        "samples_per_sec": n_mlp_samples / (ms_step * 1e-3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic: seeded hemisphere poses, He-uniform random weights",
        "config": {"workload": args.workload, "rays": R, "poses": wl["poses"], "H": H, "W": W, "focal": f,
                   "n_coarse": wl["nc"], "n_fine": wl["nf"],
                   "net": {1: "8x256", 2: "4x64", 3: "4096 cells 2x32", 4: "hash-field"}[kind],
                   "chunk": wl["chunk"],
                   **({"occupancy": "128^3 at 10%", "term_T": 1e-2} if occ_keep is not None else {})},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic(args.workload, dt_name),
                     "kernel": {1: "k_render_nerf", 2: "k_render_nerf", 3: "kilo pipeline", 4: "k_render_hash"}[kind],
                     "kernel_ms": ms_kernel,
                     "flop_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        o_h, d_h = ro.cpu().numpy(), rd.cpu().numpy()
        nf_h = near.cpu().numpy()
        ff_h = far.cpu().numpy()
        if kind == 4:
            from oracle import encoding as oenc
            og = oenc.hashgrid_3d()
            base = cpu_baseline(wl, kind, o_h, d_h, nf_h, ff_h, (og, tabs, coarse_p), None, args.cpu_seconds)
        else:
            occ_d = si.occupancy_dense(si.occupancy_bits(128, 0.1, seed=0)) if occ_keep is not None else None
            base = cpu_baseline(wl, kind, o_h, d_h, nf_h, ff_h, coarse_p, fine_p, args.cpu_seconds, occ_d)
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


def _calibration_copy(args, torch):
    """One plain device copy of --calibrate-copy MiB, whose FETCH_SIZE and
    WRITE_SIZE in a counter pass give the scale of those counters."""
    if args.calibrate_copy > 0:
        src = torch.empty(args.calibrate_copy << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def _timed(args, step, torch):
    _calibration_copy(args, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_kernel = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    return ms_step, ms_kernel


def _cpu_rate(fn, n_total, target_s, unit, what):
    """Runs the oracle on growing evenly spaced samples until it takes about
    target_s seconds; returns the cpu_baseline record (all threads, plus one
    thread)."""
    threads = host_threads()[0]

    def measure(t_s, cores):
        n = 1024
        while True:
            sel = np.linspace(0, n_total - 1, min(n, n_total)).astype(np.int64)
            t = time.perf_counter()
            fn(sel)
            dt = time.perf_counter() - t
            if dt >= 0.3 * t_s or len(sel) == n_total:
                break
            n = int(n * min(16.0, max(2.0, t_s / max(dt, 1e-3))))
        return {"value": len(sel) / dt, "unit": unit, "cores": cores, "kind": "oracle",
                "sample": f"{len(sel)} {what} evenly spaced over the workload, float64 oracle, {dt:.1f} s"}

    return with_single_thread(lambda: measure(target_s / 2, 1), measure(target_s, int(threads)))


def standalone(args, wl):
    """One standalone step of the path against the HBM roofline."""
    import torch
    import seeded_inputs as si
    import volume_rendering_amd as v

    dev = torch.device("cuda")
    name = args.workload
    if name in ("encode", "composite", "mlp"):
        P = si.poses(wl["poses"], seed=0, hemisphere=wl["hemi"])
        H, W, f = wl["H"], wl["W"], wl["focal"]
        R, N = wl["poses"] * H * W, wl["nc"]
        ro = torch.empty((R, 3), device=dev)
        rd = torch.empty((R, 3), device=dev)
        for p in range(wl["poses"]):
            v.nerf_gen_rays(P[p], W, H, f, f, 0.5 * W, 0.5 * H, ro[p * H * W:(p + 1) * H * W],
                            rd[p * H * W:(p + 1) * H * W])
        near = torch.full((R,), 2.0, device=dev)
        far = torch.full((R,), 6.0, device=dev)
        z = torch.empty((R, N), device=dev)
        v.nerf_sample_stratified(near, far, N, 0, 0, True, z)
    if name in ("train", "train_hierarchical"):
        return train_bench(args, wl)
    if name.startswith("hash_inr"):
        return inr_bench(args, wl)
    if name == "sweep":
        return sweep_bench(args, wl)
    if name == "mlp":
        Rm = wl["rays"]
        x = (ro[:Rm, None, :] + z[:Rm, :, None] * rd[:Rm, None, :]).reshape(-1, 3).contiguous()
        dirs = (rd[:Rm] / rd[:Rm].norm(dim=1, keepdim=True)).contiguous()
        n = x.shape[0]
        enc_x = torch.empty((n, 63), device=dev)
        enc_v = torch.empty((Rm, 27), device=dev)
        v.nerf_encode_freq(x, 10, True, True, 0, enc_x)
        v.nerf_encode_freq(dirs, 4, True, True, 0, enc_v)
        params = si.nerf_params(si.NERF_8x256, seed=0, net_id=0)
        packed = v.weights.pack_to_device(1, 1, params)
        raw = torch.empty((n, 4), device=dev)

        def step():
            v.nerf_mlp(1, 1, packed, enc_x, enc_v, N, raw)

        ms_step, ms_kernel = _timed(args, step, torch)
        flops = 2.0 * MACS_8x256 * n
        achieved = flops / (ms_kernel * 1e-3) / 1e12
        out_rec = {
            "metric": "samples/s, 8x256 network on encoded inputs (MFMA util %)",
            "value": n / (ms_step * 1e-3), "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic: coarse-workload sample points and directions, He-uniform random weights",
            "config": {"workload": name, "samples": n, "rays": Rm, "samples_per_ray": N, "net": "8x256",
                       "inputs": "float32 encodings in HBM (63 + 27 per ray)"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK["bf16"], "unit": "TFLOP/s",
                         "frac": achieved / PEAK["bf16"], "traffic": None, "kernel": "k_mlp",
                         "kernel_ms": ms_kernel, "flop_per_launch": flops},
        }
        if not args.no_cpu_baseline:
            from oracle import mlp as omlp
            ex_h, ev_h = enc_x.cpu().numpy(), enc_v.cpu().numpy()
            base = _cpu_rate(lambda sel: omlp.nerf_forward(params, ex_h[sel], ev_h[sel // N]), n, args.cpu_seconds,
                             "samples/s", "samples")
            out_rec["cpu_baseline"] = base
        print(json.dumps(out_rec), flush=True)
        return
    if name == "encode":
        x = (ro[:, None, :] + z[:, :, None] * rd[:, None, :]).reshape(-1, 3).contiguous()
        n = x.shape[0]
        L = 10
        out = torch.empty((n, 3 + 6 * L), device=dev)

        def step():
            v.nerf_encode_freq(x, L, True, True, 0, out)

        units, unit = n, "points/s"
        bytes_per_unit = 12 + 4 * (3 + 6 * L)
        kernel = "k_encode_freq"
        config = {"workload": name, "points": n, "L": L, "include_input": True, "out": "f32",
                  "source": "8 poses x 400x400 rays x 64 stratified samples"}
        data = "synthetic: seeded hemisphere poses, jittered stratified depths"
        if not args.no_cpu_baseline:
            from oracle import encoding as oenc
            xh = x.cpu().numpy()
            base = _cpu_rate(lambda sel: oenc.freq_encode(xh[sel], L), n, args.cpu_seconds, "points/s", "points")
    elif name == "composite":
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        raw = (torch.randn((R, N, 4), device=dev, generator=g) * 3.0).contiguous()
        rgb = torch.empty((R, 3), device=dev)
        depth = torch.empty((R,), device=dev)
        acc = torch.empty((R,), device=dev)
        w = torch.empty((R, N), device=dev)

        def step():
            v.nerf_composite(raw, z, rd, False, rgb, depth, acc, w)

        units, unit = R * N, "samples/s"
        bytes_per_unit = 16 + 4 + 4 + 32.0 / N  # raw, z, weights out per sample; rays_d + rgb, depth, acc per ray
        kernel = "k_composite"
        config = {"workload": name, "rays": R, "samples_per_ray": N, "weights_out": True,
                  "source": "8 poses x 400x400 rays x 64 stratified samples"}
        data = "synthetic: seeded hemisphere poses, jittered depths, raw ~ 3 N(0,1) (seeded device generator)"
        if not args.no_cpu_baseline:
            from oracle import composite as ocomp
            raw_h, z_h, d_h = raw.cpu().numpy(), z.cpu().numpy(), rd.cpu().numpy()
            base = _cpu_rate(lambda sel: ocomp.volume_render(raw_h[sel], z_h[sel], d_h[sel]), R, args.cpu_seconds,
                             "samples/s", "rays x 64 samples")
            base["value"] *= N
            if "value" in base.get("single_thread", {}):
                base["single_thread"]["value"] *= N
    else:  # hashgrid
        n = wl["points"]
        grid = v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048)
        tabs = si.hash_tables(list(grid.size)[:16], seed=0, scale=1e-4)
        tdev = torch.from_numpy(np.concatenate(tabs, 0)).to(dev)
        grid.tables = tdev.data_ptr()
        xh = si.query_points(n, seed=0)
        x = torch.from_numpy(xh).to(dev)
        out = torch.empty((n, 32), device=dev)

        def step():
            v.nerf_encode_hashgrid(x, grid, out)

        units, unit = n, "points/s"
        # point in (12 B) + 32 float32 features out (128 B) + 16 levels x 8
        # corners x 4 B gathered from the tables (512 B); the gathers are
        # served by L2 and the memory-side cache, not only by HBM
        bytes_per_unit = 12 + 128 + 512
        kernel = "k_encode_hash + k_encode_hash_lds"
        config = {"workload": name, "points": n, "levels": 16, "table_size": 2 ** 19, "n_min": 16, "n_max": 2048}
        data = "synthetic: seeded uniform points in the unit cube, tables U(-1e-4, 1e-4) float16"
        if not args.no_cpu_baseline:
            from oracle import encoding as oenc
            og = oenc.hashgrid_3d()
            base = _cpu_rate(lambda sel: og.encode(xh[sel], tabs), n, args.cpu_seconds, "points/s", "points")

    ms_step, ms_kernel = _timed(args, step, torch)
    achieved = bytes_per_unit * units / (ms_kernel * 1e-3) / 1e9
    out_rec = {
        "metric": {"encode": "points/s, frequency encoding (HBM GB/s %)",
                   "composite": "samples/s, compositing (HBM GB/s %)",
                   "hashgrid": "points/s, hash-grid encoding (HBM GB/s %)"}[name],
        "value": units / (ms_step * 1e-3), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": data, "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(name, "f32"),
                     "kernel": kernel, "kernel_ms": ms_kernel, "bytes_per_launch": bytes_per_unit * units},
    }
    if not args.no_cpu_baseline:
        out_rec["cpu_baseline"] = base
    print(json.dumps(out_rec), flush=True)


def train_bench(args, wl):
    """One training step of the 8x256 network on a batch of 4096 random rays
    (nerf_train_step: forward, compositing, loss, every gradient, Adam); with
    n_fine > 0 the page's two-network step: the coarse network on 64
    stratified samples (weights out), inverse-CDF resampling, the fine
    network on the 192 merged samples."""
    import torch
    import seeded_inputs as si
    import volume_rendering_amd as v
    from volume_rendering_amd import _binding as B

    dev = torch.device("cuda")
    P = si.poses(wl["poses"], seed=0, hemisphere=wl["hemi"])
    H, W, f = wl["H"], wl["W"], wl["focal"]
    R_all, R, NC, NF = wl["poses"] * H * W, wl["rays"], wl["nc"], wl["nf"]
    ro_all = torch.empty((R_all, 3), device=dev)
    rd_all = torch.empty((R_all, 3), device=dev)
    for p in range(wl["poses"]):
        v.nerf_gen_rays(P[p], W, H, f, f, 0.5 * W, 0.5 * H, ro_all[p * H * W:(p + 1) * H * W],
                        rd_all[p * H * W:(p + 1) * H * W])
    sel = torch.from_numpy(si.subset(R_all, R, seed=0)).to(dev)
    ro, rd = ro_all[sel].contiguous(), rd_all[sel].contiguous()
    near = torch.full((R,), 2.0, device=dev)
    far = torch.full((R,), 6.0, device=dev)
    tgt_h = si.target_colors(R, seed=0)
    tgt = torch.from_numpy(tgt_h).to(dev)
    dtype = 1 if args.dtype == "bf16" else 0
    nets_h = [si.nerf_params(si.NERF_8x256, seed=0, net_id=k) for k in range(2 if NF else 1)]
    state = [(torch.from_numpy(si.flat_params(ph)).to(dev),) for ph in nets_h]
    state = [(p_[0], torch.zeros_like(p_[0]), torch.zeros_like(p_[0])) for p_ in state]
    loss = torch.empty(2, device=dev)
    cfgs = [B.nerf_train_cfg(net=B.nerf_mlp_desc(1, dtype), n_samples=n, use_pi=1, white_bkgd=0, jitter=1, seed=0,
                             ray_offset=0, lr=5e-4, beta1=0.9, beta2=0.999, eps=1e-8) for n in ([NC, NC + NF] if NF
                                                                                                else [NC])]
    ws = torch.empty(max(v.nerf_train_workspace_size(c, R) for c in cfgs), dtype=torch.uint8, device=dev)
    if NF:
        w_c = torch.empty((R, NC), device=dev)
        z_c = torch.empty((R, NC), device=dev)
        z2 = torch.empty((R, NC + NF), device=dev)
        cfgs[0].weights = w_c.data_ptr()
        cfgs[1].z = z2.data_ptr()
    it = [0]

    def step():
        it[0] += 1
        for c in cfgs:
            c.seed = it[0]
        p0, m0, v0 = state[0]
        v.nerf_train_step(ro, rd, near, far, tgt, cfgs[0], p0, loss[0:1], m0, v0, it[0], workspace=ws)
        if NF:
            v.nerf_sample_stratified(near, far, NC, it[0], 0, True, z_c)
            v.nerf_sample_pdf(z_c, w_c, NF, it[0], 0, z_merged=z2)
            p1, m1, v1 = state[1]
            v.nerf_train_step(ro, rd, near, far, tgt, cfgs[1], p1, loss[1:2], m1, v1, it[0], workspace=ws)

    ms_step, ms_kernel = _timed(args, step, torch)
    S = R * (NC + (NC + NF if NF else 0))  # network samples of the step
    flops = 2.0 * (2 * MACS_8x256 + MACS_8x256_DINPUT) * S
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    dt_name = "bf16" if dtype else "f32"
    out_rec = {
        "metric": ("training rays/s, coarse 64 + fine 128 samples, two 8x256 networks (MFMA util %)" if NF else
                   "training rays/s, one network pass (8x256, 64 samples per ray; MFMA util %)"),
        "value": R / (ms_step * 1e-3), "unit": "rays/s", "samples_per_sec": S / (ms_step * 1e-3), "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt_name,
        "data": "synthetic: 4096 seeded random rays of 8 hemisphere poses at 400x400, random target colours, "
                "He-uniform random weights",
        "config": {"workload": args.workload, "rays": R, "n_coarse": NC, "n_fine": NF, "net": "8x256",
                   "networks": len(state), "optimizer": "Adam"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK[dt_name], "unit": "TFLOP/s",
                     "frac": achieved / PEAK[dt_name],
                     "traffic": measured_traffic("train", dt_name) if not NF else None,
                     "kernel": "whole step (every kernel)",
                     "kernel_ms": ms_kernel, "flop_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        from oracle import backward as obwd
        o_h, d_h = ro.cpu().numpy(), rd.cpu().numpy()
        n_h, f_h = near.cpu().numpy(), far.cpu().numpy()
        mode = "bf16" if dtype else "f64"
        if NF:
            fn = (lambda s_: obwd.hierarchical_train_step(nets_h[0], nets_h[1], o_h[s_], d_h[s_], n_h[s_], f_h[s_],
                                                          tgt_h[s_], NC, NF, 10, 4, seed=0, mode=mode,
                                                          ray_offset=s_))
        else:
            fn = (lambda s_: obwd.train_loss_and_grads(nets_h[0], o_h[s_], d_h[s_], n_h[s_], f_h[s_], tgt_h[s_], NC,
                                                       10, 4, seed=0, mode=mode, ray_offset=s_))
        out_rec["cpu_baseline"] = _cpu_rate(fn, R, args.cpu_seconds, "rays/s", "rays (loss and every gradient)")
    print(json.dumps(out_rec), flush=True)


def sweep_bench(args, wl):
    """The page's pose-sweep video: every frame of a 360 degree sweep rendered
    with the hierarchical sampler and the two 8x256 networks on a white
    background (nerf_render_poses), against the MFMA roofline of the render."""
    import torch
    import seeded_inputs as si
    import volume_rendering_amd as v
    from volume_rendering_amd import _binding as B

    dev = torch.device("cuda")
    n, H, W, f, NC, NF = wl["frames"], wl["H"], wl["W"], wl["focal"], wl["nc"], wl["nf"]
    dtype = 1 if args.dtype == "bf16" else 0
    dt_name = "bf16" if dtype else "f32"
    P = si.sweep_poses(n, elevation_deg=30.0)
    pc = si.nerf_params(si.NERF_8x256, seed=0, net_id=0)
    pf = si.nerf_params(si.NERF_8x256, seed=0, net_id=1)
    nets = [v.weights.pack_to_device(1, dtype, pc), v.weights.pack_to_device(1, dtype, pf)]
    w = B.nerf_weights(net=B.nerf_mlp_desc(1, dtype), coarse=nets[0].data_ptr(), fine=nets[1].data_ptr())
    cfg = B.nerf_render_cfg(mode=B.NERF_MODE_NERF, n_coarse=NC, n_fine=NF, use_pi=1, white_bkgd=1, jitter=1, seed=0)
    R = H * W
    rgb = torch.empty((n, R, 3), device=dev)
    depth = torch.empty((n, R), device=dev)
    acc = torch.empty((n, R), device=dev)
    ws = torch.empty(32 * R, dtype=torch.uint8, device=dev)

    def step():
        v.nerf_render_poses(P, W, H, f, f, 0.5 * W, 0.5 * H, 2.0, 6.0, w, cfg, rgb, depth, acc, workspace=ws)

    ms_step, ms_kernel = _timed(args, step, torch)
    rays = n * R
    flops = 2.0 * MACS_8x256 * rays * (NC + NC + NF)
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    out = {
        "metric": "pose-sweep frames/s (24 frames, 400x400, coarse64+fine128, 8x256, white background; MFMA util %)",
        "value": n / (ms_step * 1e-3), "unit": "frames/s", "rays_per_sec": rays / (ms_step * 1e-3), "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt_name,
        "data": "synthetic: seeded sweep poses, He-uniform random weights",
        "config": {"workload": args.workload, "frames": n, "H": H, "W": W, "focal": f, "n_coarse": NC,
                   "n_fine": NF, "net": "8x256", "white_bkgd": 1},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK[dt_name], "unit": "TFLOP/s",
                     "frac": achieved / PEAK[dt_name], "traffic": None, "kernel": "k_render_nerf (every frame)",
                     "kernel_ms": ms_kernel, "flop_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        from oracle import rays as orays
        o_l, d_l = zip(*[orays.get_rays(H, W, f, f, 0.5 * W, 0.5 * H, P[k]) for k in range(n)])
        ro, rd = np.concatenate(o_l), np.concatenate(d_l)
        near, far = np.full(rays, 2.0, np.float32), np.full(rays, 6.0, np.float32)
        rec = cpu_baseline(dict(wl, poses=n), 1, ro, rd, near, far, pc, pf, args.cpu_seconds)
        for r in (rec, rec.get("single_thread", {})):
            if "value" in r:
                r["value"] /= R  # rays/s -> frames/s
                r["unit"] = "frames/s"
        out["cpu_baseline"] = rec
    print(json.dumps(out), flush=True)


def inr_bench(args, wl):
    """Full-batch training steps of the hash-grid INR (nerf_hash_inr_train_step:
    lookups, decoder forward and backward, table gradients, decoder
    gradients, loss, Adam over every parameter), against the vector-ALU
    roofline: per point 2 FLOP for each multiply-add of the decoder forward
    (H F + H O), backward (H O + H F) and weight gradients (H F + H + O H + O),
    and of the 4 corners x 2 features x L levels interpolation, gathered and
    scattered."""
    import torch
    import seeded_inputs as si
    import volume_rendering_amd as v
    from volume_rendering_amd import _binding as B

    dev = torch.device("cuda")
    res, L, T, H = wl["res"], wl["L"], wl["T"], wl["hidden"]
    O, F = 1, 2 * wl["L"]
    g = B.nerf_hashgrid_init(L, T, wl["nmin"], wl["nmax"], dim=2)
    cfg = B.nerf_hash_inr_cfg(hidden=H, n_out=O, lr=wl["lr"], beta1=0.9, beta2=0.999, eps=1e-8)
    sizes = [min(T, (int(g.res[l]) + 1) ** 2) for l in range(L)]
    tables, mlp = si.hash_inr_params(sizes, L, H, O, seed=1)
    flat = si.hash_inr_flat(tables, mlp)
    assert flat.size == B.nerf_hash_inr_param_count(g, cfg)
    coords, target = si.inr_target_image(res)
    n = coords.shape[0]
    x, t = torch.from_numpy(coords).to(dev), torch.from_numpy(target).to(dev)
    params = torch.from_numpy(flat).to(dev)
    m, vv = torch.zeros_like(params), torch.zeros_like(params)
    loss = torch.empty(1, device=dev)
    ws = torch.empty(v.nerf_hash_inr_workspace_size(g, cfg, n), dtype=torch.uint8, device=dev)
    it = [0]

    def step():
        it[0] += 1
        v.nerf_hash_inr_train_step(x, t, g, cfg, params, loss, m, vv, it[0], workspace=ws)

    ms_step, ms_kernel = _timed(args, step, torch)
    flop_point = 2 * (H * F + H * O + H * O + H * F + H * F + H + O * H + O) + 2 * 2 * (4 * F)
    flops = float(flop_point) * n
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    peak = PEAK["f32"]
    out_rec = {
        "metric": "hash-grid INR training points/s (one full-batch Adam step; vector-ALU roofline %)",
        "value": n / (ms_step * 1e-3), "unit": "points/s", "steps_per_sec": 1e3 / ms_step, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic: the seeded {res}x{res} test image (sines, stripes, a disk), seeded U(+-1e-4) tables "
                "and U(+-1/sqrt(fan_in)) decoder",
        "config": {"workload": args.workload, "points": n, "levels": L, "table_size": T, "n_min": wl["nmin"],
                   "n_max": wl["nmax"], "hidden": H, "params": int(flat.size), "optimizer": "Adam", "lr": wl["lr"]},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(args.workload, "f32"), "kernel": "whole step (every kernel)",
                     "kernel_ms": ms_kernel, "flop_per_launch": flops, "flop_per_point": flop_point},
        "final_loss": float(loss.item()),
    }
    if not args.no_cpu_baseline:
        from oracle import backward as obwd
        from oracle import encoding, hash_inr
        og = encoding.HashGrid(2, L, T, wl["nmin"], wl["nmax"])
        pf = flat.astype(np.float64)
        z = np.zeros_like(pf)

        def fn(sel):
            _, _, dt, dm = hash_inr.forward_backward(og, tables, mlp, coords[sel], target[sel])
            obwd.adam(pf, hash_inr.flatten(dt, dm), z, z, 1, wl["lr"])

        out_rec["cpu_baseline"] = _cpu_rate(fn, n, args.cpu_seconds, "points/s",
                                            "points (forward, every gradient, Adam over all parameters)")
    print(json.dumps(out_rec), flush=True)


if __name__ == "__main__":
    main()

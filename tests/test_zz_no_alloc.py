"""nerf_render_noalloc, the render for callers that cannot allocate, against
nerf_render on the same inputs through the C ABI: the many-network render
(the only mode with a workspace) gives bit-identical outputs and live-sample
counts on two calls in a row, the second with fewer rays, and chunks larger
than the fixed scratch are refused."""
import numpy as np
import pytest

import seeded_inputs as si
from tests.gpu_util import dev, empty, host, page_rays, say, torch_cuda

pytestmark = pytest.mark.gpu


def _scene(v, dtype):
    stacked = si.cell_params_stacked(4096, seed=0)
    cells = v.weights.pack_many_to_device(3, dtype, [si.cell_slice(stacked, c) for c in range(4096)])
    occ = dev(si.occupancy_bits(128, 0.1, seed=0).view(np.int32))
    return cells, occ


def _render(v, torch, fn, o, d, cells, occ, dtype, chunk=0, workspace=None):
    import volume_rendering_amd._binding as B
    R = o.shape[0]
    nlive = torch.zeros(1, dtype=torch.int64, device="cuda")
    cfg = B.nerf_render_cfg(mode=2, n_coarse=192, use_pi=1, jitter=1, seed=0, chunk=chunk, term_T=1e-2,
                            box_lo=-1.5, box_hi=1.5, occ_res=128, cell_res=16, occ=occ.data_ptr(),
                            dbg_n_live=nlive.data_ptr())
    if workspace is not None:
        cfg.workspace, cfg.workspace_bytes = workspace.data_ptr(), workspace.numel()
    w = B.nerf_weights(net=B.nerf_mlp_desc(3, dtype), cells=cells.data_ptr(), n_cells=4096)
    near = torch.full((R,), 2.0, device="cuda")
    far = torch.full((R,), 6.0, device="cuda")
    rgb, depth, acc = empty((R, 3)), empty(R), empty(R)
    fn(dev(o), dev(d), near, far, w, cfg, rgb, depth, acc)
    return host(rgb), host(depth), host(acc), int(host(nlive)[0])


@pytest.mark.parametrize("dtype", [0, 1])
def test_noalloc_matches_render_on_two_calls(dtype):
    torch = torch_cuda()
    import volume_rendering_amd as v
    pose = si.poses(1, seed=0)[0]
    o_all, d_all = page_rays(800, 800, 1110.0, pose)
    cells, occ = _scene(v, dtype)
    # 60,000 rays need several chunks of the fixed scratch; then 3,001 rays, one chunk
    for R, seed in ((60000, 21), (3001, 22)):
        say(f"noalloc dtype={dtype} rays={R}")
        sel = si.subset(800 * 800, R, seed=seed)
        o, d = o_all[sel], d_all[sel]
        ref = _render(v, torch, v.nerf_render, o, d, cells, occ, dtype)
        got = _render(v, torch, v.nerf_render_noalloc, o, d, cells, occ, dtype)
        for a, b in zip(ref[:3], got[:3]):
            assert np.array_equal(a, b)
        assert ref[3] == got[3] and ref[3] > 0
        say(f"  identical: {R} rays, {got[3]} live samples")


def test_noalloc_refuses_what_does_not_fit():
    torch = torch_cuda()
    import volume_rendering_amd as v
    pose = si.poses(1, seed=0)[0]
    o, d = page_rays(200, 150, 200.0, pose)  # 30,000 rays: one chunk of them needs ~178 MiB
    cells, occ = _scene(v, 0)
    with pytest.raises(v.NerfError, match="NERF_ERR_WORKSPACE"):
        _render(v, torch, v.nerf_render_noalloc, o, d, cells, occ, 0, chunk=30000)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(v.NerfError, match="workspace must be NULL"):
        _render(v, torch, v.nerf_render_noalloc, o, d, cells, occ, 0, workspace=ws)

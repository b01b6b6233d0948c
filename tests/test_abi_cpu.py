"""Host-side checks of the C ABI library (no GPU needed): it loads, exports
every declared symbol, validates arguments before touching the device, lays
out hash grids and packs weights as documented."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import seeded_inputs as si
import volume_rendering_amd as v
from volume_rendering_amd import _binding as B
from oracle import encoding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(nerf_[a-z0-9_]+)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    L = v.lib()
    names = declared_symbols()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert set(B.EXPORTED) == names


def test_checked_library_exports_the_same_symbols():
    """The normal library has no index checks (nerf_check_flags returns -1
    without touching a device); the checked one, built from the same sources
    with -DNERF_CHECK, exports every declared symbol too."""
    assert v.nerf_check_flags() == -1
    path = os.path.join(ROOT, "volume_rendering_amd", "libnerf_mi355x_checked.so")
    assert os.path.exists(path), "build both libraries: python -m volume_rendering_amd.build"
    L = C.CDLL(path)
    for n in declared_symbols():
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = v.lib()
    assert v.nerf_abi_version() == 2
    assert L.nerf_status_str(0) == b"NERF_OK"
    assert L.nerf_status_str(3) == b"NERF_ERR_WORKSPACE"


def test_hashgrid_init_matches_oracle_layout():
    for T, Lv, nmin, nmax in ((2 ** 19, 16, 16, 2048), (2 ** 12, 8, 8, 160), (2 ** 8, 8, 8, 160)):
        g = v.nerf_hashgrid_init(Lv, T, nmin, nmax)
        og = encoding.HashGrid(3, Lv, T, nmin, nmax)
        assert list(g.res)[:Lv] == og.res
        assert [bool(d) for d in list(g.direct)[:Lv]] == og.direct
        assert list(g.size)[:Lv] == og.sizes
        assert g.total_entries == sum(og.sizes)
        assert list(g.offset)[:Lv] == list(np.cumsum([0] + og.sizes[:-1]))


def test_hashgrid_init_2d_reproduces_the_printed_tables(golden_dir):
    # Experiment 1 (T = 2^12) and Experiment 4 (T = 2^8, 2^14), 8 levels from 8 to 160
    rows = [l.split() for l in open(os.path.join(golden_dir, "hashgrid2d_experiment1.txt")) if l[0] != "#"]
    g = v.nerf_hashgrid_init(8, 2 ** 12, 8, 160, dim=2)
    assert g.dim == 2 and list(g.level_mask)[:8] == [1.0] * 8
    assert list(g.res)[:8] == [int(r[1]) for r in rows]
    assert [bool(d) for d in list(g.direct)[:8]] == [r[3] == "direct" for r in rows]
    assert list(g.size)[:8] == [min(int(r[2]), 2 ** 12) for r in rows]
    for r in (l.split() for l in open(os.path.join(golden_dir, "hashgrid2d_experiment4.txt")) if l[0] != "#"):
        T, n_hash, L = map(int, r)
        g = v.nerf_hashgrid_init(L, T, 8, 160, dim=2)
        assert sum(not d for d in list(g.direct)[:L]) == n_hash


def test_hashgrid_init_rejects_bad_arguments():
    for args in ((1, 2 ** 19, 16, 2048), (17, 2 ** 19, 16, 2048), (16, 3000, 16, 2048), (16, 2 ** 19, 0, 10),
                 (16, 2 ** 19, 20, 10)):
        with pytest.raises(v.NerfError, match="INVALID_ARGUMENT"):
            v.nerf_hashgrid_init(*args)
    with pytest.raises(v.NerfError, match="INVALID_ARGUMENT"):
        v.nerf_hashgrid_init(16, 2 ** 19, 16, 2048, dim=4)


def _unpack_layer(buf, kind, prec, li, layers, n_in):
    """Reads layer li back out of a packed buffer using the layout the
    header and nets.hpp document (tile = 64 lanes, bf16: 8 values/lane)."""
    # the tile/bias offsets are recomputed here from the documented rules
    def steps(seg):
        kindc, width, L = seg
        ob = -(-width // 32)
        if kindc == "H":
            return (2 if prec else 16) * ob
        if kindc == "E":
            pairs = 3 * L + 2
            return -(-pairs // 8) if prec else 16 * (-(-pairs // 16))
        if kindc == "F":
            return -(-width // 16) if prec else -(-width // 2)
        return 0

    def tiles(l):
        return -(-l[0] // 32) * (steps(l[1]) + steps(l[2]))

    tb = 1024 if prec else 256
    off = sum(tiles(layers[i]) for i in range(li)) * tb
    n_out, s0, s1 = layers[li]
    S1, S2 = steps(s0), steps(s1)
    W = np.full((-(-n_out // 32) * 32, n_in), np.nan)
    t = 0
    for ob in range(-(-n_out // 32)):
        for st in range(S1 + S2):
            seg, sst, base = (s0, st, 0) if st < S1 else (s1, st - S1, s0[1])
            for lane in range(64):
                row, h = 32 * ob + lane % 32, lane // 32
                for j in range(8 if prec else 1):
                    if prec:
                        raw = buf[off + t * 1024 + lane * 16 + 2 * j: off + t * 1024 + lane * 16 + 2 * j + 2]
                        val = np.frombuffer(b"\0\0" + raw.tobytes(), dtype=np.float32)[0]
                    else:
                        val = np.frombuffer(buf[off + t * 256 + lane * 4: off + t * 256 + lane * 4 + 4].tobytes(),
                                            dtype=np.float32)[0]
                    c = _col(seg, prec, sst, h, j)
                    if c >= 0 and row < n_out:
                        W[row, base + c] = val
                    else:
                        assert val == 0.0
            t += 1
    return W[:n_out]


def _col(seg, prec, step, h, j):
    kindc, width, L = seg
    if kindc == "H":
        if prec:
            n = 32 * (step // 2) + 8 * (2 * (step % 2) + j // 4) + 4 * h + (j % 4)
        else:
            n = 32 * (step // 16) + 8 * ((step % 16) // 4) + 4 * h + (step % 4)
        return n if n < width else -1
    if kindc == "E":
        P, comp = (8 * step + 4 * h + j // 2, j % 2) if prec else (2 * (step // 2) + h, step % 2)
        if P < 3 * L:
            return 3 + 6 * (P // 3) + 3 * comp + P % 3
        if P == 3 * L:
            return comp
        if P == 3 * L + 1 and comp == 0:
            return 2
        return -1
    f = 16 * step + 8 * h + j if prec else 2 * step + h
    return f if f < width else -1


LAYERS_4x64 = [(64, ("E", 39, 6), ("N", 0, 0)), (64, ("H", 64, 0), ("N", 0, 0)), (64, ("H", 64, 0), ("N", 0, 0)),
               (64, ("H", 64, 0), ("N", 0, 0)), (1, ("H", 64, 0), ("N", 0, 0)), (64, ("H", 64, 0), ("N", 0, 0)),
               (32, ("H", 64, 0), ("E", 27, 4)), (3, ("H", 32, 0), ("N", 0, 0))]


@pytest.mark.parametrize("prec", [0, 1])
def test_pack_roundtrip_tiny_net(prec):
    from oracle.mlp import round_bf16
    p = si.nerf_params(si.NERF_4x64, seed=3)
    buf = v.weights.pack(B.NERF_NET_4x64, prec, p)
    arrs = v.weights.forward_order(p)
    for li in range(8):
        Wref = arrs[2 * li]
        W = _unpack_layer(buf, B.NERF_NET_4x64, prec, li, LAYERS_4x64, Wref.shape[1])
        expect = round_bf16(Wref) if prec else Wref.astype(np.float64)
        assert np.array_equal(W, expect), li


def test_pack_rejects_bad_arguments():
    p = si.nerf_params(si.NERF_4x64, seed=3)
    arrs = v.weights.forward_order(p)
    with pytest.raises(v.NerfError, match="INVALID_ARGUMENT"):
        B.nerf_pack_mlp(B.NERF_NET_4x64, 0, arrs[:-2])
    with pytest.raises(v.NerfError):
        B.nerf_pack_mlp(99, 0, arrs)
    assert B.nerf_mlp_packed_bytes(99, 0) == 0


def test_validation_errors_before_any_launch():
    L = v.lib()
    # NULL weights/cfg
    assert L.nerf_render(None, None, None, None, 10, None, None, None, None, None, None) == 1
    cfg = B.nerf_render_cfg(mode=0, n_coarse=300)
    w = B.nerf_weights(net=B.nerf_mlp_desc(1, 1))
    assert L.nerf_render(None, None, None, None, 10, C.byref(w), C.byref(cfg), None, None, None, None) == 1
    assert b"n_coarse" in L.nerf_last_error()
    cfg = B.nerf_render_cfg(mode=0, n_coarse=64, n_fine=128)
    assert L.nerf_render(None, None, None, None, 10, C.byref(w), C.byref(cfg), None, None, None, None) == 1
    w = B.nerf_weights(net=B.nerf_mlp_desc(3, 0))
    assert L.nerf_render(None, None, None, None, 10, C.byref(w), C.byref(cfg), None, None, None, None) == 2
    assert L.nerf_sample_pdf(None, None, 4, 2, 8, 0, 0, None, None, None, None) == 1
    assert L.nerf_sample_pdf(None, None, 4, 200, 100, 0, 0, None, None, None, None) == 1
    assert L.nerf_sample_stratified(None, None, 4, 0, 0, 0, 1, None, None) == 1
    assert L.nerf_encode_freq(None, 4, 3, 20, 1, 1, 0, None, None) == 1
    assert L.nerf_composite(None, None, None, 4, 0, 0, None, None, None, None, None) == 1
    # empty inputs are accepted without launching anything
    assert L.nerf_sample_stratified(None, None, 0, 16, 0, 0, 1, None, None) == 0
    assert L.nerf_composite(None, None, None, 0, 64, 0, None, None, None, None, None) == 0
    assert L.nerf_sample_pdf(None, None, 0, 64, 128, 0, 0, None, None, None, None) == 0


def test_render_poses_validation():
    L = v.lib()
    K = B.nerf_intrinsics(8, 8, 10.0, 10.0, 4.0, 4.0)
    cfg = B.nerf_render_cfg(mode=0, n_coarse=16)
    w = B.nerf_weights(net=B.nerf_mlp_desc(2, 0))
    # no poses: nothing to do
    assert L.nerf_render_poses(None, 0, C.byref(K), 2.0, 6.0, C.byref(w), C.byref(cfg), None, 0, None, None, None,
                               None) == 0
    # debug outputs are refused, before anything is launched
    cfg.dbg_z = 16
    assert L.nerf_render_poses(None, 2, C.byref(K), 2.0, 6.0, C.byref(w), C.byref(cfg), None, 0, None, None, None,
                               None) == 1
    assert b"debug outputs" in L.nerf_last_error()
    cfg.dbg_z = None
    assert L.nerf_render_poses(None, 2, C.byref(K), 2.0, 6.0, C.byref(w), C.byref(cfg), None, 0, None, None, None,
                               None) == 1
    bad = B.nerf_intrinsics(0, 8, 10.0, 10.0, 4.0, 4.0)
    assert L.nerf_render_poses(None, 2, C.byref(bad), 2.0, 6.0, C.byref(w), C.byref(cfg), None, 0, None, None, None,
                               None) == 1


def test_sweep_poses_look_at_the_origin():
    P = si.sweep_poses(24, elevation_deg=30.0, radius=4.0)
    assert P.shape == (24, 3, 4)
    for p in P:
        t = p[:, 3].astype(np.float64)
        assert abs(np.linalg.norm(t) - 4.0) < 1e-5 and abs(t[2] - 2.0) < 1e-5  # 4 sin 30
        # the camera looks down its -z axis: the third column points away from the origin
        assert np.allclose(p[:, 2], t / 4.0, atol=1e-6)


def test_train_param_count_and_validation():
    L = v.lib()
    for kind, shape in [(1, si.NERF_8x256), (2, si.NERF_4x64), (3, si.NERF_CELL_2x32)]:
        assert B.nerf_train_param_count(kind) == shape.n_params()
        assert si.flat_params(si.nerf_params(shape)).size == shape.n_params()
    assert B.nerf_train_param_count(4) == 0  # the hash field is not trained here
    cfg = B.nerf_train_cfg(net=B.nerf_mlp_desc(2, 0), n_samples=32, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    need = B.nerf_train_workspace_size(cfg, 1000)
    assert need > 1000 * 32 * 4
    assert B.nerf_train_workspace_size(cfg, 2000) > need
    P = C.c_void_p(256)  # never dereferenced: every call below fails validation first
    args = [P] * 5

    def call(n_rays, c, m=P, vv=P, step=1, ws=None, wsb=0, params=P, loss=P):
        return L.nerf_train_step(*args, n_rays, C.byref(c), params, m, vv, step, None, loss, None, ws, wsb, None)

    assert call(0, cfg) == 0  # no rays: nothing to do
    assert call(1000, cfg, ws=P, wsb=need - 1) == 3
    assert b"workspace" in L.nerf_last_error()
    assert call(1000, cfg, m=None) == 1  # one Adam moment without the other
    assert call(1000, cfg, step=0) == 1
    assert call(1000, cfg, params=None) == 1
    bad = B.nerf_train_cfg(net=B.nerf_mlp_desc(2, 0), n_samples=300)
    assert call(1000, bad) == 1 and b"n_samples" in L.nerf_last_error()
    hashnet = B.nerf_train_cfg(net=B.nerf_mlp_desc(4, 0), n_samples=32)
    assert call(1000, hashnet) == 2
    assert call(1 << 24, cfg) == 2  # 2^28 samples at most
    assert B.nerf_train_workspace_size(hashnet, 10) == 0


def test_hash_inr_param_count_and_validation():
    from oracle import encoding
    L = v.lib()
    g = B.nerf_hashgrid_init(8, 2 ** 12, 8, 160, dim=2)
    og = encoding.HashGrid(2, 8, 2 ** 12, 8, 160)
    cfg = B.nerf_hash_inr_cfg(hidden=32, n_out=1, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8)
    tables, mlp = si.hash_inr_params(og.sizes, og.L, 32, 1)
    assert B.nerf_hash_inr_param_count(g, cfg) == si.hash_inr_flat(tables, mlp).size
    assert B.nerf_hash_inr_param_count(g, cfg) == 2 * sum(og.sizes) + 32 * 16 + 32 + 32 + 1  # 577 decoder params
    # the feature gradients (2 floats per level and point) plus partial sums:
    # one table partial per chunk of at least 4096 points
    tab = 2 * sum(og.sizes)
    ws = B.nerf_hash_inr_workspace_size(g, cfg, 9216)
    assert 9216 * 16 * 4 + 3 * tab * 4 <= ws < 9216 * 16 * 4 + 3 * tab * 4 + (1 << 20)
    ws1, ws2 = (B.nerf_hash_inr_workspace_size(g, cfg, n) for n in (1 << 22, 1 << 23))
    assert ws2 - ws1 >= (1 << 22) * 16 * 4
    assert B.nerf_hash_inr_workspace_size(g, cfg, (1 << 27) + 1) > 0  # sized; the step itself refuses it
    bad = B.nerf_hash_inr_cfg(hidden=65, n_out=1)
    assert B.nerf_hash_inr_param_count(g, bad) == 0
    P = C.c_void_p(256)
    # no points: nothing to do; the grid's tables pointer is not needed
    assert L.nerf_hash_inr_train_step(None, None, 0, C.byref(g), C.byref(cfg), None, None, None, 0, None, None, None,
                                      None, 0, None) == 0
    assert L.nerf_hash_inr_train_step(P, P, 10, C.byref(g), C.byref(bad), P, None, None, 0, None, P, None, None, 0,
                                      None) == 1
    assert L.nerf_hash_inr_train_step(P, P, 10, C.byref(g), C.byref(cfg), P, P, None, 1, None, P, None, None, 0,
                                      None) == 1  # one Adam moment
    assert L.nerf_hash_inr_train_step(P, P, (1 << 27) + 1, C.byref(g), C.byref(cfg), P, None, None, 0, None, P, None,
                                      None, 0, None) == 1
    assert L.nerf_hash_inr_train_step(C.c_void_p(264), P, 10, C.byref(g), C.byref(cfg), P, None, None, 0, None, P,
                                      None, None, 0, None) == 1  # x not 16-byte aligned
    need = B.nerf_hash_inr_workspace_size(g, cfg, 10)
    assert L.nerf_hash_inr_train_step(P, P, 10, C.byref(g), C.byref(cfg), P, None, None, 0, None, P, None, P,
                                      need - 1, None) == 3

"""ctypes binding of libnerf_mi355x.so.

Argument marshalling only: tensors are passed as device pointers with the
current HIP stream; every step of the render runs in the library's kernels.
The functions carry the C names.  The library is loaded from this package
directory (built in-tree by ``volume_rendering_amd.build``); a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnerf_mi355x.so")
_lib = None

NERF_OK = 0
NERF_F32, NERF_BF16 = 0, 1
NERF_NET_8x256, NERF_NET_4x64, NERF_NET_CELL_2x32, NERF_NET_HASH_FIELD = 1, 2, 3, 4
NERF_MODE_NERF, NERF_MODE_HASH, NERF_MODE_KILO = 0, 1, 2
HASH_MAX_LEVELS = 16

EXPORTED = [
    "nerf_abi_version", "nerf_status_str", "nerf_last_error", "nerf_hashgrid_init", "nerf_mlp_packed_bytes",
    "nerf_pack_mlp", "nerf_gen_rays", "nerf_sample_stratified", "nerf_encode_freq", "nerf_encode_sh16",
    "nerf_encode_hashgrid", "nerf_mlp", "nerf_composite", "nerf_sample_pdf", "nerf_render",
    "nerf_render_workspace_size", "nerf_render_noalloc", "nerf_render_poses", "nerf_train_param_count",
    "nerf_train_workspace_size", "nerf_train_step", "nerf_hash_inr_param_count", "nerf_hash_inr_workspace_size",
    "nerf_hash_inr_train_step", "nerf_check_flags",
]


class NerfError(RuntimeError):
    pass


class nerf_intrinsics(C.Structure):
    _fields_ = [("W", C.c_int32), ("H", C.c_int32), ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float),
                ("cy", C.c_float)]


class nerf_mlp_desc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("dtype", C.c_int32)]


class nerf_hashgrid(C.Structure):
    _fields_ = [("n_levels", C.c_int32), ("n_feat", C.c_int32), ("table_size", C.c_uint32),
                ("res", C.c_int32 * HASH_MAX_LEVELS), ("direct", C.c_int32 * HASH_MAX_LEVELS),
                ("size", C.c_uint32 * HASH_MAX_LEVELS), ("offset", C.c_uint64 * HASH_MAX_LEVELS),
                ("total_entries", C.c_uint64), ("tables", C.c_void_p), ("dim", C.c_int32),
                ("level_mask", C.c_float * HASH_MAX_LEVELS)]


class nerf_weights(C.Structure):
    _fields_ = [("net", nerf_mlp_desc), ("coarse", C.c_void_p), ("fine", C.c_void_p), ("cells", C.c_void_p),
                ("n_cells", C.c_int32), ("grid", C.POINTER(nerf_hashgrid))]


class nerf_render_cfg(C.Structure):
    _fields_ = [("mode", C.c_int32), ("n_coarse", C.c_int32), ("n_fine", C.c_int32), ("use_pi", C.c_int32),
                ("white_bkgd", C.c_int32), ("jitter", C.c_int32), ("seed", C.c_uint64), ("ray_offset", C.c_uint64),
                ("chunk", C.c_int64), ("term_T", C.c_float), ("box_lo", C.c_float), ("box_hi", C.c_float),
                ("occ_res", C.c_int32), ("cell_res", C.c_int32), ("occ", C.c_void_p), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("dbg_z", C.c_void_p), ("dbg_w_coarse", C.c_void_p),
                ("dbg_n_live", C.c_void_p)]


class nerf_train_cfg(C.Structure):
    _fields_ = [("net", nerf_mlp_desc), ("n_samples", C.c_int32), ("use_pi", C.c_int32), ("white_bkgd", C.c_int32),
                ("jitter", C.c_int32), ("seed", C.c_uint64), ("ray_offset", C.c_uint64), ("lr", C.c_float),
                ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float), ("z", C.c_void_p),
                ("weights", C.c_void_p)]


class nerf_hash_inr_cfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_out", C.c_int32), ("lr", C.c_float), ("beta1", C.c_float),
                ("beta2", C.c_float), ("eps", C.c_float)]


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise NerfError(f"{_LIB_PATH} is missing: build it with `python -m volume_rendering_amd.build`")
        L = C.CDLL(_LIB_PATH)
        P, I, I64, U64, S = C.c_void_p, C.c_int, C.c_int64, C.c_uint64, C.c_size_t
        sig = {
            "nerf_abi_version": (I, []),
            "nerf_check_flags": (I64, []),
            "nerf_status_str": (C.c_char_p, [I]),
            "nerf_last_error": (C.c_char_p, []),
            "nerf_hashgrid_init": (I, [C.POINTER(nerf_hashgrid), I, I, C.c_uint32, I, I]),
            "nerf_mlp_packed_bytes": (S, [C.POINTER(nerf_mlp_desc)]),
            "nerf_pack_mlp": (I, [C.POINTER(nerf_mlp_desc), C.POINTER(C.c_void_p), I, P, S]),
            "nerf_gen_rays": (I, [P, C.POINTER(nerf_intrinsics), P, P, P]),
            "nerf_sample_stratified": (I, [P, P, I64, I, U64, U64, I, P, P]),
            "nerf_encode_freq": (I, [P, I64, I, I, I, I, I, P, P]),
            "nerf_encode_sh16": (I, [P, I64, P, P]),
            "nerf_encode_hashgrid": (I, [P, I64, C.POINTER(nerf_hashgrid), P, P, P]),
            "nerf_mlp": (I, [C.POINTER(nerf_mlp_desc), P, P, P, I64, I, P, P]),
            "nerf_composite": (I, [P, P, P, I64, I, I, P, P, P, P, P]),
            "nerf_sample_pdf": (I, [P, P, I64, I, I, U64, U64, P, P, P, P]),
            "nerf_render": (I, [P, P, P, P, I64, C.POINTER(nerf_weights), C.POINTER(nerf_render_cfg), P, P, P, P]),
            "nerf_render_workspace_size": (S, [C.POINTER(nerf_render_cfg), I64]),
            "nerf_render_noalloc": (I, [P, P, P, P, I64, C.POINTER(nerf_weights), C.POINTER(nerf_render_cfg), P, P,
                                        P, P]),
            "nerf_render_poses": (I, [P, I, C.POINTER(nerf_intrinsics), C.c_float, C.c_float, C.POINTER(nerf_weights),
                                      C.POINTER(nerf_render_cfg), P, S, P, P, P, P]),
            "nerf_train_param_count": (I64, [I]),
            "nerf_train_workspace_size": (S, [C.POINTER(nerf_train_cfg), I64]),
            "nerf_train_step": (I, [P, P, P, P, P, I64, C.POINTER(nerf_train_cfg), P, P, P, I64, P, P, P, P, S, P]),
            "nerf_hash_inr_param_count": (I64, [C.POINTER(nerf_hashgrid), C.POINTER(nerf_hash_inr_cfg)]),
            "nerf_hash_inr_workspace_size": (S, [C.POINTER(nerf_hashgrid), C.POINTER(nerf_hash_inr_cfg), I64]),
            "nerf_hash_inr_train_step": (I, [P, P, I64, C.POINTER(nerf_hashgrid), C.POINTER(nerf_hash_inr_cfg), P, P, P,
                                             I64, P, P, P, P, S, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != NERF_OK:
        L = lib()
        raise NerfError(f"{what}: {L.nerf_status_str(status).decode()}: {L.nerf_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise NerfError("tensor must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ----------------------------------------------------------------------------
# Host helpers
# ----------------------------------------------------------------------------

def nerf_abi_version() -> int:
    return lib().nerf_abi_version()


def nerf_check_flags() -> int:
    """Failed index-check bits since the last call (checked library), or -1."""
    return int(lib().nerf_check_flags())


def nerf_hashgrid_init(n_levels=16, table_size=2 ** 19, n_min=16, n_max=2048, dim=3) -> nerf_hashgrid:
    g = nerf_hashgrid()
    _check(lib().nerf_hashgrid_init(C.byref(g), dim, n_levels, table_size, n_min, n_max), "nerf_hashgrid_init")
    return g


def nerf_mlp_packed_bytes(kind: int, dtype: int) -> int:
    d = nerf_mlp_desc(kind, dtype)
    return lib().nerf_mlp_packed_bytes(C.byref(d))


def nerf_pack_mlp(kind: int, dtype: int, tensors) -> np.ndarray:
    """Packs float32 host arrays (forward order: W_0, b_0, ...) into the
    device layout; returns a uint8 host array for the caller to upload."""
    d = nerf_mlp_desc(kind, dtype)
    n = lib().nerf_mlp_packed_bytes(C.byref(d))
    if n == 0:
        raise NerfError(f"unsupported network kind {kind} / dtype {dtype}")
    arrs = [np.ascontiguousarray(t, dtype=np.float32) for t in tensors]
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = np.zeros(n, dtype=np.uint8)
    _check(lib().nerf_pack_mlp(C.byref(d), ptrs, len(arrs), out.ctypes.data, n), "nerf_pack_mlp")
    return out


def nerf_render_workspace_size(cfg: nerf_render_cfg, n_rays: int) -> int:
    return lib().nerf_render_workspace_size(C.byref(cfg), n_rays)


# ----------------------------------------------------------------------------
# Device steps (tensors are torch device tensors)
# ----------------------------------------------------------------------------

def nerf_gen_rays(pose: np.ndarray, W, H, fx, fy, cx, cy, rays_o, rays_d):
    K = nerf_intrinsics(W, H, fx, fy, cx, cy)
    p = np.ascontiguousarray(pose, dtype=np.float32).reshape(12)
    _check(lib().nerf_gen_rays(p.ctypes.data, C.byref(K), _ptr(rays_o), _ptr(rays_d), _stream()), "nerf_gen_rays")


def nerf_sample_stratified(t_near, t_far, n, seed, ray_offset, jitter, z):
    _check(lib().nerf_sample_stratified(_ptr(t_near), _ptr(t_far), t_near.numel(), n, seed, ray_offset,
                                        int(jitter), _ptr(z), _stream()), "nerf_sample_stratified")


def nerf_encode_freq(x, n_freq, include_input, use_pi, out_dtype, out):
    n, d = x.shape
    _check(lib().nerf_encode_freq(_ptr(x), n, d, n_freq, int(include_input), int(use_pi), out_dtype, _ptr(out),
                                  _stream()), "nerf_encode_freq")


def nerf_encode_sh16(dirs, out):
    _check(lib().nerf_encode_sh16(_ptr(dirs), dirs.shape[0], _ptr(out), _stream()), "nerf_encode_sh16")


def nerf_encode_hashgrid(x, grid: nerf_hashgrid, out, idx_dbg=None):
    _check(lib().nerf_encode_hashgrid(_ptr(x), x.shape[0], C.byref(grid), _ptr(out), _ptr(idx_dbg), _stream()),
           "nerf_encode_hashgrid")


def nerf_mlp(kind, dtype, packed, enc_x, enc_v, samples_per_ray, raw):
    d = nerf_mlp_desc(kind, dtype)
    _check(lib().nerf_mlp(C.byref(d), _ptr(packed), _ptr(enc_x), _ptr(enc_v), enc_x.shape[0], samples_per_ray,
                          _ptr(raw), _stream()), "nerf_mlp")


def nerf_composite(raw, z, rays_d, white_bkgd, rgb, depth, acc, weights=None):
    R, N = z.shape
    _check(lib().nerf_composite(_ptr(raw), _ptr(z), _ptr(rays_d), R, N, int(white_bkgd), _ptr(rgb), _ptr(depth),
                                _ptr(acc), _ptr(weights), _stream()), "nerf_composite")


def nerf_sample_pdf(z_coarse, w_coarse, n_fine, seed, ray_offset, z_fine=None, bin_idx=None, z_merged=None):
    R, Nc = z_coarse.shape
    _check(lib().nerf_sample_pdf(_ptr(z_coarse), _ptr(w_coarse), R, Nc, n_fine, seed, ray_offset, _ptr(z_fine),
                                 _ptr(bin_idx), _ptr(z_merged), _stream()), "nerf_sample_pdf")


def nerf_render(rays_o, rays_d, t_near, t_far, weights: nerf_weights, cfg: nerf_render_cfg, rgb, depth, acc):
    _check(lib().nerf_render(_ptr(rays_o), _ptr(rays_d), _ptr(t_near), _ptr(t_far), rays_o.shape[0],
                             C.byref(weights), C.byref(cfg), _ptr(rgb), _ptr(depth), _ptr(acc), _stream()),
           "nerf_render")


def nerf_render_noalloc(rays_o, rays_d, t_near, t_far, weights: nerf_weights, cfg: nerf_render_cfg, rgb, depth, acc):
    _check(lib().nerf_render_noalloc(_ptr(rays_o), _ptr(rays_d), _ptr(t_near), _ptr(t_far), rays_o.shape[0],
                                     C.byref(weights), C.byref(cfg), _ptr(rgb), _ptr(depth), _ptr(acc), _stream()),
           "nerf_render_noalloc")


def nerf_render_poses(poses: np.ndarray, W, H, fx, fy, cx, cy, t_near, t_far, weights: nerf_weights,
                      cfg: nerf_render_cfg, rgb, depth, acc, workspace=None):
    """One image per pose: ``poses`` host float32 [n, 3, 4]; rgb [n, H*W, 3],
    depth and acc [n, H*W] device tensors; ``workspace`` an optional device
    uint8 tensor of at least 32*W*H bytes."""
    K = nerf_intrinsics(W, H, fx, fy, cx, cy)
    p = np.ascontiguousarray(poses, dtype=np.float32).reshape(-1, 12)
    ws, wsb = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib().nerf_render_poses(p.ctypes.data, p.shape[0], C.byref(K), float(t_near), float(t_far),
                                   C.byref(weights), C.byref(cfg), ws, wsb, _ptr(rgb), _ptr(depth), _ptr(acc),
                                   _stream()), "nerf_render_poses")


# ----------------------------------------------------------------------------
# Training step
# ----------------------------------------------------------------------------

def nerf_train_param_count(kind: int) -> int:
    return lib().nerf_train_param_count(kind)


def nerf_train_workspace_size(cfg: nerf_train_cfg, n_rays: int) -> int:
    return lib().nerf_train_workspace_size(C.byref(cfg), n_rays)


def nerf_train_step(rays_o, rays_d, t_near, t_far, target_rgb, cfg: nerf_train_cfg, params, loss, adam_m=None,
                    adam_v=None, step=0, grad=None, rgb=None, workspace=None):
    """One training step; ``params`` (and the Adam moments) are float32
    device tensors updated in place, ``loss`` a float32 device tensor [1],
    ``workspace`` an optional device uint8 tensor.  ``cfg.z`` and
    ``cfg.weights`` are device pointers (``tensor.data_ptr()``) or None."""
    ws, wsb = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib().nerf_train_step(_ptr(rays_o), _ptr(rays_d), _ptr(t_near), _ptr(t_far), _ptr(target_rgb),
                                 rays_o.shape[0], C.byref(cfg), _ptr(params), _ptr(adam_m), _ptr(adam_v), int(step),
                                 _ptr(grad), _ptr(loss), _ptr(rgb), ws, wsb, _stream()), "nerf_train_step")


# ----------------------------------------------------------------------------
# Hash-grid INR training step
# ----------------------------------------------------------------------------

def nerf_hash_inr_param_count(grid: nerf_hashgrid, cfg: nerf_hash_inr_cfg) -> int:
    return lib().nerf_hash_inr_param_count(C.byref(grid), C.byref(cfg))


def nerf_hash_inr_workspace_size(grid: nerf_hashgrid, cfg: nerf_hash_inr_cfg, n: int) -> int:
    return lib().nerf_hash_inr_workspace_size(C.byref(grid), C.byref(cfg), n)


def nerf_hash_inr_train_step(x, target, grid: nerf_hashgrid, cfg: nerf_hash_inr_cfg, params, loss, adam_m=None,
                             adam_v=None, step=0, grad=None, pred=None, workspace=None):
    """One full-batch step of the hash-grid INR; ``params`` and the Adam
    moments are float32 device tensors updated in place."""
    ws, wsb = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib().nerf_hash_inr_train_step(_ptr(x), _ptr(target), x.shape[0], C.byref(grid), C.byref(cfg),
                                          _ptr(params), _ptr(adam_m), _ptr(adam_v), int(step), _ptr(grad),
                                          _ptr(loss), _ptr(pred), ws, wsb, _stream()), "nerf_hash_inr_train_step")

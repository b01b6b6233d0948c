"""Marshalling of network weights into the library's packed device layout.

A network's parameters are given as a dict of float32 arrays ``(W, b)``
with ``W`` row-major [out, in]:
  NeRF family:  layers (list), sigma, feature, dir, rgb
  hash field:   density (list of 2), sigma, feature, color (list of 2), rgb
The library's ``nerf_pack_mlp`` does the packing; this module only orders
the arrays and moves the packed bytes to the device.
"""
from __future__ import annotations

import numpy as np

from . import _binding as B


def forward_order(params: dict) -> list:
    """Weight and bias arrays in the order ``nerf_pack_mlp`` documents."""
    if "layers" in params:
        seq = list(params["layers"]) + [params[k] for k in ("sigma", "feature", "dir", "rgb")]
    else:
        seq = list(params["density"]) + [params["sigma"], params["feature"]] + list(params["color"]) + [params["rgb"]]
    out = []
    for W, b in seq:
        out += [np.asarray(W, dtype=np.float32), np.asarray(b, dtype=np.float32)]
    return out


def pack(kind: int, dtype: int, params: dict) -> np.ndarray:
    return B.nerf_pack_mlp(kind, dtype, forward_order(params))


def to_device(packed: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(packed).to(device)


def pack_to_device(kind: int, dtype: int, params: dict, device="cuda"):
    return to_device(pack(kind, dtype, params), device)


def pack_many_to_device(kind: int, dtype: int, param_list, device="cuda"):
    """Packs several networks of one kind back to back (cell networks)."""
    import torch
    stride = B.nerf_mlp_packed_bytes(kind, dtype)
    host = np.empty(stride * len(param_list), dtype=np.uint8)
    for i, p in enumerate(param_list):
        host[i * stride:(i + 1) * stride] = pack(kind, dtype, p)
    return torch.from_numpy(host).to(device)

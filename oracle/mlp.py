"""Radiance-field networks (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

``nerf_forward`` follows "Spatial Intelligence - Part 1: NeRF", Section 2
Code, 4. The NeRF network: ``depth`` Linear+ReLU layers on the position
encoding; after the layer whose index equals ``skip`` the position encoding
is concatenated after the hidden state (so the next layer sees
[h, gamma(x)]); a density head on the last hidden state; a feature layer
with no activation; a direction layer with ReLU on [feature, gamma(d)]; an
rgb head.  The output is (rgb_raw, sigma_raw), no activations (the
compositor applies them).  The page never sets ``skip`` in ``__init__``; the
reading is skip = 4 ("layer 4 ... before layer 5" in the prose after the
listing), or none for networks without a skip.

``hash_field_forward`` is the same structure for a hash-grid field: a
density net of two ReLU layers on the grid features, density head, linear
feature layer, then a colour net of two ReLU layers on [feature, direction
encoding] and the rgb head.

Precision modes
  "f64"   float64 arithmetic on the float32 weights (the definition).
  "bf16"  emulates a bfloat16 matrix engine: weights and every layer's input
          activations rounded to bfloat16 (round to nearest even), products
          accumulated in float64, biases kept in float32.
"""
from __future__ import annotations

import numpy as np


def round_bf16(a) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even), returned as
    float64.  Done on the float32 bit pattern: add 0x7FFF plus the lowest kept
    bit, then clear the low 16 bits."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = a32.view(np.uint32).astype(np.uint64)
    bits = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _linear(x, Wb, mode: str):
    W, b = Wb
    W = np.asarray(W, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    if mode == "bf16":
        return round_bf16(x) @ round_bf16(W).T + b
    return np.asarray(x, dtype=np.float64) @ W.astype(np.float64).T + b


def _relu(x):
    return np.maximum(x, 0.0)


def nerf_forward(params: dict, pos_enc, dir_enc, mode: str = "f64") -> np.ndarray:
    """NeRF network on encoded inputs: ``pos_enc`` [P, pos_ch], ``dir_enc``
    [P, dir_ch].  Returns float64 [P, 4] = (rgb_raw, sigma_raw)."""
    shape = params["shape"]
    pos_enc = np.asarray(pos_enc, dtype=np.float64)
    h = pos_enc
    for i, Wb in enumerate(params["layers"]):
        h = _relu(_linear(h, Wb, mode))
        if shape.skip >= 0 and i == shape.skip:
            h = np.concatenate([h, pos_enc], axis=-1)
    sigma = _linear(h, params["sigma"], mode)
    feature = _linear(h, params["feature"], mode)
    g = _relu(_linear(np.concatenate([feature, np.asarray(dir_enc, dtype=np.float64)], axis=-1), params["dir"], mode))
    rgb = _linear(g, params["rgb"], mode)
    return np.concatenate([rgb, sigma], axis=-1)


def hash_field_forward(params: dict, feats, dir_enc, mode: str = "f64") -> np.ndarray:
    """Hash-grid field network.  ``feats`` [P, 32] interpolated grid features,
    ``dir_enc`` [P, 16].  Returns float64 [P, 4] = (rgb_raw, sigma_raw)."""
    h = np.asarray(feats, dtype=np.float64)
    for Wb in params["density"]:
        h = _relu(_linear(h, Wb, mode))
    sigma = _linear(h, params["sigma"], mode)
    feature = _linear(h, params["feature"], mode)
    g = np.concatenate([feature, np.asarray(dir_enc, dtype=np.float64)], axis=-1)
    for Wb in params["color"]:
        g = _relu(_linear(g, Wb, mode))
    rgb = _linear(g, params["rgb"], mode)
    return np.concatenate([rgb, sigma], axis=-1)


def nerf_forward_naive(params: dict, pos_enc, dir_enc) -> np.ndarray:
    """The same network written as explicit loops over samples, output units
    and inputs, in plain Python floats.  For a handful of samples only."""
    shape = params["shape"]

    def lin(vec, Wb, relu):
        W, b = Wb
        out = []
        for o in range(W.shape[0]):
            s = float(b[o])
            for i in range(W.shape[1]):
                s += float(W[o, i]) * vec[i]
            out.append(max(s, 0.0) if relu else s)
        return out

    res = []
    for p in range(len(pos_enc)):
        pe = [float(v) for v in pos_enc[p]]
        h = pe
        for i, Wb in enumerate(params["layers"]):
            h = lin(h, Wb, True)
            if shape.skip >= 0 and i == shape.skip:
                h = h + pe
        sigma = lin(h, params["sigma"], False)
        feat = lin(h, params["feature"], False)
        g = lin(feat + [float(v) for v in dir_enc[p]], params["dir"], True)
        rgb = lin(g, params["rgb"], False)
        res.append(rgb + sigma)
    return np.array(res, dtype=np.float64)


def hash_field_forward_naive(params: dict, feats, dir_enc) -> np.ndarray:
    """The hash-grid field written as explicit loops over samples, output
    units and inputs, in plain Python floats: density layers on the grid
    features, density head and feature layer on the last density state, then
    the colour layers on [feature, direction encoding] and the rgb head.  For
    a handful of samples only."""

    def lin(vec, Wb, relu):
        W, b = Wb
        out = []
        for o in range(W.shape[0]):
            s = float(b[o])
            for i in range(W.shape[1]):
                s += float(W[o, i]) * vec[i]
            out.append(max(s, 0.0) if relu else s)
        return out

    res = []
    for p in range(len(feats)):
        h = [float(v) for v in feats[p]]
        for Wb in params["density"]:
            h = lin(h, Wb, True)
        sigma = lin(h, params["sigma"], False)
        feat = lin(h, params["feature"], False)
        g = feat + [float(v) for v in dir_enc[p]]
        for Wb in params["color"]:
            g = lin(g, Wb, True)
        rgb = lin(g, params["rgb"], False)
        res.append(rgb + sigma)
    return np.array(res, dtype=np.float64)

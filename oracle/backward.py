"""Gradients and the training step (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Spatial Intelligence - Part 1: NeRF", Section 1 Theory, 5. Training (the
photometric loss between rendered and true pixel colours) and Section 2 Code,
7. Training loop (mean squared error of the rendered rgb, Adam, PSNR =
-10 log10(MSE)).  The slice here is one network pass: stratified samples,
position and direction encodings, the NeRF-family network, compositing, MSE
against target colours, the gradient of the loss with respect to every
weight and bias, and one Adam step (Kingma and Ba, "Adam: A Method for
Stochastic Optimization", Algorithm 1, with bias correction).

Everything is float64 ("f64", the definition) or emulates bfloat16 matrix
products ("bf16": weights and layer inputs rounded to bfloat16, float64
accumulation), the same readings as the forward oracle.
"""
from __future__ import annotations

import numpy as np

from . import composite, encoding, mlp, sampling
from .mlp import round_bf16


def _rb(a, mode):
    """An operand of a matrix product: rounded to bfloat16 ("bf16"), else
    taken exactly as given (float32 fixtures convert to float64 exactly)."""
    return round_bf16(a) if mode == "bf16" else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Network: forward with the values the backward needs, and the backward
# ----------------------------------------------------------------------------

def nerf_forward_cache(params: dict, pos_enc, dir_enc, mode: str = "f64"):
    """The network of ``oracle.mlp.nerf_forward`` keeping, for every dense
    layer, its input and its output.  Returns (raw [P,4], cache)."""
    shape = params["shape"]
    pe = np.asarray(pos_enc, dtype=np.float64)
    de = np.asarray(dir_enc, dtype=np.float64)
    cache = []

    def dense(x, Wb, relu, name):
        W, b = Wb
        y = _rb(x, mode) @ _rb(W, mode).T + np.asarray(b, dtype=np.float64)
        out = np.maximum(y, 0.0) if relu else y
        cache.append((name, x, out, relu))
        return out

    h = pe
    for i, Wb in enumerate(params["layers"]):
        h = dense(h, Wb, True, ("layers", i))
        if shape.skip >= 0 and i == shape.skip:
            h = np.concatenate([h, pe], axis=-1)
    sigma = dense(h, params["sigma"], False, ("sigma",))
    feature = dense(h, params["feature"], False, ("feature",))
    g = dense(np.concatenate([feature, de], axis=-1), params["dir"], True, ("dir",))
    rgb = dense(g, params["rgb"], False, ("rgb",))
    return np.concatenate([rgb, sigma], axis=-1), cache


def nerf_backward(params: dict, cache, d_raw, mode: str = "f64") -> dict:
    """Gradient of a scalar loss with respect to every weight and bias, given
    dL/draw [P,4] (rgb_raw, sigma_raw) and the forward cache.  The products
    of the backward use the same operand rounding as the forward ("bf16":
    the layer input, the weights and the incoming gradient rounded to
    bfloat16).  Returns a dict shaped like ``params`` with (dW, db) pairs."""
    shape = params["shape"]
    by = {c[0]: c for c in cache}
    W_of = {("layers", i): Wb[0] for i, Wb in enumerate(params["layers"])}
    for k in ("sigma", "feature", "dir", "rgb"):
        W_of[(k,)] = params[k][0]
    grads = {}

    def back(name, d_out):
        """dL/d(input) of layer `name` from dL/d(output)."""
        _, x, out, relu = by[name]
        d_pre = d_out * (out > 0.0) if relu else d_out
        grads[name] = (_rb(d_pre, mode).T @ _rb(x, mode), d_pre.sum(axis=0))
        return _rb(d_pre, mode) @ _rb(W_of[name], mode)

    d_raw = np.asarray(d_raw, dtype=np.float64)
    d_g = back(("rgb",), d_raw[:, :3])
    d_fd = back(("dir",), d_g)
    Wd = shape.width
    d_h = back(("feature",), d_fd[:, :Wd]) + back(("sigma",), d_raw[:, 3:4])
    for i in reversed(range(shape.depth)):
        if shape.skip >= 0 and i == shape.skip:
            d_h = d_h[:, :Wd]  # the encoding columns concatenated after this layer take no gradient back
        d_h = back(("layers", i), d_h)
    out = {"shape": shape, "layers": [grads[("layers", i)] for i in range(shape.depth)]}
    for k in ("sigma", "feature", "dir", "rgb"):
        out[k] = grads[(k,)]
    return out


# ----------------------------------------------------------------------------
# Compositing backward
# ----------------------------------------------------------------------------

def composite_backward(raw, z, rays_d, d_rgb, white_bkgd: bool = False):
    """dL/draw [R,N,4] of the compositor (``oracle.composite.volume_render``,
    no termination) given dL/drgb [R,3].

    With c_i = sigmoid(r_i), s_i = 1 - alpha_i + 1e-10, T_i = prod_{j<i} s_j,
    w_i = T_i alpha_i and e_i = dL/drgb . c_i (white background:
    dL/drgb . (c_i - 1), since rgb gains 1 - sum w):
      dL/dr_i     = w_i dL/drgb * c_i (1 - c_i)
      dL/dalpha_i = T_i (e_i - R_i),  R_i = sum_{k>i} e_k alpha_k prod_{i<j<k} s_j
      dL/dsigma_raw_i = dL/dalpha_i * delta_i (1 - alpha_i) * [sigma_raw_i > 0]."""
    raw = np.asarray(raw, dtype=np.float64)
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    R, N, _ = raw.shape
    dnorm = np.linalg.norm(np.asarray(rays_d, dtype=np.float64), axis=-1, keepdims=True)
    delta = np.concatenate([z[:, 1:] - z[:, :-1], np.full((R, 1), 1e10)], axis=1) * dnorm
    c = composite.sigmoid(raw[..., :3])
    sig = np.maximum(raw[..., 3], 0.0)
    alpha = 1.0 - np.exp(-sig * delta)
    s = 1.0 - alpha + 1e-10
    T = np.cumprod(np.concatenate([np.ones((R, 1)), s[:, :-1]], axis=1), axis=1)
    w = T * alpha
    d_rgb = np.asarray(d_rgb, dtype=np.float64)
    e = np.einsum("rnc,rc->rn", c - 1.0 if white_bkgd else c, d_rgb)
    Rsum = np.zeros((R, N))
    for i in range(N - 2, -1, -1):
        Rsum[:, i] = e[:, i + 1] * alpha[:, i + 1] + s[:, i + 1] * Rsum[:, i + 1]
    d_alpha = T * (e - Rsum)
    d_raw = np.zeros_like(raw)
    d_raw[..., :3] = w[..., None] * d_rgb[:, None, :] * c * (1.0 - c)
    d_raw[..., 3] = d_alpha * delta * (1.0 - alpha) * (raw[..., 3] > 0.0)
    return d_raw


# ----------------------------------------------------------------------------
# Loss, training step, Adam
# ----------------------------------------------------------------------------

def mse(rgb, target):
    """The page's loss: mean over rays and channels of the squared error."""
    d = np.asarray(rgb, np.float64) - np.asarray(target, np.float64)
    return float(np.mean(d * d))


def psnr(mse_value: float) -> float:
    return -10.0 * np.log10(mse_value)


def train_loss_and_grads(params, rays_o, rays_d, t_near, t_far, target, n_samples, L_pos=10, L_dir=4, seed=0,
                         jitter=True, mode="f64", use_pi=True, white_bkgd=False, ray_offset=0):
    """Loss (MSE of the rendered rgb against ``target``) and its gradient for
    one network pass over stratified samples.  Returns (loss, rgb, grads)."""
    z = sampling.stratified(t_near, t_far, n_samples, seed, jitter, ray_offset)
    loss, rgb, grads, _ = train_pass(params, rays_o, rays_d, z, target, L_pos, L_dir, mode, use_pi, white_bkgd)
    return loss, rgb, grads


def train_pass(params, rays_o, rays_d, z, target, L_pos=10, L_dir=4, mode="f64", use_pi=True, white_bkgd=False):
    """One network pass over given sample depths ``z`` [R, N] (float32,
    ascending): loss, rendered rgb, the gradient of the loss with respect to
    every parameter, and the compositing weights [R, N].  The depths carry no
    gradient (the page's fine samples come from the coarse weights under
    no_grad)."""
    z = np.asarray(z, dtype=np.float32)
    R, N = z.shape
    x = sampling.points(rays_o, rays_d, z)
    pe = encoding.freq_encode(x.reshape(-1, 3), L_pos, True, use_pi)
    de = np.repeat(encoding.freq_encode(sampling.view_dirs(rays_d), L_dir, True, use_pi), N, axis=0)
    raw, cache = nerf_forward_cache(params, pe, de, mode)
    raw = raw.reshape(R, N, 4)
    rgb, _, _, w = composite.volume_render(raw, z, rays_d, white_bkgd)
    loss = mse(rgb, target)
    d_rgb = 2.0 * (rgb - np.asarray(target, np.float64)) / rgb.size
    d_raw = composite_backward(raw, z, rays_d, d_rgb, white_bkgd).reshape(R * N, 4)
    return loss, rgb, nerf_backward(params, cache, d_raw, mode), w


def hierarchical_train_step(coarse, fine, rays_o, rays_d, t_near, t_far, target, n_coarse=64, n_fine=128,
                            L_pos=10, L_dir=4, seed=0, jitter=True, mode="f64", use_pi=True, white_bkgd=False,
                            ray_offset=0):
    """The page's training objective on one batch (Section 2 Code, 7.
    Training loop: MSE of the coarse and of the fine rendering): the coarse
    network on stratified samples, fine samples drawn from the coarse
    weights (``sampling.hierarchical_fine_samples``, weights as float32, no
    gradient through them) and merged, the fine network on the merged
    samples.  The loss is the sum of the two MSEs, so each network's
    gradient is that of its own term.  Returns dict(loss_c, loss_f, rgb_c,
    rgb_f, grads_c, grads_f, w_c, z_c, bins, z2)."""
    z_c = sampling.stratified(t_near, t_far, n_coarse, seed, jitter, ray_offset)
    loss_c, rgb_c, g_c, w_c = train_pass(coarse, rays_o, rays_d, z_c, target, L_pos, L_dir, mode, use_pi,
                                         white_bkgd)
    _, bins, z2 = sampling.hierarchical_fine_samples(z_c, w_c.astype(np.float32), n_fine, seed, ray_offset)
    loss_f, rgb_f, g_f, _ = train_pass(fine, rays_o, rays_d, z2, target, L_pos, L_dir, mode, use_pi, white_bkgd)
    return dict(loss_c=loss_c, loss_f=loss_f, rgb_c=rgb_c, rgb_f=rgb_f, grads_c=g_c, grads_f=g_f, w_c=w_c, z_c=z_c,
                bins=bins, z2=z2)


def flatten(params_or_grads) -> np.ndarray:
    """Weights and biases in the order nerf_pack_mlp takes them, flattened
    (row-major weights), float64."""
    seq = list(params_or_grads["layers"]) + [params_or_grads[k] for k in ("sigma", "feature", "dir", "rgb")]
    return np.concatenate([np.asarray(a, np.float64).ravel() for Wb in seq for a in Wb])


def unflatten(flat, like: dict) -> dict:
    """Inverse of ``flatten`` with the shapes of ``like`` (float32 arrays)."""
    out = {"shape": like["shape"]}
    pos = 0

    def take(a):
        nonlocal pos
        n = np.asarray(a).size
        v = np.asarray(flat[pos:pos + n], np.float64).reshape(np.asarray(a).shape).astype(np.float32)
        pos += n
        return v

    out["layers"] = [(take(W), take(b)) for W, b in like["layers"]]
    for k in ("sigma", "feature", "dir", "rgb"):
        out[k] = (take(like[k][0]), take(like[k][1]))
    return out


def adam(p, g, m, v, t: int, lr: float, beta1=0.9, beta2=0.999, eps=1e-8):
    """One Adam step (bias-corrected) on flat float64 arrays; returns (p, m, v)."""
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    return p - lr * m_hat / (np.sqrt(v_hat) + eps), m, v

"""Training the hash-grid INR (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Instant-NGP - Visual Experiments (a 2D multiresolution hash grid)", shared
toolkit (``HashGrid2D``, ``HashINR``, ``train``) and Experiment 2: the
learnable feature tables of a multiresolution grid, a decoder with one
hidden ReLU layer on the concatenated features, the mean squared error
against target values, and Adam on the tables and the decoder together.

Readings: the grid is ``encoding.HashGrid`` (2D as in the notebook, or 3D);
every table stores 2 features per entry in float32; the decoder is
Linear(L*2 -> hidden), ReLU, Linear(hidden -> n_out); the loss is the mean
over points and outputs of the squared error.  Parameters are one flat
vector: the tables level by level (entries x features, row-major), then
W1 [hidden, L*2], b1, W2 [n_out, hidden], b2.  Everything is float64.
"""
from __future__ import annotations

import numpy as np

from .encoding import HashGrid


def corner_weights(grid: HashGrid, x, l: int):
    """Table indices [P, 2^dim] and multilinear weights [P, 2^dim] (float64)
    of level l, corners in the order of ``HashGrid.level_indices``."""
    idx, w = grid.level_indices(x, l)
    w = w.astype(np.float64)
    wt = np.ones(idx.shape, dtype=np.float64)
    for corner in range(idx.shape[1]):
        for a in range(grid.dim):
            bit = (corner >> (grid.dim - 1 - a)) & 1
            wt[:, corner] *= w[:, a] if bit else 1.0 - w[:, a]
    return idx, wt


def forward_backward(grid: HashGrid, tables, mlp, x, target, level_mask=None):
    """Loss, prediction [P, n_out] and the gradient of the loss with respect
    to every table entry (list of [size_l, 2]) and decoder parameter
    ((dW1, db1, dW2, db2)).  The feature gradient of a point reaches each of
    its corners' entries times that corner's weight (and the level's mask);
    entries shared by several corners or points add up."""
    W1, b1, W2, b2 = (np.asarray(a, np.float64) for a in mlp)
    x = np.asarray(x, np.float32)
    target = np.asarray(target, np.float64)
    P = x.shape[0]
    L = grid.L
    mask = np.ones(L) if level_mask is None else np.asarray(level_mask, np.float64)
    looks = [corner_weights(grid, x, l) for l in range(L)]
    feats = np.zeros((P, 2 * L))
    for l, (idx, wt) in enumerate(looks):
        tab = np.asarray(tables[l], np.float64)
        feats[:, 2 * l:2 * l + 2] = mask[l] * np.einsum("pc,pcf->pf", wt, tab[idx])
    pre = feats @ W1.T + b1
    h = np.maximum(pre, 0.0)
    y = h @ W2.T + b2
    diff = y - target
    loss = float(np.mean(diff * diff))
    dy = 2.0 * diff / diff.size
    dW2 = dy.T @ h
    db2 = dy.sum(axis=0)
    dpre = (dy @ W2) * (pre > 0.0)
    dW1 = dpre.T @ feats
    db1 = dpre.sum(axis=0)
    dfeat = dpre @ W1
    dtab = []
    for l, (idx, wt) in enumerate(looks):
        g = np.zeros((grid.sizes[l], 2))
        contrib = mask[l] * wt[:, :, None] * dfeat[:, None, 2 * l:2 * l + 2]
        np.add.at(g, idx.reshape(-1), contrib.reshape(-1, 2))
        dtab.append(g)
    return loss, y, dtab, (dW1, db1, dW2, db2)


def flatten(tables, mlp) -> np.ndarray:
    return np.concatenate([np.asarray(t, np.float64).ravel() for t in tables] +
                          [np.asarray(a, np.float64).ravel() for a in mlp])


def unflatten(flat, grid: HashGrid, hidden: int, n_out: int):
    flat = np.asarray(flat, np.float64)
    pos = 0
    tables = []
    for s in grid.sizes:
        tables.append(flat[pos:pos + 2 * s].reshape(s, 2))
        pos += 2 * s
    shapes = [(hidden, 2 * grid.L), (hidden,), (n_out, hidden), (n_out,)]
    mlp = []
    for sh in shapes:
        n = int(np.prod(sh))
        mlp.append(flat[pos:pos + n].reshape(sh))
        pos += n
    assert pos == flat.size
    return tables, tuple(mlp)


def train(grid: HashGrid, tables, mlp, x, target, steps: int, lr: float, beta1=0.9, beta2=0.999, eps=1e-8,
          level_mask=None):
    """``steps`` full-batch Adam steps (the notebook's ``train``); returns the
    final flat parameters and the loss before each step."""
    from .backward import adam
    hidden, n_out = np.asarray(mlp[0]).shape[0], np.asarray(mlp[2]).shape[0]
    p = flatten(tables, mlp)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    losses = []
    for t in range(1, steps + 1):
        tb, ml = unflatten(p, grid, hidden, n_out)
        loss, _, dt, dm = forward_backward(grid, tb, ml, x, target, level_mask)
        losses.append(loss)
        p, m, v = adam(p, flatten(dt, dm), m, v, t, lr, beta1, beta2, eps)
    return p, losses

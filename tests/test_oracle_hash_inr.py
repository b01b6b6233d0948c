"""Pins of the hash-grid INR training oracle (oracle/hash_inr.py): central
differences for every parameter, closed forms of a point on a grid vertex and
of masked levels, and the notebook's claim that the INR fits its test image
(Experiment 2 of "Instant-NGP - Visual Experiments")."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import encoding, hash_inr


def _setup(dim, seed=0, hidden=5, n_out=2, P=7):
    grid = encoding.HashGrid(dim, 3, 16 if dim == 2 else 32, 2, 9)  # a direct level and hashed ones
    tables, mlp = si.hash_inr_params(grid.sizes, grid.L, hidden, n_out, seed=seed)
    tables = [t * 1e3 for t in tables]  # features of order 0.1, so every path matters
    g = np.random.default_rng(seed)
    x = g.random((P, dim)).astype(np.float32)
    target = g.random((P, n_out))
    return grid, tables, mlp, x, target


@pytest.mark.parametrize("dim", [2, 3])
def test_gradients_match_central_differences(dim):
    grid, tables, mlp, x, target = _setup(dim)
    assert any(grid.direct) and not all(grid.direct)
    mask = [1.0, 0.5, 1.0]
    loss, _, dt, dm = hash_inr.forward_backward(grid, tables, mlp, x, target, mask)
    ana = hash_inr.flatten(dt, dm)
    flat = hash_inr.flatten(tables, mlp)
    hidden, n_out = mlp[0].shape[0], mlp[2].shape[0]

    def L(f):
        tb, ml = hash_inr.unflatten(f, grid, hidden, n_out)
        return hash_inr.forward_backward(grid, tb, ml, x, target, mask)[0]

    h = 1e-6
    num = np.empty_like(flat)
    for k in range(flat.size):
        fp, fm = flat.copy(), flat.copy()
        fp[k] += h
        fm[k] -= h
        num[k] = (L(fp) - L(fm)) / (2 * h)
    scale = np.abs(num).max()
    assert np.max(np.abs(ana - num)) <= 1e-6 * scale + 1e-10
    touched = np.count_nonzero(ana[:2 * sum(grid.sizes)])
    assert touched > 0.3 * min(2 * sum(grid.sizes), 2 * 8 * x.shape[0])


def test_point_on_a_vertex_touches_one_entry_per_direct_level():
    """On a direct level a point on a grid vertex has weight 1 at that vertex
    and 0 elsewhere, so only that entry's gradient is nonzero, and it equals
    the feature gradient."""
    grid, tables, mlp, _, _ = _setup(2)
    N = grid.res[0]
    x = np.array([[1.0 / N, 1.0 / N]], np.float32)  # the interior vertex (1, 1) of level 0
    target = np.zeros((1, 2))
    _, _, dt, dm = hash_inr.forward_backward(grid, tables, mlp, x, target)
    nz = np.flatnonzero(np.abs(dt[0]).sum(axis=1))
    assert grid.direct[0] and list(nz) == [1 * (N + 1) + 1]


def test_masked_level_takes_no_gradient_and_others_are_unchanged():
    grid, tables, mlp, x, target = _setup(3, seed=2)
    _, _, dt_full, _ = hash_inr.forward_backward(grid, tables, mlp, x, target, [1.0, 1.0, 1.0])
    _, _, dt_mask, _ = hash_inr.forward_backward(grid, tables, mlp, x, target, [1.0, 0.0, 1.0])
    assert np.all(dt_mask[1] == 0.0) and np.any(dt_full[1] != 0.0)
    # with level 1's features gone the others' gradients change only through the decoder
    feats_full = grid.encode(x, tables, [1.0, 1.0, 1.0])
    feats_mask = grid.encode(x, tables, [1.0, 0.0, 1.0])
    assert np.all(feats_mask[:, 2:4] == 0.0) and np.array_equal(feats_mask[:, :2], feats_full[:, :2])


def test_training_fits_the_test_image():
    """Experiment 2's setting at a smaller image: an 8-level grid (T = 2^12,
    N from 8 to 160) and a 32-wide decoder fitted with Adam at lr 1e-2; the
    page's hash model reaches a tiny error in 800 steps, and here 300 steps
    already bring the loss down by three orders of magnitude."""
    coords, target = si.inr_target_image(40)
    grid = encoding.HashGrid(2, 8, 2 ** 12, 8, 160)
    tables, mlp = si.hash_inr_params(grid.sizes, grid.L, 32, 1, seed=1)
    _, losses = hash_inr.train(grid, tables, mlp, coords, target, steps=300, lr=1e-2)
    assert losses[-1] < 1e-3 * losses[0]

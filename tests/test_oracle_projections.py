"""Pins of the oracle's projections (hidden state to queries and streams; heads
back to the model width)."""
import numpy as np

from oracle import method


def test_project_identity_and_permutation():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 1, (5, 8))
    np.testing.assert_array_equal(method.project(x, np.eye(8)), x)
    perm = rng.permutation(8)
    np.testing.assert_array_equal(method.project(x, np.eye(8)[perm]), x[:, perm])


def test_project_brute_force():
    rng = np.random.default_rng(1)
    x, W = rng.normal(0, 1, (3, 7)), rng.normal(0, 1, (4, 7))
    y = method.project(x, W)
    for r in range(3):
        for n in range(4):
            assert abs(y[r, n] - sum(x[r, k] * W[n, k] for k in range(7))) < 1e-12


def test_absorption_identity():
    """q~_h . c = q_h . (W_UK^h c): the absorbed query scores a latent c as the
    head query scores the head key the latent expands to."""
    rng = np.random.default_rng(2)
    R, H, dh, D = 3, 4, 5, 9
    qh = rng.normal(0, 1, (R, H, dh))
    WUK = rng.normal(0, 1, (H, dh, D))
    qt = method.absorb_queries(qh, WUK)
    c = rng.normal(0, 1, D)
    for r in range(R):
        for h in range(H):
            assert abs(qt[r, h] @ c - qh[r, h] @ (WUK[h] @ c)) < 1e-10


def test_absorption_brute_force_and_unit_heads():
    rng = np.random.default_rng(3)
    R, H, dh, D = 2, 2, 3, 4
    qh = rng.normal(0, 1, (R, H, dh))
    WUK = rng.normal(0, 1, (H, dh, D))
    qt = method.absorb_queries(qh, WUK)
    for r in range(R):
        for h in range(H):
            for d in range(D):
                assert abs(qt[r, h, d] - sum(qh[r, h, k] * WUK[h, k, d] for k in range(dh))) < 1e-12
    # a unit head query picks one row of W_UK
    e = np.zeros((1, H, dh))
    e[0, 1, 2] = 1.0
    np.testing.assert_array_equal(method.absorb_queries(e, WUK)[0, 1], WUK[1, 2])
    np.testing.assert_array_equal(method.absorb_queries(e, WUK)[0, 0], np.zeros(D))

"""Pins of the oracle's compressor and entry storage (closed forms and invariants)."""
import numpy as np
import pytest

from oracle import codecs, method


def _rand(rng, N, D, scale=1.0):
    return rng.normal(0, scale, (N, D))


def _window(j, m, o, N):
    return [i for i in range(m * j - o, m * j + m) if 0 <= i < N]


@pytest.mark.parametrize("m,o,N,D", [(4, 4, 64, 8), (128, 0, 512, 4), (4, 0, 40, 3), (2, 6, 30, 2)])
def test_uniform_gates_give_mean_pooling(m, o, N, D):
    """Equal gate logits over a window make the pool the plain mean of its tokens."""
    rng = np.random.default_rng(0)
    v = _rand(rng, N, D)
    g = np.full((N, D), 0.37)
    c = method.compress(v, g, np.zeros((m + o, D)), m, o)
    assert c.shape == (N // m, D)
    for j in range(N // m):
        np.testing.assert_allclose(c[j], v[_window(j, m, o, N)].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_hca_uniform_is_block_mean():
    rng = np.random.default_rng(1)
    v = _rand(rng, 1024, 6)
    c = method.compress(v, np.zeros_like(v), np.zeros((128, 6)), 128, 0)
    np.testing.assert_allclose(c, v.reshape(8, 128, 6).mean(axis=1), rtol=1e-13, atol=1e-14)


def test_per_channel_constant_gate_shift_is_invisible():
    rng = np.random.default_rng(2)
    v, g = _rand(rng, 64, 5), _rand(rng, 64, 5)
    bp = rng.normal(0, 1, (8, 5))
    shift = rng.normal(0, 10, (1, 5))
    np.testing.assert_allclose(method.compress(v, g + shift, bp, 4, 4), method.compress(v, g, bp, 4, 4),
                               rtol=1e-12, atol=1e-13)


def test_dominant_position_copies_its_token():
    rng = np.random.default_rng(3)
    N, D, m, o = 64, 4, 4, 4
    v, g = _rand(rng, N, D), _rand(rng, N, D)
    for slot in range(m + o):
        bp = np.zeros((m + o, D))
        bp[slot] = 1000.0
        c = method.compress(v, g, bp, m, o)
        for j in range(N // m):
            i = m * j - o + slot
            if i >= 0:
                np.testing.assert_allclose(c[j], v[i], rtol=0, atol=1e-12)


def test_stride1_no_overlap_is_identity():
    rng = np.random.default_rng(4)
    v, g = _rand(rng, 33, 7), _rand(rng, 33, 7)
    np.testing.assert_array_equal(method.compress(v, g, rng.normal(0, 1, (1, 7)), 1, 0), v)


def test_weights_sum_to_one_and_linear_in_values():
    rng = np.random.default_rng(5)
    N, D = 48, 3
    g = _rand(rng, N, D, 3.0)
    bp = rng.normal(0, 1, (8, D))
    ones = method.compress(np.ones((N, D)), g, bp, 4, 4)
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-14)
    v1, v2 = _rand(rng, N, D), _rand(rng, N, D)
    lhs = method.compress(2.5 * v1 - 0.75 * v2, g, bp, 4, 4)
    rhs = 2.5 * method.compress(v1, g, bp, 4, 4) - 0.75 * method.compress(v2, g, bp, 4, 4)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


def test_pool_stays_in_convex_hull():
    rng = np.random.default_rng(6)
    N, D, m, o = 64, 5, 4, 4
    v, g = _rand(rng, N, D), _rand(rng, N, D, 4.0)
    c = method.compress(v, g, rng.normal(0, 1, (8, D)), m, o)
    for j in range(N // m):
        w = v[_window(j, m, o, N)]
        assert np.all(c[j] <= w.max(axis=0) + 1e-12) and np.all(c[j] >= w.min(axis=0) - 1e-12)


def test_chunking_does_not_change_result():
    rng = np.random.default_rng(7)
    v, g = _rand(rng, 400, 3), _rand(rng, 400, 3)
    bp = rng.normal(0, 1, (8, 3))
    np.testing.assert_array_equal(method.compress(v, g, bp, 4, 4, chunk=7), method.compress(v, g, bp, 4, 4))


def test_golden_closed_forms(golden):
    for name in ("compress_csa_log_gates", "compress_position_bias"):
        case = golden[name]
        v = np.array(case["v"], float)
        g = np.log(np.array(case["g_is_log_of"], float))
        bp = np.log(np.array(case["bpos_is_log_of"], float)) if "bpos_is_log_of" in case else np.array(case["bpos"], float)
        c = method.compress(v, g, bp, case["m"], case["o"])
        np.testing.assert_allclose(c, np.array(case["expected"]), rtol=1e-14, err_msg=name)


def test_store_e4m3_scale_and_error_bound():
    rng = np.random.default_rng(8)
    c = rng.normal(0, 1, (200, 64)) * rng.uniform(0.01, 10, (200, 1))
    c[3] = 0.0
    st = method.store_entries(c, "e4m3")
    amax = np.abs(c).max(axis=1)
    assert st["scale"][3] == 1.0 and np.all(st["values"][3] == 0)
    nz = amax > 0
    np.testing.assert_allclose(st["scale"][nz], amax[nz] / 448, rtol=2 ** -24)
    # the largest-magnitude channel lands on +-448 (up to the fp32 rounding of the scale)
    top = np.abs(codecs.e4m3_decode(st["codes"])).max(axis=1)
    assert np.all(top[nz] == 448.0)
    # relative error of a normal e4m3 value is at most half an ulp = 2^-4
    y = c / st["scale"][:, None]
    normal = np.abs(y) >= 2 ** -6
    err = np.abs(st["values"] - c)
    assert np.all(err[normal] <= 2 ** -4 * np.abs(c[normal]) * (1 + 1e-12))
    assert np.all(err[~normal] <= 2 ** -10 * np.broadcast_to(st["scale"][:, None], c.shape)[~normal] * (1 + 1e-12))
    np.testing.assert_array_equal(codecs.e4m3_decode(st["codes"]) * st["scale"][:, None], st["values"])


def test_store_keys_e4m3_unscaled():
    k = np.array([[0.3, -500.0, 17.0, 1e-4]])
    st = method.store_keys(k, "e4m3")
    assert st["scale"] is None
    np.testing.assert_array_equal(st["values"], codecs.round_e4m3(k))


def test_brute_force_loops_tiny():
    """Explicit loops over (entry, channel, token) on a tiny ragged case."""
    import math
    rng = np.random.default_rng(9)
    N, D, m, o = 23, 3, 4, 4
    v, g, bp = _rand(rng, N, D), _rand(rng, N, D, 2.0), rng.normal(0, 1, (m + o, D))
    c = method.compress(v, g, bp, m, o)
    for j in range(N // m):
        for d in range(D):
            toks = [i for i in range(m * j - o, m * j + m) if i >= 0]
            a = [g[i, d] + bp[i - m * j + o, d] for i in toks]
            mx = max(a)
            e = [math.exp(x - mx) for x in a]
            ref = sum(ei * v[i, d] for ei, i in zip(e, toks)) / sum(e)
            assert abs(c[j, d] - ref) <= 1e-13 * max(1.0, abs(ref))


@pytest.mark.parametrize("m,o,N,block", [(4, 4, 203, 7), (4, 4, 4096, 100), (128, 0, 1300, 3), (2, 6, 101, 5)])
def test_blocked_compress_equals_whole(m, o, N, block):
    """The entry-blocked driver used at million-token sizes gives the whole-array result."""
    from tests.compare import blocked_compress
    rng = np.random.default_rng(N + block)
    D = 6
    v, g, bp = _rand(rng, N, D), _rand(rng, N, D, 2.0), rng.normal(0, 1, (m + o, D))
    np.testing.assert_array_equal(blocked_compress(v, g, bp, m, o, block=block), method.compress(v, g, bp, m, o))

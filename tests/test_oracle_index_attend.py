"""Pins of the oracle's visibility rule, lightning indexer, top-k and attention."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import method, pipeline


# ---------------------------------------------------------------- visibility / window
def test_visibility_matches_enumeration():
    for m in (1, 4, 128):
        for W in (0, 3, 128):
            for t in list(range(0, 700, 7)) + [4095, 65535]:
                brute = 0
                while m * (brute + 1) <= t - W:
                    brute += 1
                assert method.entries_visible(t, m, W) == brute, (t, m, W)


def test_golden_visibility(golden):
    for c in golden["visibility"]["cases"]:
        assert method.entries_visible(c["t"], c["m"], c["W"]) == c["e_vis"], c


def test_window_contains_t_and_is_w_long():
    assert method.window_positions(0, 128).tolist() == [0]
    assert method.window_positions(5, 128).tolist() == list(range(6))
    w = method.window_positions(1000, 128)
    assert w[0] == 873 and w[-1] == 1000 and len(w) == 128


# ---------------------------------------------------------------- indexer
def test_golden_indexer_topk(golden):
    c = golden["indexer_topk"]
    s = method.index_scores(np.array(c["q"], float), np.array(c["w"], float), np.array(c["keys"], float))
    np.testing.assert_array_equal(s, c["expected_scores"])
    assert not np.signbit(s[3])
    assert method.topk(s, 2).tolist() == c["expected_top2"]
    assert method.topk(s, 4).tolist() == c["expected_top4"]
    assert method.topk(s, 7).tolist() == c["expected_top7"]


def test_indexer_unit_query_reduces_to_relu_of_a_coordinate():
    rng = np.random.default_rng(0)
    keys = rng.normal(0, 1, (50, 6))
    q = np.zeros((1, 6))
    q[0, 2] = 1.0
    np.testing.assert_array_equal(method.index_scores(q, np.array([1.0]), keys), np.maximum(keys[:, 2], 0))


def test_indexer_positive_homogeneity_and_zero_sign():
    rng = np.random.default_rng(1)
    q, w, keys = rng.normal(0, 1, (4, 8)), rng.normal(0, 1, 4), rng.normal(0, 1, (100, 8))
    s = method.index_scores(q, w, keys)
    np.testing.assert_allclose(method.index_scores(q, w, 4.0 * keys), 4.0 * s, rtol=1e-15, atol=0)
    # all dot products negative -> every head term is zero -> +0.0
    s0 = method.index_scores(np.abs(q), -np.abs(w), -np.abs(keys))
    assert np.all(s0 == 0) and not np.any(np.signbit(s0))


def test_indexer_heads_add():
    rng = np.random.default_rng(2)
    q, w, keys = rng.normal(0, 1, (3, 5)), rng.normal(0, 1, 3), rng.normal(0, 1, (40, 5))
    parts = sum(method.index_scores(q[h:h + 1], w[h:h + 1], keys) for h in range(3))
    np.testing.assert_allclose(method.index_scores(q, w, keys), parts, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- top-k
def _dominates(s, a, b):
    return s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_unique_dominating_subset(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    s = rng.integers(-2, 3, n).astype(float)          # many exact ties
    for k in range(1, n + 2):
        kk = min(k, n)
        winners = [set(S) for S in itertools.combinations(range(n), kk)
                   if all(_dominates(s, a, b) for a in S for b in range(n) if b not in S)]
        assert len(winners) == 1
        got = method.topk(s, k)
        assert sorted(winners[0]) == got[:kk].tolist() and np.all(got[kk:] == -1)


def test_topk_special_cases():
    s = np.array([0.5, 3.0, 3.0, -1.0, 3.0])
    assert method.topk(s, 1).tolist() == [int(np.argmax(s))] == [1]      # argmax: first maximum
    assert method.topk(s, 2).tolist() == [1, 2]                          # tie -> lower index
    assert method.topk(s, 10).tolist() == [0, 1, 2, 3, 4] + [-1] * 5     # k >= n keeps all
    assert method.topk(np.zeros(0), 3).tolist() == [-1, -1, -1]          # nothing visible


def test_topk_matches_python_sort():
    rng = np.random.default_rng(7)
    s = np.round(rng.normal(0, 1, 3000), 2)
    ref = sorted(sorted(range(len(s)), key=lambda j: (-s[j], j))[:257])
    assert method.topk(s, 257).tolist() == ref


# ---------------------------------------------------------------- attention
def _sdpa(q, kv, tau, causal=False):
    """torch's CPU scaled_dot_product_attention in fp64 (a library routine)."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None]          # [1][H][Lq][D]
    kt = torch.from_numpy(np.ascontiguousarray(kv))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau, is_causal=causal)[0].numpy()


def test_golden_attend(golden):
    c = golden["attend_log_logits"]
    o, lse, p = method.attend(np.log(np.array(c["q_is_log_of"], float)), np.array(c["items"], float), c["tau"])
    np.testing.assert_allclose(p, c["expected_p"], rtol=1e-14)
    np.testing.assert_allclose(o, c["expected_o"], rtol=1e-14)
    np.testing.assert_allclose(lse, c["expected_lse"], rtol=1e-14)


def test_attend_matches_sdpa_and_rows_sum_to_one():
    rng = np.random.default_rng(3)
    q, items = rng.normal(0, 1, (8, 16)), rng.normal(0, 1, (70, 16))
    o, lse, p = method.attend(q, items, 0.25)
    np.testing.assert_allclose(o, _sdpa(q[:, None, :], items, 0.25)[:, 0, :], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(p >= 0)
    logits = 0.25 * q @ items.T
    np.testing.assert_allclose(lse, np.log(np.exp(logits).sum(axis=1)), rtol=1e-13)


def test_attend_permutation_invariant():
    rng = np.random.default_rng(4)
    q, items = rng.normal(0, 1, (4, 8)), rng.normal(0, 1, (33, 8))
    perm = rng.permutation(33)
    np.testing.assert_allclose(method.attend(q, items[perm], 0.3)[0], method.attend(q, items, 0.3)[0],
                               rtol=1e-13, atol=1e-14)


def _small_sequence(rng, N, D, DI):
    return {"entries": rng.normal(0, 1, (N // 4, D)), "keys": rng.normal(0, 1, (N // 4, DI)),
            "v": rng.normal(0, 1, (N, D))}


def test_csa_with_all_entries_kept_equals_dense():
    """top-k >= visible entries => CSA is dense attention over entries + window."""
    rng = np.random.default_rng(5)
    seq = _small_sequence(rng, 600, 16, 8)
    q, qI, w = rng.normal(0, 1, (4, 16)), rng.normal(0, 1, (2, 8)), rng.normal(0, 1, 2)
    t = 599
    csa = method.csa_row(t, q, qI, w, seq["entries"], seq["keys"], seq["v"], 4, 128, 10 ** 6, 0.25)
    hca = method.hca_row(t, q, seq["entries"], seq["v"], 4, 128, 0.25)
    assert csa["e_vis"] == hca["e_vis"] == 117
    np.testing.assert_allclose(csa["o"], hca["o"], rtol=1e-14, atol=1e-15)
    items = np.concatenate([seq["entries"][:117], seq["v"][472:600]])
    np.testing.assert_allclose(hca["o"], _sdpa(q[:, None, :], items, 0.25)[:, 0, :], rtol=1e-12, atol=1e-13)


def test_csa_attends_only_selected_entries():
    rng = np.random.default_rng(6)
    seq = _small_sequence(rng, 800, 8, 4)
    q, qI, w = rng.normal(0, 1, (2, 8)), rng.normal(0, 1, (3, 4)), rng.normal(0, 1, 3)
    r = method.csa_row(799, q, qI, w, seq["entries"], seq["keys"], seq["v"], 4, 128, 16, 0.5)
    sel = r["idx"][r["idx"] >= 0]
    assert len(sel) == 16 and sel.max() < r["e_vis"]
    assert r["p"].shape == (2, 16 + 128)
    # scores of the chosen entries dominate every other visible entry
    others = np.setdiff1d(np.arange(r["e_vis"]), sel)
    assert r["scores"][sel].min() >= r["scores"][others].max()


def test_short_context_is_causal_attention():
    """t < W: no entry is visible and every row is plain causal attention over the raw stream."""
    rng = np.random.default_rng(7)
    T, D, H = 100, 8, 3
    v = rng.normal(0, 1, (T, D))
    entries = rng.normal(0, 1, (T // 4, D))
    keys = rng.normal(0, 1, (T // 4, 4))
    qs = rng.normal(0, 1, (T, H, D))
    ref = _sdpa(np.transpose(qs, (1, 0, 2)), v, 0.2, causal=True)         # [H][T][D]
    for t in range(T):
        r = method.csa_row(t, qs[t], rng.normal(0, 1, (2, 4)), rng.normal(0, 1, 2), entries, keys, v, 4, 128, 8, 0.2)
        assert r["e_vis"] == 0 and np.all(r["idx"] == -1)
        np.testing.assert_allclose(r["o"], ref[:, t, :], rtol=1e-12, atol=1e-13)
        h = method.hca_row(t, qs[t], entries, v, 128, 128, 0.2)
        np.testing.assert_allclose(h["o"], ref[:, t, :], rtol=1e-12, atol=1e-13)


def test_absorbed_latent_equals_explicit_heads():
    rng = np.random.default_rng(8)
    H, dh, D, n = 4, 8, 32, 50
    qh = rng.normal(0, 1, (H, dh))
    W_UK, W_UV = rng.normal(0, D ** -0.5, (H, dh, D)), rng.normal(0, D ** -0.5, (H, dh, D))
    items = rng.normal(0, 1, (n, D))
    tau = 1 / math.sqrt(dh)
    explicit = method.attend_unabsorbed(qh, W_UK, W_UV, items, tau)
    qt = np.einsum("hkd,hk->hd", W_UK, qh)
    o_lat, _, _ = method.attend(qt, items, tau)
    absorbed = np.einsum("hkd,hd->hk", W_UV, o_lat)
    np.testing.assert_allclose(absorbed, explicit, rtol=1e-12, atol=1e-13)
    W_o = rng.normal(0, 1, (5, H * dh))
    np.testing.assert_allclose(method.layer_output(o_lat, W_o, W_UV), W_o @ explicit.reshape(-1), rtol=1e-12)


def test_layer_output_without_absorption_concatenates_heads():
    o = np.arange(6, dtype=float).reshape(2, 3)
    np.testing.assert_array_equal(method.layer_output(o, np.eye(6)), np.arange(6))


def test_pipeline_tiny_brute_force_loops():
    """Whole CSA row from streams with explicit loops at N = 64 (a second, loop-only
    derivation of every step: compress, store, score, select, attend)."""
    rng = np.random.default_rng(9)
    N, D, DI, m, o, W, k, H = 64, 4, 3, 4, 4, 8, 5, 2

    class L:  # minimal layer spec
        kind, d_h = "csa", 4
    L.m, L.o, L.W, L.k, L.D = m, o, W, k, D
    st = {"v": rng.normal(0, 1, (N, D)), "g": rng.normal(0, 1, (N, D)),
          "vI": rng.normal(0, 1, (N, DI)), "gI": rng.normal(0, 1, (N, DI))}
    wts = {"bpos": rng.normal(0, 1, (m + o, D)), "bposI": rng.normal(0, 1, (m + o, DI))}
    caches = pipeline.layer_caches(L, st, wts, "f32", "f32")
    q, qI, w = rng.normal(0, 1, (H, D)), rng.normal(0, 1, (2, DI)), rng.normal(0, 1, 2)
    t = N - 1
    r = pipeline.decode_row(L, caches, st["v"], q, t, qI, w)

    def pool(val, gate, bp, j, d):
        toks = [i for i in range(m * j - o, m * j + m) if i >= 0]
        a = [gate[i][d] + bp[i - m * j + o][d] for i in toks]
        e = [math.exp(x - max(a)) for x in a]
        return sum(ei * val[i][d] for ei, i in zip(e, toks)) / sum(e)

    f32 = lambda x: float(np.float32(x))
    ent = [[f32(pool(st["v"], st["g"], wts["bpos"], j, d)) for d in range(D)] for j in range(N // m)]
    key = [[f32(pool(st["vI"], st["gI"], wts["bposI"], j, d)) for d in range(DI)] for j in range(N // m)]
    ev = (t - W) // m
    s = [sum(w[h] * max(0.0, sum(qI[h][d] * key[j][d] for d in range(DI))) for h in range(2)) for j in range(ev)]
    order = sorted(range(ev), key=lambda j: (-s[j], j))[:k]
    sel = sorted(order)
    assert r["idx"].tolist() == sel
    items = [ent[j] for j in sel] + [list(st["v"][i]) for i in range(t - W + 1, t + 1)]
    for h in range(H):
        lg = [0.5 * sum(q[h][d] * it[d] for d in range(D)) for it in items]
        e = [math.exp(x - max(lg)) for x in lg]
        for d in range(D):
            ref = sum(ei * it[d] for ei, it in zip(e, items)) / sum(e)
            assert abs(r["o"][h][d] - ref) < 1e-12

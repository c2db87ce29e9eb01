"""The seeded generator: determinism, chunk independence, shapes and distributions."""
import numpy as np
import pytest

from workloads import ALL, CSA_PREFILL_32K_BF16, PAIR_DEC_128K_BF16, gen


def test_hidden_states_chunk_independent():
    wl = PAIR_DEC_128K_BF16.with_sizes(N=20000, d_model=64)
    full = gen.hidden_states(wl, 3)
    assert full.shape == (20000, 64) and full.dtype == np.float32
    np.testing.assert_array_equal(gen.hidden_states(wl, 3, 4000, 13001), full[4000:13001])
    assert not np.array_equal(gen.hidden_states(wl, 4)[:100], full[:100])
    assert abs(full.std() - 1) < 0.01 and abs(full.mean()) < 0.01


def test_heavy_tokens():
    wl = CSA_PREFILL_32K_BF16.with_sizes(d_model=16)
    hp = gen.heavy_positions(wl, 0)
    assert len(hp) == 328 and len(np.unique(hp)) == 328
    x = gen.hidden_states(wl, 0, 0, 4096)
    base = gen.hidden_states(wl.with_sizes(heavy_frac=0.0), 0, 0, 4096)
    sel = hp[hp < 4096]
    np.testing.assert_array_equal(x[sel], 8 * base[sel])
    rest = np.setdiff1d(np.arange(4096), sel)
    np.testing.assert_array_equal(x[rest], base[rest])


def test_weight_statistics_and_shapes():
    wl = PAIR_DEC_128K_BF16
    for li in range(2):
        w = gen.layer_weights(wl.with_sizes(d_model=512), li)
        assert w["W_c"].shape == (512, 512) and abs(w["W_c"].std() * np.sqrt(512) - 1) < 0.02
        assert w["W_UK"].shape == (64, 128, 512) and abs(w["W_UK"].std() * np.sqrt(512) - 1) < 0.02
    np.testing.assert_array_equal(gen.weight(wl, 0, "W_g"), gen.weight(wl, 0, "W_g"))


def test_streams_and_queries_are_rounded_projections():
    wl = PAIR_DEC_128K_BF16.with_sizes(N=512, d_model=256)
    x = gen.hidden_states(wl, 0)
    w = gen.layer_weights(wl, 0)
    st = gen.layer_streams(wl, 0, x, w)
    assert st["v"].shape == (512, 512) and st["vI"].shape == (512, 128)
    # bf16-exact values, within half a bf16 ulp of the fp64 projection
    for name, W in (("v", w["W_c"]), ("gI", w["W_gI"])):
        a = st[name]
        assert np.array_equal(a.view(np.uint32) & 0xFFFF, np.zeros_like(a, np.uint32))
        ref = x.astype(np.float64) @ W.T.astype(np.float64)
        assert np.all(np.abs(a - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    q = gen.layer_queries(wl, 0, x[-1:], w)
    assert q["q"].shape == (1, 64, 512) and q["qI"].shape == (1, 64, 128) and q["w"].shape == (1, 64)
    ref = np.einsum("hkd,hk->hd", w["W_UK"].astype(np.float64), q["q_heads"][0].astype(np.float64))
    assert np.all(np.abs(q["q"][0] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


def test_all_workloads_declared():
    names = [w.name for w in ALL]
    assert len(set(names)) == 5
    for w in ALL:
        for L in w.layers:
            assert L.W == 128
            if L.kind == "csa":
                assert (L.m, L.o) == (4, 4) and L.k > 0
            else:
                assert (L.m, L.o) == (128, 0)


def test_index_term_magnitude_and_score_check():
    """The score check's scale: sum_h |w_h| max(0, q_h . k) of the largest key."""
    from tests.compare import assert_scores_close, index_term_magnitude
    q = np.array([[1.0, 2.0], [3.0, -1.0]])          # two heads, D_I = 2
    w = np.array([-2.0, 0.5])
    keys = np.array([[1.0, 1.0], [0.0, -1.0]])
    # key 0: q.k = (3, 2) -> 2*3 + 0.5*2 = 7; key 1: (-2, 1) -> 0 + 0.5*1 = 0.5
    assert index_term_magnitude(q, w, keys) == 7.0
    scores = np.array([-2.0 * 3 + 0.5 * 2, 0.5])      # -5, 0.5
    assert_scores_close(scores + 1e-6, scores, q, w, keys, rtol=2e-6)
    with pytest.raises(AssertionError):
        assert_scores_close(scores + 1e-4, scores, q, w, keys, rtol=2e-6)

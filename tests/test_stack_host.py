"""Host logic of the layer stack without a GPU: the hybrid schedule and the
arena's memory plan."""
import pytest
import torch

from sequence_compressed_kv_amd import stack as stk

HCA = stk.StackLayer("hca", m=128, o=0, D=512, H=64, d_h=128, W=128)
CSA = stk.StackLayer("csa", m=4, o=4, D=512, H=64, d_h=128, W=128, H_I=64, D_I=128, k=1024)


def test_hybrid_schedule():
    kinds = [L.kind for L in stk.hybrid_schedule(9, CSA, HCA)]
    assert kinds == ["hca", "hca", "csa", "hca", "csa", "hca", "csa", "hca", "csa"]
    assert [L.kind for L in stk.hybrid_schedule(2, CSA, HCA)] == ["hca", "hca"]


def test_weight_shapes():
    s = stk.layer_weight_shapes(CSA, 4096)
    assert s["W_q"] == (8192, 4096) and s["W_o"] == (4096, 8192) and s["W_UK"] == (64, 128, 512)
    assert s["W_iq"] == (8192, 4096) and s["W_w"] == (64, 4096) and s["bposI"] == (8, 128)
    h = stk.layer_weight_shapes(stk.StackLayer("hca", 128, 0, 128, 32, 128), 2048)
    assert "W_UK" not in h and "W_iq" not in h          # latent = head dim: nothing to absorb


def test_arena_plan_is_aligned_and_disjoint():
    layers = stk.hybrid_schedule(4, CSA, HCA)
    weights = [{} for _ in layers]
    st = stk.Stack(layers, weights, 4096, B=2, N_max=1000, device="cpu")
    plan = st.plan
    assert len(plan) == 3 * 3 + 6                       # 3 HCA layers x 3 buffers, 1 CSA layer x 6
    spans = sorted((off, off + nb) for _, off, nb in plan)
    assert all(off % 256 == 0 for off, _ in spans)
    assert all(a_end <= b_off for (_, a_end), (b_off, _) in zip(spans, spans[1:]))
    assert spans[-1][1] == st.arena.size
    c = st.caches[2]
    assert c["entries"].shape == (2, 250, 512) and c["keys"].shape == (2, 256 // 32, 16, 32, 8)
    assert c["win"].shape == (2, 128, 512) and c["vI_ring"].shape == (2, 8, 128)
    assert st.caches[0]["entries"].shape == (2, 7, 512)
    # views alias the one allocation
    c["win"].fill_(1)
    assert int(st.arena.buf.view(torch.uint8).sum()) > 0


def test_window_ring_must_hold_a_pooling_window():
    bad = stk.StackLayer("hca", m=128, o=0, D=512, H=64, d_h=128, W=64)
    with pytest.raises(ValueError):
        stk.Stack([bad], [{}], 4096, B=1, N_max=512, device="cpu")


def test_arena_mxfp4_keys():
    """A CSA layer with MXFP4 keys reserves 17 D_I bytes per 32 entries and hands the
    calls an Mxfp4Keys view of them."""
    import dataclasses
    from sequence_compressed_kv_amd import _lib
    csa4 = dataclasses.replace(CSA, keys="mxfp4")
    st = stk.Stack(stk.hybrid_schedule(3, csa4, HCA), [{} for _ in range(3)], 4096, B=2, N_max=1000, device="cpu")
    k = st.caches[2]["keys"]
    assert isinstance(k, _lib.Mxfp4Keys) and k.D_I == 128 and k.E_cap == 256
    assert k.tiles.shape == (2, 8, 17 * 128) and k.tiles.dtype == torch.uint8
    (name, off, nb), = [p for p in st.plan if p[0] == "2.index_keys"]
    assert nb == 2 * 8 * 17 * 128 and off % 256 == 0
    with pytest.raises(ValueError):
        stk.Stack([dataclasses.replace(CSA, keys="e2m1")], [{}], 4096, B=1, N_max=512, device="cpu")

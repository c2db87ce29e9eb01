"""The decode step (index + top-k, CSA and HCA attention) captured in a HIP graph:
every replay, with eager work on the same buffers between the replays, writes the
same bits as the eager calls.  Covers the one-block top-k (batch of rows) and the
many-block top-k of a single long row (its histogram is cleared by a kernel, not a
memset)."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")
DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


@pytest.mark.parametrize("B,N,k", [(4, 16384, 256), (1, 160000, 2048)])
def test_step_graph_replays_equal_eager_calls(B, N, k):
    print(f"graph replay B={B} N={N} k={k}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(11 + B)
    bf = torch.bfloat16
    H, D, H_I, D_I, W = 64, 512, 64, 128, 128
    t = N - 1
    Ec, Eh = N // 4, N // 128
    keys = sk.to_key_tiles(torch.randn(B, Ec, D_I, device=DEV, generator=g).to(bf))
    ent_c = torch.randn(B, Ec, D, device=DEV, generator=g).to(bf)
    ent_h = torch.randn(B, Eh, D, device=DEV, generator=g).to(bf)
    win_c = torch.randn(B, W, D, device=DEV, generator=g).to(bf)
    win_h = torch.randn(B, W, D, device=DEV, generator=g).to(bf)

    def queries():
        return ((torch.randn(B, H_I, D_I, device=DEV, generator=g)).to(bf),
                torch.randn(B, H_I, device=DEV, generator=g),
                (torch.randn(B, H, D, device=DEV, generator=g) * 0.05).to(bf),
                (torch.randn(B, H, D, device=DEV, generator=g) * 0.05).to(bf))

    qI, w, qc, qh = queries()
    pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
    rows = sk.RowSpec.decode(pos, t)
    idx = torch.empty(B, k, dtype=torch.int32, device=DEV)
    out_c = torch.empty(B, H, D, device=DEV)
    out_h = torch.empty(B, H, D, device=DEV)
    tau = 1.0 / math.sqrt(128)
    ws_i = sk.csa_index_topk(rows, qI, w, keys, idx, m=4, W=W, k=k)
    ws_c = sk.csa_attend(rows, qc, ent_c, idx, win_c, out_c, m=4, W=W, softmax_scale=tau)
    ws_h = sk.hca_attend(rows, qh, ent_h, win_h, out_h, m=128, W=W, softmax_scale=tau)

    def step(a, b, c, d):
        sk.csa_index_topk(rows, a, b, keys, idx, m=4, W=W, k=k, workspace=ws_i)
        sk.csa_attend(rows, c, ent_c, idx, win_c, out_c, m=4, W=W, softmax_scale=tau, workspace=ws_c)
        sk.hca_attend(rows, d, ent_h, win_h, out_h, m=128, W=W, softmax_scale=tau, workspace=ws_h)

    step(qI, w, qc, qh)
    torch.cuda.synchronize()
    want = [idx.clone(), out_c.clone(), out_h.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(qI, w, qc, qh)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(qI, w, qc, qh)
    torch.cuda.synchronize()
    other = queries()
    for rep in range(4):
        # eager work on the same outputs and workspaces between the replays
        step(*other)
        torch.cuda.synchronize()
        assert not torch.equal(out_c, want[1])
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("idx", "out_c", "out_h"), (idx, out_c, out_h), want):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager call"

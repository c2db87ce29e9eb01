"""A random-weight layer stack (HCA, HCA, CSA, HCA) through the library, prefill
and decode, against the oracle run layer by layer.

Both sides store at the same points: every layer's hidden rows, streams,
queries, pooled entries, keys and attention outputs in bf16; the oracle computes
in fp64 between them.  The CSA layer keeps every visible entry (k >= E_vis), so
the selection is unique and the chain's result has no legitimate alternatives.
Differences come from fp32 accumulation and bf16 rounding flips, which the chain
carries forward; the tolerance per layer output is stated with the check."""
import numpy as np
import pytest
import torch

from oracle import codecs, method, pipeline
from tests.gpu_util import DEV, host

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")
from sequence_compressed_kv_amd import stack as stk  # noqa: E402

D_MODEL = 256
HCA = stk.StackLayer("hca", m=128, o=0, D=128, H=16, d_h=64, W=128)
CSA = stk.StackLayer("csa", m=4, o=4, D=128, H=16, d_h=64, W=128, H_I=32, D_I=64, k=256)
B, N = 2, 1100


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def make_weights(layers, seed=0):
    rng = np.random.default_rng(seed)
    out = []
    for L in layers:
        w = {}
        for name, shape in stk.layer_weight_shapes(L, D_MODEL).items():
            fan_in = D_MODEL if name.startswith("bpos") else shape[-1]
            a = rng.standard_normal(shape).astype(np.float32) / np.sqrt(fan_in)
            w[name] = a if name.startswith("bpos") else bf16(a)
        out.append(w)
    return out


def to_dev(w):
    return {k: torch.from_numpy(v).to(DEV).to(torch.float32 if k.startswith("bpos") else torch.bfloat16).contiguous()
            for k, v in w.items()}


def oracle_layer(L, w, x):
    """One layer for one sequence: x [n][d_model] (bf16 values) -> y [n][d_model] (fp64),
    every row causal."""
    n = x.shape[0]
    st = {"v": bf16(method.project(x, w["W_c"])), "g": bf16(method.project(x, w["W_g"]))}
    if L.kind == "csa":
        st["vI"] = bf16(method.project(x, w["W_cI"]))
        st["gI"] = bf16(method.project(x, w["W_gI"]))
    caches = pipeline.layer_caches(L, st, w, "bf16", L.keys if L.kind == "csa" else "bf16")
    qh = method.project(x, w["W_q"]).reshape(n, L.H, L.d_h)
    q = bf16(method.absorb_queries(qh, w["W_UK"]) if L.D != L.d_h else qh)
    qI = bf16(method.project(x, w["W_iq"]).reshape(n, L.H_I, L.D_I)) if L.kind == "csa" else None
    wI = method.project(x, w["W_w"]) if L.kind == "csa" else None
    y = np.empty((n, D_MODEL))
    for t in range(n):
        r = pipeline.decode_row(L, caches, st["v"], q[t], t, None if qI is None else qI[t],
                                None if wI is None else wI[t])
        if L.kind == "csa":
            assert (r["idx"] >= 0).sum() == r["e_vis"], "the test keeps every visible entry"
        y[t] = method.layer_output(bf16(r["o"]), w["W_o"], w.get("W_UV"))
    return y


def oracle_stack(layers, weights, x):
    """Every layer's output for every sequence: list over layers of [B][n][d_model]."""
    outs = []
    h = x
    for L, w in zip(layers, weights):
        y = np.stack([oracle_layer(L, w, h[b]) for b in range(h.shape[0])])
        outs.append(y)
        h = bf16(y)
    return outs


def normwise(g, o):
    return float(np.max(np.abs(g - o))) / max(float(np.max(np.abs(o))), 1e-30)


# bf16 rounding of every stored value is 2^-9 relative; a layer's output mixes
# thousands of such values with weights of both signs, and the chain carries the
# input's differences forward with a gain near one: 3e-2 of the output's largest
# magnitude per layer bounds the measured 1e-3 .. 1e-2 with margin, while a wrong
# entry, head or window item moves rows by O(1).
TOL = 3e-2


@pytest.mark.parametrize("keys", ["bf16", "mxfp4"])
def test_stack_prefill_and_decode(keys):
    """keys: the CSA layer's indexer key storage (MXFP4: FP4 blocks of 32 channels
    with a power-of-two scale; the oracle stores its keys the same way)."""
    import dataclasses
    layers = stk.hybrid_schedule(4, dataclasses.replace(CSA, keys=keys), HCA)
    assert [L.kind for L in layers] == ["hca", "hca", "csa", "hca"]
    w_host = make_weights(layers)
    rng = np.random.default_rng(1)
    x = bf16(rng.standard_normal((B, N, D_MODEL)).astype(np.float32))
    print(f"stack prefill B={B} N={N} layers={[L.kind for L in layers]} keys={keys}", flush=True)
    st = stk.Stack(layers, [to_dev(w) for w in w_host], D_MODEL, B, N_max=N + 100)
    names = [n for n, _, _ in st.plan]
    assert len(names) == len(set(names)) and all(off % 256 == 0 for _, off, _ in st.plan)
    # prefill N - 1 tokens, then decode token N - 1 through the stack
    xd = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    outs = st.prefill(xd[:, :N - 1].contiguous())
    dec = st.decode(xd[:, N - 1].contiguous(), torch.full((B,), N - 1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    ora = oracle_stack(layers, w_host, x)
    for li, L in enumerate(layers):
        g = host(outs[li])
        o = ora[li][:, :N - 1]
        err = normwise(g, o)
        err_d = normwise(host(dec[li]), ora[li][:, N - 1])
        print(f"layer {li} ({L.kind}): prefill err {err:.2e}  decode err {err_d:.2e}  max|y| {np.abs(o).max():.3f}",
              flush=True)
        assert np.isfinite(g).all()
        assert err <= TOL, f"layer {li} prefill: {err:.3e}"
        assert err_d <= TOL, f"layer {li} decode: {err_d:.3e}"


def test_stack_decode_steps_replay_as_graph():
    """Three decode steps eagerly, then the same steps captured once per position and
    replayed: identical outputs (every workspace of the step is preallocated)."""
    layers = stk.hybrid_schedule(3, CSA, HCA)
    w_host = make_weights(layers, seed=3)
    rng = np.random.default_rng(4)
    n0 = 600
    x = torch.from_numpy(bf16(rng.standard_normal((B, n0 + 3, D_MODEL)).astype(np.float32))).to(DEV).to(torch.bfloat16)
    st = stk.Stack(layers, [to_dev(w) for w in w_host], D_MODEL, B, N_max=n0 + 8)
    st.prefill(x[:, :n0].contiguous())
    snap = st.arena.buf.clone()
    pos = [torch.full((B,), n0 + i, dtype=torch.int32, device=DEV) for i in range(3)]
    xs = [x[:, n0 + i].contiguous() for i in range(3)]
    eager = []
    for i in range(3):
        eager.append(st.decode(xs[i], pos[i])[-1].clone())
    torch.cuda.synchronize()
    st.arena.buf.copy_(snap)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(3):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                st.decode(xs[i], pos[i])
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    st.arena.buf.copy_(snap)
    torch.cuda.synchronize()
    for i in range(3):
        graphs[i].replay()
        torch.cuda.synchronize()
        assert torch.equal(st._decode_ws[-1]["y"], eager[i]), f"step {i}"


def test_stack_layer_by_layer_with_selection_cut():
    """The CSA layer keeps 64 of up to 242 visible entries (k < E_vis), and every
    layer is checked against the oracle on the GPU's own inputs to that step, so
    no difference is carried from layer to layer: the stored entries and keys
    against the oracle's pool of the GPU's streams (code space); the selection of
    every row under the swap rule, with the oracle's scores over the GPU's keys
    and indexer queries; every row's attention over the GPU's caches, queries and
    selection within 2e-2 absolute; and the output projection of the GPU's
    attention outputs (bf16 output: 1e-2 of the largest magnitude)."""
    import dataclasses
    from tests.compare import bf16_code_flips, topk_parity
    csa = dataclasses.replace(CSA, k=64)
    layers = stk.hybrid_schedule(4, csa, HCA)
    w_host = make_weights(layers, seed=7)
    rng = np.random.default_rng(8)
    n = N
    x = bf16(rng.standard_normal((B, n, D_MODEL)).astype(np.float32))
    print(f"stack layer by layer B={B} N={n} layers={[L.kind for L in layers]} k={csa.k}", flush=True)
    st = stk.Stack(layers, [to_dev(w) for w in w_host], D_MODEL, B, N_max=n + 8)
    rec = []
    outs = st.prefill(torch.from_numpy(x).to(DEV).to(torch.bfloat16), record=rec)
    torch.cuda.synchronize()
    cut_rows = 0
    for li, L in enumerate(layers):
        w, t = w_host[li], rec[li]["t"]
        tau = 1.0 / np.sqrt(L.d_h)
        o_gpu = host(rec[li]["o"]).reshape(B, n, L.H, L.D)
        y_gpu = host(outs[li])
        worst = 0.0
        for b in range(B):
            r = slice(b * n, (b + 1) * n)
            v, g = host(t["v"][r]), host(t["g"][r])
            c = method.compress(v, g, w["bpos"], L.m, L.o)
            se = method.store_entries(c, "bf16")
            E = c.shape[0]
            ent = host(st.caches[li]["entries"][b])[:E]
            _, unexp = bf16_code_flips(ent, c, se["values"], magnitude=method.compress(np.abs(v), g, w["bpos"], L.m, L.o))
            assert unexp == 0, f"layer {li} seq {b}: {unexp} entry codes unexplained"
            q = host(t["q"][r])
            if L.kind == "csa":
                vI, gI = host(t["vI"][r]), host(t["gI"][r])
                cI = method.compress(vI, gI, w["bposI"], L.m, L.o)
                sI = method.store_keys(cI, "bf16")
                keys = host(sk.from_key_tiles(st.caches[li]["keys"][b:b + 1])[0])[:E]
                _, unexp = bf16_code_flips(keys, cI, sI["values"],
                                           magnitude=method.compress(np.abs(vI), gI, w["bposI"], L.m, L.o))
                assert unexp == 0, f"layer {li} seq {b}: {unexp} key codes unexplained"
                qI, wI, gidx = host(t["qI"][r]), host(t["w"][r]), host(rec[li]["idx"][b])
            for p in range(n):
                ev = min(method.entries_visible(p, L.m, L.W), E)
                if L.kind == "csa":
                    s = method.index_scores(qI[p], wI[p], keys[:ev])
                    ok, msg = topk_parity(gidx[p], method.topk(s, L.k), s)
                    assert ok, f"layer {li} seq {b} row {p} (E_vis={ev}): {msg}"
                    sel = gidx[p][gidx[p] >= 0]
                    cut_rows += int(len(sel) < ev)
                    items = np.concatenate([ent[sel], v[method.window_positions(p, L.W)]])
                else:
                    items = np.concatenate([ent[:ev], v[method.window_positions(p, L.W)]])
                oo, _, _ = method.attend(q[p], items, tau)
                err = float(np.max(np.abs(o_gpu[b, p] - oo)))
                worst = max(worst, err)
                assert err <= 2e-2, f"layer {li} seq {b} row {p}: attention error {err:.3e}"
            yo = np.stack([method.layer_output(o_gpu[b, p], w["W_o"], w.get("W_UV")) for p in range(n)])
            ey = normwise(y_gpu[b], yo)
            assert ey <= 1e-2, f"layer {li} seq {b}: output projection error {ey:.3e}"
        print(f"  layer {li} ({L.kind}): attention max abs err {worst:.2e}", flush=True)
    assert cut_rows > 1000, f"only {cut_rows} rows had more visible entries than k"

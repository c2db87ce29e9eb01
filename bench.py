"""Decode-step benchmark of the CSA + HCA layer pair at 128K context, batch 32.

One step = csa_index_topk (lightning-indexer scoring + top-1024) + csa_attend +
hca_attend for all 32 sequences, caches and queries resident in HBM.  Prints one JSON line:
queries/s, the step's HBM rate against the 8 TB/s peak, the roofline record of
the dominant kernel (indexer scoring: back-to-back launches timed with HIP
events on its stream; HBM traffic from a committed counter summary while the
kernel sources match it), the 32K causal prefill indexer rate against the bf16
MFMA peak, and the CPU oracle timed on a bounded sample of the same step.

Caches come from the seeded recipe of the full-size parity tests (x ~ N(0,1),
weights N(0, 1/fan_in), fp32 projections rounded to bf16, then the library's
own compressors) with hidden states drawn by torch on the GPU; compression is
not part of the timed step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0          # dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
STEP_COUNTERS = "pair_decode_128k_bf16.step_kernels.counters.txt"
STEP_1M_COUNTERS = "pair_decode_1m_fp8.step_kernels.counters.txt"
COMPRESS_COUNTERS = "compressors_128k_bf16_1m_fp8.counters.txt"
PREFILL_COUNTERS = "csa_prefill_32k_bf16.kernels.counters.txt"
FP4_COUNTERS = "pair_decode_128k_mxfp4_keys.step_kernels.counters.txt"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=2, help="cache copies rotated between steps (defeats the MALL)")
    ap.add_argument("--batch", type=int, default=None, help="override the batch (default 32)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill indexer measurement")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-context fp8 decode measurement")
    ap.add_argument("--no-append", action="store_true", help="skip the steady-state decode-with-appends measurement")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole-layer decode step (projections) measurement")
    ap.add_argument("--no-stack", action="store_true", help="skip the HCA prefill and the layer-stack measurements")
    ap.add_argument("--no-fp4", action="store_true", help="skip the decode step with MXFP4 indexer keys")
    ap.add_argument("--no-compress", action="store_true", help="skip the bulk compressor measurement")
    ap.add_argument("--only", choices=["prefill", "1m", "layer", "stack", "fp4", "compress"], default=None,
                    help="run only that side measurement and print its record (for profiling its kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def family_digest(family: str) -> str:
    """sha256 of a kernel family's sources (csrc/<family>.hip + device_common.h +
    sckv_internal.h): names the kernel version a committed counter summary was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in (family + ".hip", "device_common.h", "sckv_internal.h"):
        with open(os.path.join(ROOT, "sequence_compressed_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_counters(name: str) -> dict:
    """Per-kernel HBM bytes per launch from a committed counter summary under
    profiles/ (FETCH_SIZE and WRITE_SIZE passes, each scaled by a copy-kernel
    calibration): {kernel: {"traffic_B", "fetch_B", "write_B", "alg_B", "ratio",
    "profiled_us"}}.  A kernel whose sources no longer hash to the summary's digest
    reports traffic null ("stale": true): its counters describe other code."""
    out = {}
    try:
        with open(os.path.join(PROFILES, name)) as f:
            lines = [ln.split(None, 1)[1] for ln in f if ln.startswith("counter: ")]
    except OSError:
        return out
    digests = {}
    for ln in lines:
        label, *fields = ln.split()
        kv = dict(x.split("=", 1) for x in fields)
        fam = kv["family"]
        if fam not in digests:
            digests[fam] = family_digest(fam)
        fresh = kv["sha256"] == digests[fam]
        fe, wr, alg = float(kv["fetch_B"]), float(kv["write_B"]), float(kv["alg_B"])
        out[label] = {"traffic_B": fe + wr if fresh else None, "fetch_B": fe if fresh else None,
                      "write_B": wr if fresh else None, "alg_B": alg,
                      "ratio": (fe + wr) / alg if fresh else None, "profiled_us": float(kv["avg_us"]),
                      "stale": not fresh}
    return out


def step_graphs(torch, step, nvar: int, steps: int, per_graph: int = 10):
    """HIP graphs that together run step(0) .. step(steps - 1) when replayed in
    order: graphs of `chunk` consecutive steps (a multiple of nvar, the number of
    input variants step(i) cycles through, so every chunk starts at variant 0),
    then one of the remaining steps.  The library's kernels on preallocated
    workspaces (no allocation or memset inside); captured after an eager pass on a
    side stream of default priority.  Returns [(graph, n_steps), ...]."""
    chunk = max(nvar, (per_graph // nvar) * nvar)
    chunk = min(chunk, (steps // nvar) * nvar) or nvar
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nvar):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i)
        return g

    full = capture(chunk) if steps >= chunk else None
    plan = [(full, chunk)] * (steps // chunk) if full is not None else []
    rest = steps - chunk * len(plan)
    if rest:
        plan.append((capture(rest), rest))
    torch.cuda.synchronize()
    return plan


def replay_matches_eager(torch, step, nvar: int, plan, outputs) -> bool:
    """The first graph of the plan against the same steps run eagerly: the outputs
    after it (its last step) must agree bit for bit."""
    g, n = plan[0]
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    for t in outputs:
        t.fill_(7)
    g.replay()
    torch.cuda.synchronize()
    return all(torch.equal(a.view(torch.uint8) if a.dtype == torch.float8_e4m3fn else a,
                           b.view(torch.uint8) if b.dtype == torch.float8_e4m3fn else b)
               for a, b in zip(outputs, want))


def replay(plan):
    for g, _ in plan:
        g.replay()


def prefill_indexer_rate(dev, sk, torch, wl, iters: int = 5, fp4: bool = False):
    """Indexer scoring of the 32K-token causal prefill (every row scores its visible
    entries): algorithmic bf16 flops per second on MFMA.  Keys, queries and
    weights are random with the workload's shapes (the rate does not depend on
    the values).  fp4: the keys are MXFP4 tiles (random codes, scale bytes near
    2^0), dequantised to bf16 inside the kernel."""
    L = wl.layers[0]
    T, E = wl.N, wl.N // L.m
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    bf = torch.bfloat16
    if fp4:
        codes = torch.randint(0, 16, (1, E, L.D_I), device=dev, generator=g, dtype=torch.uint8)
        scale = torch.randint(124, 130, (1, E, L.D_I // 32), device=dev, generator=g, dtype=torch.uint8)
        keys = sk.mxfp4_pack(codes, scale)
    else:
        keys = sk.to_key_tiles(torch.randn(1, E, L.D_I, device=dev, generator=g).to(bf))
    qI = torch.randn(T, L.H_I, L.D_I, device=dev, generator=g).to(bf)
    w = torch.randn(T, L.H_I, device=dev, generator=g)
    cover = max(0, (T - 1 - L.W) // L.m)
    scores = torch.empty(T, (cover + 63) // 64 * 64, device=dev)
    rows = sk.RowSpec.causal(T)
    pairs = sum(max(0, (t - L.W) // L.m) for t in range(T))
    flops = 2.0 * pairs * L.H_I * L.D_I
    for _ in range(2):
        sk.csa_index_score(rows, qI, w, keys, scores, m=L.m, W=L.W, k=L.k)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        sk.csa_index_score(rows, qI, w, keys, scores, m=L.m, W=L.W, k=L.k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": wl.name + ("_mxfp4_keys" if fp4 else ""), "kernel": "index_score_causal_lds", "rows": T,
            "visible_pairs": pairs, "tflop": flops / 1e12, "ms": ms, "achieved_tflops": tf,
            "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS,
            "traffic_B": kernel_counters(PREFILL_COUNTERS).get(
                "index_score_causal_lds_" + ("mxfp4" if fp4 else "bf16") + "_keys", {}).get("traffic_B")}


def prefill_attend_rate(dev, sk, torch, wl, iters: int = 3):
    """CSA attention of the 32K-token causal prefill: every row t attends to its
    min(k, E_vis(t)) selected entries (spread evenly over the visible ones) plus
    its window.  Algorithmic flops on MFMA: (Q.K^T + P.V) x 2 per (row, item,
    head, latent dim); queries, entries and the stream are random with the
    workload's shapes (the rate does not depend on the values)."""
    L = wl.layers[0]
    T, E = wl.N, wl.N // L.m
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 17)
    bf = torch.bfloat16
    q = (torch.randn(T, L.H, L.D, device=dev, generator=g) * 0.3).to(bf)
    ent = torch.randn(1, E, L.D, device=dev, generator=g).to(bf)
    stream_v = torch.randn(1, T, L.D, device=dev, generator=g).to(bf)
    t = torch.arange(T, device=dev)
    ev = torch.clamp(torch.div(t - L.W, L.m, rounding_mode="floor"), min=0).clamp(max=E)
    kk = torch.clamp(ev, max=L.k)
    i = torch.arange(L.k, device=dev)
    idx = torch.div(i[None, :] * ev[:, None], kk.clamp(min=1)[:, None], rounding_mode="floor")
    idx = torch.where(i[None, :] < kk[:, None], idx, torch.full_like(idx, -1)).to(torch.int32).contiguous()
    items = int(kk.sum().item()) + sum(min(L.W, int(x) + 1) for x in range(T))
    flops = 4.0 * items * L.H * L.D
    out = torch.empty(T, L.H, L.D, device=dev)
    rows = sk.RowSpec.causal(T)
    tau = 1.0 / math.sqrt(L.d_h)
    ws = sk.csa_attend(rows, q, ent, idx, stream_v, out, m=L.m, W=L.W, softmax_scale=tau)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        sk.csa_attend(rows, q, ent, idx, stream_v, out, m=L.m, W=L.W, softmax_scale=tau, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": wl.name, "kernel": "attend_dma512", "rows": T, "row_items": items, "tflop": flops / 1e12,
            "ms": ms, "achieved_tflops": tf, "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS,
            "traffic_B": kernel_counters(PREFILL_COUNTERS).get("attend_dma512_prefill", {}).get("traffic_B")}


def prefill_projection_rate(dev, sk, torch, wl, iters: int = 3):
    """The projections of the 32K-token causal prefill layer: layer_inputs (W_q with
    the absorption into the latent, W_iq, W_w and the four stream weights) and
    layer_output (W_UV, W_o) over all 32768 rows, on the tiled bf16 GEMM.
    Algorithmic flops: 2 x rows x (in x out) of every product; the absorption
    counts its d_h x D product once (its two-part split runs it twice)."""
    L = wl.layers[0]
    T, dm = wl.N, wl.d_model
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 29)
    bf = torch.bfloat16

    def rnd(*shape, fan_in):
        return (torch.randn(*shape, device=dev, generator=g) / math.sqrt(fan_in)).to(bf)

    x = torch.randn(T, dm, device=dev, generator=g).to(bf)
    Wq, WUK, WUV = rnd(L.H * L.d_h, dm, fan_in=dm), rnd(L.H, L.d_h, L.D, fan_in=L.D), rnd(L.H, L.d_h, L.D, fan_in=L.D)
    Wo, Wiq, Ww = rnd(dm, L.H * L.d_h, fan_in=L.H * L.d_h), rnd(L.H_I * L.D_I, dm, fan_in=dm), rnd(L.H_I, dm, fan_in=dm)
    Wc, Wg, WcI, WgI = (rnd(L.D, dm, fan_in=dm), rnd(L.D, dm, fan_in=dm), rnd(L.D_I, dm, fan_in=dm),
                        rnd(L.D_I, dm, fan_in=dm))
    q = torch.empty(T, L.H, L.D, device=dev, dtype=bf)
    qI = torch.empty(T, L.H_I, L.D_I, device=dev, dtype=bf)
    w = torch.empty(T, L.H_I, device=dev)
    v, gg = torch.empty(T, L.D, device=dev, dtype=bf), torch.empty(T, L.D, device=dev, dtype=bf)
    vI, gI = torch.empty(T, L.D_I, device=dev, dtype=bf), torch.empty(T, L.D_I, device=dev, dtype=bf)
    o = (torch.randn(T, L.H, L.D, device=dev, generator=g) * 0.5).to(bf)
    y = torch.empty(T, dm, device=dev, dtype=bf)

    def inputs(ws=None):
        return sk.layer_inputs(x, Wq, q, W_UK=WUK, W_iq=Wiq, qI=qI, W_w=Ww, w=w, W_c=Wc, v=v, W_g=Wg, g=gg,
                               W_cI=WcI, vI=vI, W_gI=WgI, gI=gI, workspace=ws)

    def output(ws=None):
        return sk.layer_output(o, Wo, y, W_UV=WUV, workspace=ws)

    ws_in, ws_out = inputs(), output()
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms_in = timed(lambda: inputs(ws_in))
    ms_out = timed(lambda: output(ws_out))
    HD = L.H * L.d_h
    fl_in = 2.0 * T * (dm * (HD + L.H_I * L.D_I + L.H_I + 2 * L.D + 2 * L.D_I) + HD * L.D)
    fl_out = 2.0 * T * (HD * L.D + HD * dm)
    tf = (fl_in + fl_out) / ((ms_in + ms_out) * 1e-3) / 1e12
    return {"workload": wl.name, "kernel": "gemm_rows", "rows": T, "tflop": (fl_in + fl_out) / 1e12,
            "ms_layer_inputs": ms_in, "ms_layer_output": ms_out, "achieved_tflops": tf,
            "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}


def prefill_hca_attend_rate(dev, sk, torch, wl, iters: int = 3):
    """HCA attention of a 32K-token causal prefill with the 128K pair's HCA shapes
    (64 heads, latent 512, 128:1 pooling, window 128): row t attends densely to
    its E_vis(t) entries plus its window.  Flops as for the CSA prefill."""
    L = wl.layers[1]
    T = 32768
    E = T // L.m
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 23)
    bf = torch.bfloat16
    q = (torch.randn(T, L.H, L.D, device=dev, generator=g) * 0.3).to(bf)
    ent = torch.randn(1, E, L.D, device=dev, generator=g).to(bf)
    stream_v = torch.randn(1, T, L.D, device=dev, generator=g).to(bf)
    items = sum(min(E, max(0, (t - L.W) // L.m)) + min(L.W, t + 1) for t in range(T))
    flops = 4.0 * items * L.H * L.D
    out = torch.empty(T, L.H, L.D, device=dev, dtype=bf)
    rows = sk.RowSpec.causal(T)
    tau = 1.0 / math.sqrt(L.d_h)
    ws = sk.hca_attend(rows, q, ent, stream_v, out, m=L.m, W=L.W, softmax_scale=tau)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        sk.hca_attend(rows, q, ent, stream_v, out, m=L.m, W=L.W, softmax_scale=tau, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tf = flops / (ms * 1e-3) / 1e12
    return {"rows": T, "row_items": items, "tflop": flops / 1e12, "ms": ms, "achieved_tflops": tf,
            "peak_tflops": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}


def stack_weights(stk, layers, d_model, dev, torch, seed):
    """Random weights of every layer, N(0, 1/fan_in), drawn by torch on the GPU."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = []
    for L in layers:
        w = {}
        for name, shape in stk.layer_weight_shapes(L, d_model).items():
            fan_in = d_model if name.startswith("bpos") else shape[-1]
            t = torch.randn(*shape, device=dev, generator=g) / math.sqrt(fan_in)
            w[name] = t if name.startswith("bpos") else t.to(torch.bfloat16)
        out.append(w)
    return out


def stack_decode_rate(dev, sk, torch, n_layers: int = 8, B: int = 32, N: int = 131072, steps: int = 16,
                      replays: int = 5):
    """Decode through a random-weight stack of the hybrid schedule (HCA, HCA, then
    CSA / HCA alternating) with the 128K pair's layer shapes, batch 32: `steps`
    consecutive tokens, every layer appending, indexing (CSA) and attending.  The
    caches hold random bf16 values (the step's cost does not depend on them;
    filling 8 layers x 32 sequences x 128K tokens through the stack is a prefill of
    its own).  Timed eagerly and as one HIP graph of the steps; each run restores
    the rings first (about 100 MB of copies per 16 steps, inside the timing)."""
    from sequence_compressed_kv_amd import stack as stk
    from workloads import PAIR_DEC_128K_BF16

    c_, h_ = PAIR_DEC_128K_BF16.layers
    csa = stk.StackLayer("csa", c_.m, c_.o, c_.D, c_.H, c_.d_h, c_.W, c_.H_I, c_.D_I, c_.k)
    hca = stk.StackLayer("hca", h_.m, h_.o, h_.D, h_.H, h_.d_h, h_.W)
    layers = stk.hybrid_schedule(n_layers, csa, hca)
    dm = PAIR_DEC_128K_BF16.d_model
    st = stk.Stack(layers, stack_weights(stk, layers, dm, dev, torch, 101), dm, B, N_max=N)
    g = torch.Generator(device=dev)
    g.manual_seed(102)
    for c in st.caches:
        for t in c.values():
            for b in range(B):
                t[b].copy_(torch.randn(t[b].shape, device=dev, generator=g))
    xs = [torch.randn(B, dm, device=dev, generator=g).to(torch.bfloat16) for _ in range(steps)]
    pos = [torch.full((B,), N - steps + i, dtype=torch.int32, device=dev) for i in range(steps)]
    # the rings as of position N - steps - 1: each run starts from them (a run's later
    # tokens overwrite the window slots its earlier steps read); the entry caches
    # need no reset, as re-appending the same tokens rewrites the same entries
    ring_names = ("win", "g_ring", "vI_ring", "gI_ring")
    rings0 = [{k: c[k].clone() for k in ring_names if k in c} for c in st.caches]

    def run():
        for c, r0 in zip(st.caches, rings0):
            for k, v in r0.items():
                c[k].copy_(v)
        for i in range(steps):
            st.decode(xs[i], pos[i])

    stream = torch.cuda.current_stream()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / steps

    run()
    torch.cuda.synchronize()
    ref = st._decode_ws[-1]["y"].clone()
    ms_eager = timed(run, replays)
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gr, stream=cap):
            run()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(st._decode_ws[-1]["y"], ref))
    ms_graph = timed(gr.replay, replays)
    return {"layers": [L.kind for L in layers], "batch": B, "context": N, "steps": steps,
            "cache_arena_bytes": st.arena.size, "ms_per_step_eager": ms_eager, "ms_per_step_graph": ms_graph,
            "tokens_per_s_graph": B / (ms_graph * 1e-3), "graph_matches_eager": same}


def stack_prefill_rate(dev, sk, torch, n_layers: int = 4, N: int = 32768, iters: int = 2):
    """Prefill of one 32K-token sequence through a random-weight stack (HCA, HCA, CSA,
    HCA) with the 32K prefill layer's shapes (CSA top-512): every layer's
    projections (tiled GEMM), compression, causal indexing and top-k (CSA),
    causal attention and output projections."""
    from sequence_compressed_kv_amd import stack as stk
    from workloads import CSA_PREFILL_32K_BF16, PAIR_DEC_128K_BF16

    c_ = CSA_PREFILL_32K_BF16.layers[0]
    h_ = PAIR_DEC_128K_BF16.layers[1]
    csa = stk.StackLayer("csa", c_.m, c_.o, c_.D, c_.H, c_.d_h, c_.W, c_.H_I, c_.D_I, c_.k)
    hca = stk.StackLayer("hca", h_.m, h_.o, h_.D, h_.H, h_.d_h, h_.W)
    layers = stk.hybrid_schedule(n_layers, csa, hca)
    dm = CSA_PREFILL_32K_BF16.d_model
    st = stk.Stack(layers, stack_weights(stk, layers, dm, dev, torch, 103), dm, 1, N_max=N)
    g = torch.Generator(device=dev)
    g.manual_seed(104)
    x = torch.randn(1, N, dm, device=dev, generator=g).to(torch.bfloat16)
    outs = st.prefill(x)
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(outs[-1].float()).all())
    del outs
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        st.prefill(x)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return {"layers": [L.kind for L in layers], "tokens": N, "ms": ms, "tokens_per_s": N / (ms * 1e-3),
            "outputs_finite": finite}


def build_caches(wl, dev, sk, torch, gen, tail: int = 0, fp4_keys: bool = False):
    """Caches of every sequence for both layers (GPU-drawn streams, library compressors).
    With tail > 0 the last `tail` tokens of every stream are returned too (third
    value: per layer, a dict of [B][tail][D] tensors) for decode appends.  With
    fp4_keys the indexer stream is also pooled into MXFP4 key tiles (c["keys_fp4"])."""
    B = wl.B
    csa, hca = wl.layers
    bf = torch.bfloat16
    Ec, Eh = wl.N // csa.m, wl.N // hca.m
    c = {"entries": torch.empty(B, Ec, csa.D, device=dev, dtype=bf),
         "keys": sk.key_tiles_empty(B, Ec, csa.D_I, bf, dev),
         "win": torch.empty(B, csa.W, csa.D, device=dev, dtype=bf)}
    h = {"entries": torch.empty(B, Eh, hca.D, device=dev, dtype=bf),
         "win": torch.empty(B, hca.W, hca.D, device=dev, dtype=bf)}
    if fp4_keys:
        c["keys_fp4"] = sk.Mxfp4Keys.empty(B, Ec, csa.D_I, dev)
    weights = gen.gpu_weights(wl, dev)
    wc, wh = weights
    slots = torch.arange(wl.N - csa.W, wl.N, device=dev) % csa.W
    tails = None
    if tail:
        tails = [{n: torch.empty(B, tail, wc[n].shape[0], device=dev, dtype=bf) for n in ("v", "g", "vI", "gI")},
                 {n: torch.empty(B, tail, wh[n].shape[0], device=dev, dtype=bf) for n in ("v", "g")}]
    for b in range(B):
        st_c, st_h = gen.gpu_sequence_streams(wl, b, weights, dev)
        if tail:
            for st, tl in zip((st_c, st_h), tails):
                for n in tl:
                    tl[n][b] = st[n][wl.N - tail:]
        kv = sk.Pool(st_c["v"][None], st_c["g"][None], wc["bpos"].contiguous(), c["entries"][b:b + 1])
        ix = sk.Pool(st_c["vI"][None], st_c["gI"][None], wc["bposI"].contiguous(), c["keys"][b:b + 1],
                     layout=sk.LAYOUT_KEY_TILES)
        sk.csa_compress(kv, ix, m=csa.m, o=csa.o)
        if fp4_keys:
            k4 = sk.Mxfp4Keys(c["keys_fp4"].tiles[b:b + 1], csa.D_I)
            sk.csa_compress(sk.Pool(st_c["vI"][None], st_c["gI"][None], wc["bposI"].contiguous(), k4,
                                    layout=sk.LAYOUT_KEY_TILES), m=csa.m, o=csa.o)
        sk.hca_compress(sk.Pool(st_h["v"][None], st_h["g"][None], wh["bpos"].contiguous(), h["entries"][b:b + 1]),
                        m=hca.m, o=hca.o)
        c["win"][b, slots] = st_c["v"][wl.N - csa.W:]
        h["win"][b, slots] = st_h["v"][wl.N - hca.W:]
        del st_c, st_h
    torch.cuda.synchronize()
    if tail:
        return c, h, tails, weights
    return c, h


def decode_append_rate(dev, sk, torch, wl, c, h, tails, weights, qc, qh, steps: int = 128, replays: int = 5):
    """Steady-state decode of the pair: `steps` consecutive tokens (the last ones
    of every sequence, re-appended at their own positions) each appended to the
    rings and caches (csa_append for the latent and indexer streams, hca_append)
    before the step's index, top-k and attention.  Timed eagerly and as one HIP
    graph of all the steps; the caches after the appends must equal the ones the
    bulk compressors built."""
    csa, hca = wl.layers
    B, N = wl.B, wl.N
    t0 = N - steps
    bf = torch.bfloat16
    wc, wh = weights
    P_lat = csa.W                                          # the window ring doubles as the value ring
    before = {k: v.clone() for k, v in c.items() if k != "keys_fp4"}, {k: v.clone() for k, v in h.items()}
    tl_c, tl_h = tails
    T = tl_c["v"].shape[1]
    # rings as of position t0 - 1 (slot = position mod P)
    pos_r = torch.arange(t0 - P_lat, t0, device=dev)
    ring0 = {"win_c": torch.empty_like(c["win"]), "win_h": torch.empty_like(h["win"]),
             "g_c": torch.empty(B, P_lat, csa.D, device=dev, dtype=bf),
             "g_h": torch.empty(B, hca.m, hca.D, device=dev, dtype=bf),
             "vI": torch.empty(B, csa.m + csa.o, csa.D_I, device=dev, dtype=bf),
             "gI": torch.empty(B, csa.m + csa.o, csa.D_I, device=dev, dtype=bf)}
    src = pos_r - (N - T)
    ring0["win_c"][:, pos_r % P_lat] = tl_c["v"][:, src]
    ring0["g_c"][:, pos_r % P_lat] = tl_c["g"][:, src]
    ring0["win_h"][:, pos_r % hca.W] = tl_h["v"][:, src]
    ring0["g_h"][:, pos_r % hca.m] = tl_h["g"][:, src]
    pi = torch.arange(t0 - (csa.m + csa.o), t0, device=dev)
    ring0["vI"][:, pi % (csa.m + csa.o)] = tl_c["vI"][:, pi - (N - T)]
    ring0["gI"][:, pi % (csa.m + csa.o)] = tl_c["gI"][:, pi - (N - T)]
    rings = {k: v.clone() for k, v in ring0.items()}
    rings["win_c"], rings["win_h"] = c["win"], h["win"]    # the attention reads the live window rings
    pos = [torch.full((B,), t, dtype=torch.int32, device=dev) for t in range(t0, N)]
    idx = torch.empty(B, csa.k, dtype=torch.int32, device=dev)
    out_c = torch.empty(B, csa.H, csa.D, device=dev)
    out_h = torch.empty(B, hca.H, hca.D, device=dev)
    tau = 1.0 / math.sqrt(csa.d_h)
    rows0 = sk.RowSpec.decode(pos[-1], N - 1)
    ws_i = sk.csa_index_topk(rows0, qc["qI"], qc["w"], c["keys"], idx, m=csa.m, W=csa.W, k=csa.k)
    ws_c = sk.csa_attend(rows0, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau)
    ws_h = sk.hca_attend(rows0, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau)
    new = [{n: tl_c[n][:, t - (N - T)].contiguous() for n in tl_c} | {"vh": tl_h["v"][:, t - (N - T)].contiguous(),
           "gh": tl_h["g"][:, t - (N - T)].contiguous()} for t in range(t0, N)]

    def reset():
        for k in ("win_c", "win_h", "g_c", "g_h", "vI", "gI"):
            rings[k].copy_(ring0[k])

    def step(s):
        p, x = pos[s], new[s]
        sk.csa_append(sk.Append(p, x["v"], x["g"], rings["win_c"], rings["g_c"], wc["bpos"], c["entries"]),
                      sk.Append(p, x["vI"], x["gI"], rings["vI"], rings["gI"], wc["bposI"], c["keys"],
                                layout=sk.LAYOUT_KEY_TILES), m=csa.m, o=csa.o)
        sk.hca_append(sk.Append(p, x["vh"], x["gh"], rings["win_h"], rings["g_h"], wh["bpos"], h["entries"]),
                      m=hca.m, o=hca.o)
        rows = sk.RowSpec.decode(p, N - 1)
        sk.csa_index_topk(rows, qc["qI"], qc["w"], c["keys"], idx, m=csa.m, W=csa.W, k=csa.k, workspace=ws_i)
        sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau,
                      workspace=ws_c)
        sk.hca_attend(rows, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau,
                      workspace=ws_h)

    def run():
        reset()
        for s_ in range(steps):
            step(s_)

    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()
    same_caches = all(torch.equal(before[0][k], c[k]) for k in before[0]) and all(torch.equal(before[1][k], h[k]) for k in h)
    ref_c, ref_h = out_c.clone(), out_h.clone()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / steps

    ms_eager = timed(run, replays)
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    out_c.zero_()
    out_h.zero_()
    g.replay()
    torch.cuda.synchronize()
    same_graph = bool(torch.equal(out_c, ref_c) and torch.equal(out_h, ref_h))
    ms_graph = timed(g.replay, replays)
    by_append = (3 * csa.D * 2 + 2 * csa.D_I * 2 + 2 * hca.D * 2) * B       # new tokens in, ring slots out
    return {"workload": wl.name, "steps": steps, "positions": [t0, N - 1], "ms_per_step_eager": ms_eager,
            "ms_per_step_graph": ms_graph, "queries_per_s_graph": B / (ms_graph * 1e-3),
            "caches_equal_bulk_compress": same_caches, "graph_matches_eager": same_graph,
            "append_bytes_per_step": by_append}


def decode_layer_rate(dev, sk, torch, wl, c, h, weights, steps: int = 32, replays: int = 5):
    """The whole decode step of the layer pair, hidden rows x_t in, layer outputs y out:
    per layer layer_inputs (queries, absorbed into the latent, and the token's
    streams in one launch), the append of the token, index + top-k (CSA), attention
    (bf16 out) and layer_output (W_UV heads, W_o).  Both layers take the same
    hidden rows (norms, residuals and the MLP between layers are not part of the
    path).  Every step appends at t = N - 1, so each emits a CSA and an HCA entry.
    Timed eagerly and as a HIP graph of `steps` steps; the projection calls are
    also timed alone, against the bytes of the weights they stream."""
    csa, hca = wl.layers
    B, N, dm = wl.B, wl.N, wl.d_model
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed * 7919 + 17)

    def rnd(*shape, fan_in):
        return (torch.randn(*shape, device=dev, generator=g) / math.sqrt(fan_in)).to(bf)

    wc, wh = weights
    Wc = {"W_q": rnd(csa.H * csa.d_h, dm, fan_in=dm), "W_UK": rnd(csa.H, csa.d_h, csa.D, fan_in=csa.D),
          "W_UV": rnd(csa.H, csa.d_h, csa.D, fan_in=csa.D), "W_o": rnd(dm, csa.H * csa.d_h, fan_in=csa.H * csa.d_h),
          "W_iq": rnd(csa.H_I * csa.D_I, dm, fan_in=dm), "W_w": rnd(csa.H_I, dm, fan_in=dm),
          "W_c": wc["v"].to(bf), "W_g": wc["g"].to(bf), "W_cI": wc["vI"].to(bf), "W_gI": wc["gI"].to(bf)}
    Wh = {"W_q": rnd(hca.H * hca.d_h, dm, fan_in=dm), "W_UK": rnd(hca.H, hca.d_h, hca.D, fan_in=hca.D),
          "W_UV": rnd(hca.H, hca.d_h, hca.D, fan_in=hca.D), "W_o": rnd(dm, hca.H * hca.d_h, fan_in=hca.H * hca.d_h),
          "W_c": wh["v"].to(bf), "W_g": wh["g"].to(bf)}
    wbytes = sum(t.numel() * 2 for t in Wc.values()) + sum(t.numel() * 2 for t in Wh.values())
    x = torch.randn(B, dm, device=dev, generator=g).to(bf)
    pos = torch.full((B,), N - 1, dtype=torch.int32, device=dev)
    rows = sk.RowSpec.decode(pos, N - 1)
    e = lambda *s, dt=bf: torch.zeros(*s, device=dev, dtype=dt)
    t_c = {"q": e(B, csa.H, csa.D), "qI": e(B, csa.H_I, csa.D_I), "w": e(B, csa.H_I, dt=torch.float32),
           "v": e(B, csa.D), "g": e(B, csa.D), "vI": e(B, csa.D_I), "gI": e(B, csa.D_I), "o": e(B, csa.H, csa.D),
           "y": e(B, dm), "g_ring": e(B, csa.W, csa.D), "vI_ring": e(B, csa.m + csa.o, csa.D_I),
           "gI_ring": e(B, csa.m + csa.o, csa.D_I), "idx": e(B, csa.k, dt=torch.int32)}
    t_h = {"q": e(B, hca.H, hca.D), "v": e(B, hca.D), "g": e(B, hca.D), "o": e(B, hca.H, hca.D), "y": e(B, dm),
           "g_ring": e(B, hca.m + hca.o, hca.D)}
    tau = 1.0 / math.sqrt(csa.d_h)

    def inputs_c(ws=None):
        return sk.layer_inputs(x, Wc["W_q"], t_c["q"], W_UK=Wc["W_UK"], W_iq=Wc["W_iq"], qI=t_c["qI"], W_w=Wc["W_w"],
                               w=t_c["w"], W_c=Wc["W_c"], v=t_c["v"], W_g=Wc["W_g"], g=t_c["g"], W_cI=Wc["W_cI"],
                               vI=t_c["vI"], W_gI=Wc["W_gI"], gI=t_c["gI"], workspace=ws)

    def inputs_h(ws=None):
        return sk.layer_inputs(x, Wh["W_q"], t_h["q"], W_UK=Wh["W_UK"], W_c=Wh["W_c"], v=t_h["v"], W_g=Wh["W_g"],
                               g=t_h["g"], workspace=ws)

    def output_c(ws=None):
        return sk.layer_output(t_c["o"], Wc["W_o"], t_c["y"], W_UV=Wc["W_UV"], workspace=ws)

    def output_h(ws=None):
        return sk.layer_output(t_h["o"], Wh["W_o"], t_h["y"], W_UV=Wh["W_UV"], workspace=ws)

    ws = {"in_c": inputs_c(), "in_h": inputs_h(), "out_c": output_c(), "out_h": output_h()}
    ws["idx"] = sk.csa_index_topk(rows, t_c["qI"], t_c["w"], c["keys"], t_c["idx"], m=csa.m, W=csa.W, k=csa.k)
    ws["att_c"] = sk.csa_attend(rows, t_c["q"], c["entries"], t_c["idx"], c["win"], t_c["o"], m=csa.m, W=csa.W,
                                softmax_scale=tau)
    ws["att_h"] = sk.hca_attend(rows, t_h["q"], h["entries"], h["win"], t_h["o"], m=hca.m, W=hca.W, softmax_scale=tau)

    def projections():
        inputs_c(ws["in_c"])
        output_c(ws["out_c"])
        inputs_h(ws["in_h"])
        output_h(ws["out_h"])

    def step():
        inputs_c(ws["in_c"])
        sk.csa_append(sk.Append(pos, t_c["v"], t_c["g"], c["win"], t_c["g_ring"], wc["bpos"], c["entries"]),
                      sk.Append(pos, t_c["vI"], t_c["gI"], t_c["vI_ring"], t_c["gI_ring"], wc["bposI"], c["keys"],
                                layout=sk.LAYOUT_KEY_TILES), m=csa.m, o=csa.o)
        sk.csa_index_topk(rows, t_c["qI"], t_c["w"], c["keys"], t_c["idx"], m=csa.m, W=csa.W, k=csa.k,
                          workspace=ws["idx"])
        sk.csa_attend(rows, t_c["q"], c["entries"], t_c["idx"], c["win"], t_c["o"], m=csa.m, W=csa.W,
                      softmax_scale=tau, workspace=ws["att_c"])
        output_c(ws["out_c"])
        inputs_h(ws["in_h"])
        sk.hca_append(sk.Append(pos, t_h["v"], t_h["g"], h["win"], t_h["g_ring"], wh["bpos"], h["entries"]),
                      m=hca.m, o=hca.o)
        sk.hca_attend(rows, t_h["q"], h["entries"], h["win"], t_h["o"], m=hca.m, W=hca.W, softmax_scale=tau,
                      workspace=ws["att_h"])
        output_h(ws["out_h"])

    def run():
        for _ in range(steps):
            step()

    stream = torch.cuda.current_stream()

    def timed(fn, n, per):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / per

    run()
    torch.cuda.synchronize()
    ref = (t_c["y"].clone(), t_h["y"].clone())
    finite = bool(torch.isfinite(ref[0].float()).all() and torch.isfinite(ref[1].float()).all())
    ms_eager = timed(run, replays, steps)
    ms_proj = timed(projections, replays * steps, 1)
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gr, stream=cap):
            run()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    t_c["y"].zero_()
    t_h["y"].zero_()
    gr.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(t_c["y"], ref[0]) and torch.equal(t_h["y"], ref[1]))
    ms_graph = timed(gr.replay, replays, steps)
    return {"workload": wl.name, "steps": steps, "ms_per_step_eager": ms_eager, "ms_per_step_graph": ms_graph,
            "tokens_per_s_graph": B / (ms_graph * 1e-3), "graph_matches_eager": same, "outputs_finite": finite,
            "projections_ms_eager": ms_proj, "projection_weight_bytes": wbytes,
            "projection_weight_GBps": wbytes / (ms_proj * 1e-3) / 1e9}


def decode_1m_rate(dev, sk, torch, gen, steps: int = 20, replicas: int = 4, fp4: bool = False):
    """Decode step of the 1M-context pair (batch 1) with fp8 caches: index + top-2048,
    CSA and HCA attention, bf16 out.  Cache replicas are rotated (the pair cache is
    smaller than the 256 MiB MALL).  fp4: the indexer keys are MXFP4 tiles (68
    bytes per key) instead of unscaled e4m3 (128 bytes)."""
    from workloads import PAIR_DEC_1M_FP8 as wl
    csa, hca = wl.layers
    t = wl.N - 1
    Ec, Eh = wl.N // csa.m, wl.N // hca.m
    f8, bf = torch.float8_e4m3fn, torch.bfloat16
    weights = gen.gpu_weights(wl, dev)
    s_c, s_h = gen.gpu_sequence_streams(wl, 0, weights, dev)
    c = {"ent": torch.empty(1, Ec, csa.D, device=dev, dtype=torch.uint8).view(f8),
         "sc": torch.empty(1, Ec, device=dev),
         "keys": (sk.Mxfp4Keys.empty(1, Ec, csa.D_I, dev) if fp4
                  else sk.key_tiles_empty(1, Ec, csa.D_I, torch.uint8, dev).view(f8)),
         "win": torch.empty(1, csa.W, csa.D, device=dev, dtype=bf)}
    h = {"ent": torch.empty(1, Eh, hca.D, device=dev, dtype=torch.uint8).view(f8),
         "sc": torch.empty(1, Eh, device=dev),
         "win": torch.empty(1, hca.W, hca.D, device=dev, dtype=bf)}
    sk.csa_compress(sk.Pool(s_c["v"][None], s_c["g"][None], weights[0]["bpos"].contiguous(), c["ent"], c["sc"]),
                    sk.Pool(s_c["vI"][None], s_c["gI"][None], weights[0]["bposI"].contiguous(), c["keys"],
                            layout=sk.LAYOUT_KEY_TILES), m=csa.m, o=csa.o)
    sk.hca_compress(sk.Pool(s_h["v"][None], s_h["g"][None], weights[1]["bpos"].contiguous(), h["ent"], h["sc"]),
                    m=hca.m, o=hca.o)
    slots = torch.arange(wl.N - csa.W, wl.N, device=dev) % csa.W
    c["win"][0, slots] = s_c["v"][wl.N - csa.W:]
    h["win"][0, slots] = s_h["v"][wl.N - hca.W:]
    del s_c, s_h
    reps = [(c, h)] + [({k: v.clone() for k, v in c.items()}, {k: v.clone() for k, v in h.items()})
                       for _ in range(replicas - 1)]
    qc, qh = gen.gpu_queries(wl, 0, 1, dev), gen.gpu_queries(wl, 1, 1, dev)
    rows = sk.RowSpec.decode(torch.tensor([t], dtype=torch.int32, device=dev), t)
    idx = torch.empty(1, csa.k, dtype=torch.int32, device=dev)
    out_c = torch.empty(1, csa.H, csa.D, device=dev, dtype=bf)
    out_h = torch.empty(1, hca.H, hca.D, device=dev, dtype=bf)
    tau = 1.0 / math.sqrt(csa.d_h)
    ws_i = sk.csa_index_topk(rows, qc["qI"], qc["w"], c["keys"], idx, m=csa.m, W=csa.W, k=csa.k)
    ws_c = sk.csa_attend(rows, qc["q"], c["ent"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau,
                         entry_scale=c["sc"])
    ws_h = sk.hca_attend(rows, qh["q"], h["ent"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau,
                         entry_scale=h["sc"])

    def step(i):
        cc, hh = reps[i % len(reps)]
        sk.csa_index_topk(rows, qc["qI"], qc["w"], cc["keys"], idx, m=csa.m, W=csa.W, k=csa.k, workspace=ws_i)
        sk.csa_attend(rows, qc["q"], cc["ent"], idx, cc["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau,
                      entry_scale=cc["sc"], workspace=ws_c)
        sk.hca_attend(rows, qh["q"], hh["ent"], hh["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau,
                      entry_scale=hh["sc"], workspace=ws_h)

    for i in range(5):
        step(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    plan = step_graphs(torch, step, len(reps), steps)
    graph_ok = replay_matches_eager(torch, step, len(reps), plan, [idx, out_c, out_h])
    replay(plan)
    torch.cuda.synchronize()
    e0.record(stream)
    replay(plan)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev_c, ev_h = (t - csa.W) // csa.m, (t - hca.W) // hca.m
    nwin = csa.W
    key_bytes = csa.D_I // 2 + csa.D_I // 32 if fp4 else csa.D_I
    by = (ev_c * key_bytes + csa.H_I * csa.D_I * 2 + csa.H_I * 4 + csa.k * 4                     # indexer + top-k
          + csa.k * (csa.D + 4) + nwin * csa.D * 2 + csa.H * csa.D * 2 * 2                       # CSA attention
          + ev_h * (hca.D + 4) + nwin * hca.D * 2 + hca.H * hca.D * 2 * 2)                       # HCA attention
    gbps = by / (ms * 1e-3) / 1e9
    return {"workload": wl.name + ("_mxfp4_keys" if fp4 else ""), "batch": 1, "context": wl.N,
            "key_bytes": key_bytes, "replicas": replicas, "ms_per_step": ms,
            "queries_per_s": 1.0 / (ms * 1e-3), "algorithmic_bytes": by, "hbm_GBps": gbps,
            "hbm_frac": gbps / PEAK_HBM_GBPS, "step_launch": "hip_graph_replay",
            "graph_replay_equals_eager": graph_ok, "eager_ms_per_step": eager_ms,
            "kernel_traffic": kernel_counters(STEP_1M_COUNTERS)}


def compress_rates(dev, sk, torch, gen, iters: int = 20):
    """The bulk compressors on one sequence's streams, as the caches are built: the
    128K pair's (CSA latent and indexer streams into bf16 entries and key tiles in
    one call, the HCA stream into bf16 entries) and the 1M pair's pre-population
    (e4m3 entries with per-entry scales and unscaled e4m3 keys).  Algorithmic bytes
    per call: each stream's values and gate logits read once, the entries (and
    scales) written."""
    from workloads import PAIR_DEC_128K_BF16, PAIR_DEC_1M_FP8
    out = {}
    stream = torch.cuda.current_stream()
    for wl, f8 in ((PAIR_DEC_128K_BF16, False), (PAIR_DEC_1M_FP8, True)):
        csa, hca = wl.layers
        N = wl.N
        Ec, Eh = N // csa.m, N // hca.m
        weights = gen.gpu_weights(wl, dev)
        s_c, s_h = gen.gpu_sequence_streams(wl, 0, weights, dev)
        if f8:
            u8, f8t = torch.uint8, torch.float8_e4m3fn
            ent_c = torch.empty(1, Ec, csa.D, device=dev, dtype=u8).view(f8t)
            keys = sk.key_tiles_empty(1, Ec, csa.D_I, u8, dev).view(f8t)
            ent_h = torch.empty(1, Eh, hca.D, device=dev, dtype=u8).view(f8t)
            sc_c, sc_h = torch.empty(1, Ec, device=dev), torch.empty(1, Eh, device=dev)
            esz = 1
        else:
            bf = torch.bfloat16
            ent_c = torch.empty(1, Ec, csa.D, device=dev, dtype=bf)
            keys = sk.key_tiles_empty(1, Ec, csa.D_I, bf, dev)
            ent_h = torch.empty(1, Eh, hca.D, device=dev, dtype=bf)
            sc_c = sc_h = None
            esz = 2
        kv = sk.Pool(s_c["v"][None], s_c["g"][None], weights[0]["bpos"].contiguous(), ent_c, sc_c)
        ix = sk.Pool(s_c["vI"][None], s_c["gI"][None], weights[0]["bposI"].contiguous(), keys,
                     layout=sk.LAYOUT_KEY_TILES)
        hk = sk.Pool(s_h["v"][None], s_h["g"][None], weights[1]["bpos"].contiguous(), ent_h, sc_h)
        scale_b = 4 if f8 else 0
        calls = {
            "csa": (lambda: sk.csa_compress(kv, ix, m=csa.m, o=csa.o),
                    2 * N * (csa.D + csa.D_I) * 2 + Ec * (csa.D * esz + scale_b + csa.D_I * esz)),
            "hca": (lambda: sk.hca_compress(hk, m=hca.m, o=hca.o), 2 * N * hca.D * 2 + Eh * (hca.D * esz + scale_b)),
        }
        for name, (fn, nbytes) in calls.items():
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(iters):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / iters
            gbps = nbytes / (ms * 1e-3) / 1e9
            out[f"{name}_{wl.name}"] = {"tokens": N, "entries": Ec if name == "csa" else Eh, "ms": ms,
                                        "algorithmic_bytes": nbytes, "GBps": gbps, "frac": gbps / PEAK_HBM_GBPS}
        del s_c, s_h, kv, ix, hk, ent_c, ent_h, keys
        torch.cuda.empty_cache()
    out["kernel_traffic"] = kernel_counters(COMPRESS_COUNTERS)
    return out


def decode_fp4_rate(dev, sk, torch, wl, c, h, qc, qh, steps: int = 50, replicas: int = 2):
    """The 128K-context decode step with the lightning indexer's keys in MXFP4 (FP4
    e2m1 codes in blocks of 32 channels with a power-of-two scale byte: 68 bytes per
    128-dim key against 256 in bf16); attention caches as in the bf16 step.  Key
    replicas are rotated as in the main step."""
    csa, hca = wl.layers
    B = wl.B
    t = wl.N - 1
    keys = [c["keys_fp4"]] + [sk.Mxfp4Keys(c["keys_fp4"].tiles.clone(), csa.D_I) for _ in range(replicas - 1)]
    pos = torch.full((B,), t, dtype=torch.int32, device=dev)
    rows = sk.RowSpec.decode(pos, t)
    idx = torch.empty(B, csa.k, dtype=torch.int32, device=dev)
    out_c = torch.empty(B, csa.H, csa.D, device=dev, dtype=torch.float32)
    out_h = torch.empty(B, hca.H, hca.D, device=dev, dtype=torch.float32)
    tau = 1.0 / math.sqrt(csa.d_h)
    ws_i = sk.csa_index_topk(rows, qc["qI"], qc["w"], keys[0], idx, m=csa.m, W=csa.W, k=csa.k)
    ws_c = sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau)
    ws_h = sk.hca_attend(rows, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau)
    cover = max(0, (t - csa.W) // csa.m)
    scores = torch.empty(B, (cover + 63) // 64 * 64, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        sk.csa_index_topk(rows, qc["qI"], qc["w"], keys[i % len(keys)], idx, m=csa.m, W=csa.W, k=csa.k,
                          workspace=ws_i)
        if ev is not None:
            ev[1].record(stream)
        sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau,
                      workspace=ws_c)
        sk.hca_attend(rows, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau,
                      workspace=ws_h)

    for i in range(10):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    topk_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(steps):
        sk.csa_index_score(rows, qc["qI"], qc["w"], keys[i % len(keys)], scores, m=csa.m, W=csa.W, k=csa.k)
    s1.record(stream)
    torch.cuda.synchronize()
    score_ms = s0.elapsed_time(s1) / steps
    plan = step_graphs(torch, step, len(keys), steps)
    graph_ok = replay_matches_eager(torch, step, len(keys), plan, [idx, out_c, out_h])
    replay(plan)
    torch.cuda.synchronize()
    e0.record(stream)
    replay(plan)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ab = algorithmic_bytes(wl)
    key_bytes = csa.D_I // 2 + csa.D_I // 32                   # e2m1 codes + one scale byte per 32 channels
    score_by = (cover * key_bytes + csa.H_I * csa.D_I * 2 + csa.H_I * 4) * B
    step_by = (ab["step"] - ab["score"]) * B + score_by
    score_gbps = score_by / (score_ms * 1e-3) / 1e9
    step_gbps = step_by / (ms * 1e-3) / 1e9
    return {"workload": wl.name + "_mxfp4_keys", "batch": B, "context": wl.N, "key_bytes": key_bytes,
            "replicas": replicas, "ms_per_step": ms, "queries_per_s": B / (ms * 1e-3),
            "step_launch": "hip_graph_replay", "graph_replay_equals_eager": graph_ok, "eager_ms_per_step": eager_ms,
            "index_topk_ms": topk_ms, "step_algorithmic_bytes": step_by, "step_hbm_GBps": step_gbps,
            "step_hbm_frac": step_gbps / PEAK_HBM_GBPS,
            "index_score": {"kernel": "index_score_decode (MXFP4 keys)", "launch_ms": score_ms,
                            "bytes_per_launch": score_by, "achieved_GBps": score_gbps,
                            "frac": score_gbps / PEAK_HBM_GBPS},
            "kernel_traffic": kernel_counters(FP4_COUNTERS)}


def algorithmic_bytes(wl):
    """Bytes one decode query must move (reads of the data it uses, writes of its results)."""
    csa, hca = wl.layers
    t = wl.N - 1
    ev_c = max(0, (t - csa.W) // csa.m)
    ev_h = max(0, (t - hca.W) // hca.m)
    nwin = min(csa.W, t + 1)
    b16 = 2
    score = ev_c * csa.D_I * b16 + csa.H_I * csa.D_I * b16 + csa.H_I * 4      # keys + indexer query + weights
    topk = csa.k * 4                                                           # indices written
    csa_att = (csa.k * csa.D + nwin * csa.D + csa.H * csa.D) * b16 + csa.k * 4 + csa.H * csa.D * 4
    hca_att = (ev_h * hca.D + nwin * hca.D + hca.H * hca.D) * b16 + hca.H * hca.D * 4
    return {"score": score, "topk": topk, "csa_attend": csa_att, "hca_attend": hca_att,
            "step": score + topk + csa_att + hca_att}


def hbm_read_reference(torch, dev, gib: int = 2, iters: int = 10):
    """Plain streaming references on the same GPU, timed with HIP events: the
    hand-written streaming read (libsckv_bench.so: every byte of `gib` GiB read once
    with 16-byte loads, 2048 blocks of 256 threads), torch's sum over the same bf16
    tensor and a device copy of it (each byte read once and written once), and the
    hand-written row gathers (`row_gather_1KB`: random 1 KB rows of the buffer).
    `GBps` is the streaming read's rate."""
    import ctypes as C
    x = torch.ones(gib * (1 << 30) // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    blib = C.CDLL(os.path.join(ROOT, "sequence_compressed_kv_amd", "libsckv_bench.so"))
    blib.sckv_bench_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    blib.sckv_bench_stream_read.restype = C.c_int
    sink = torch.empty(2048, dtype=torch.int32, device=dev)

    def kernel_read():
        e = blib.sckv_bench_stream_read(x.data_ptr(), x.numel() * 2, sink.data_ptr(), 2048, stream.cuda_stream)
        if e != 0:
            raise RuntimeError(f"streaming-read reference failed: hipError {e}")

    def rate(fn, nbytes):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) / iters * 1e-3) / 1e9

    nb = x.numel() * 2
    kread = rate(kernel_read, nb)
    read = rate(lambda: x.sum(), nb)
    copy = rate(lambda: y.copy_(x), 2 * nb)

    # random 1 KB rows of the same buffer, gathered 32 to a chunk by blocks of 8
    # waves as decode attention gathers its items: through the asynchronous
    # global -> LDS copies (three chunks in flight) and with loads into registers
    # (one chunk in flight); the shapes of one 128K-context attention launch
    # (192 blocks x 6 chunks) and of a long gather (256 blocks x 45 chunks)
    blib.sckv_bench_gather_rows.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                            C.c_void_p]
    blib.sckv_bench_gather_rows.restype = C.c_int
    nrows = nb // 1024
    g = torch.Generator(device=dev).manual_seed(11)
    gather = {}
    for blocks, nch in ((192, 6), (256, 45)):
        rows = torch.randint(0, nrows, (blocks * nch * 32,), device=dev, generator=g, dtype=torch.int32)
        for mode, name in ((1, "lds_copy"), (0, "registers")):
            def run(mode=mode, rows=rows, blocks=blocks, nch=nch):
                e = blib.sckv_bench_gather_rows(x.data_ptr(), rows.data_ptr(), blocks, nch, mode, sink.data_ptr(),
                                                stream.cuda_stream)
                if e != 0:
                    raise RuntimeError(f"row-gather reference failed: hipError {e}")
            gather[f"{name}_{blocks}x{nch}_GBps"] = rate(run, blocks * nch * 32 * 1024)
    del x, y
    return {"stream_read_kernel_GBps": kread, "sum_read_GBps": read, "copy_GBps": copy, "bytes": nb, "GBps": kread,
            "row_gather_1KB": gather}


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"cpu_count": os.cpu_count(), "model": model}


def cpu_baseline(wl, budget_s: float):
    """The oracle (numpy fp64) on one sequence of the same workload, timed on the host
    with all BLAS threads and with one."""
    import numpy as np

    from oracle import method, pipeline
    from workloads import gen

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = os.cpu_count()
    csa, hca = wl.layers
    t0 = time.time()
    x = gen.hidden_states(wl, 0)
    prep = []
    for li, L in enumerate(wl.layers):
        w = gen.layer_weights(wl, li)
        st = gen.layer_streams(wl, li, x, w)
        q = gen.layer_queries(wl, li, x[wl.N - 1:], w)
        caches = pipeline.layer_caches(L, st, w, wl.entry_store, wl.key_store)
        prep.append((L, caches, st["v"], q))
    del x
    setup_s = time.time() - t0
    t = wl.N - 1
    n = 0
    t1 = time.time()
    while True:
        for L, caches, v, q in prep:
            if L.kind == "csa":
                pipeline.decode_row(L, caches, v, q["q"][0], t, q["qI"][0], q["w"][0])
            else:
                pipeline.decode_row(L, caches, v, q["q"][0], t)
        n += 1
        el = time.time() - t1
        if el >= budget_s:
            break
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, t2 = 0, time.time()
            while True:
                for L, caches, v, q in prep:
                    if L.kind == "csa":
                        pipeline.decode_row(L, caches, v, q["q"][0], t, q["qI"][0], q["w"][0])
                    else:
                        pipeline.decode_row(L, caches, v, q["q"][0], t)
                n1 += 1
                el1 = time.time() - t2
                if el1 >= budget_s / 2:
                    break
        one = n1 / el1
    return {"value": n / el, "unit": "queries/s", "cores": int(cores), "kind": "oracle",
            "value_1thread": one, "host": host_cpu(),
            "sample": f"{n} decode queries of sequence 0 (CSA top-{csa.k} + HCA, fp64 numpy) in {el:.1f} s with "
                      f"{int(cores)} threads (and {budget_s / 2:.0f} s on one thread); cache preparation "
                      f"{setup_s:.0f} s untimed"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU: the decode path shards by sequence with no exchange, and only the "
              "single-GPU share is built and measured here; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        x = torch.empty(256 * 1024 * 1024 // 4, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4, "launches": 5}))
        return

    import sequence_compressed_kv_amd as sk
    from workloads import CSA_PREFILL_32K_BF16, PAIR_DEC_128K_BF16, gen

    if args.only == "prefill":
        print(json.dumps({"prefill_indexer": prefill_indexer_rate("cuda:0", sk, torch, CSA_PREFILL_32K_BF16),
                          "prefill_indexer_fp4": prefill_indexer_rate("cuda:0", sk, torch, CSA_PREFILL_32K_BF16,
                                                                      fp4=True),
                          "prefill_attend": prefill_attend_rate("cuda:0", sk, torch, CSA_PREFILL_32K_BF16),
                          "prefill_projections": prefill_projection_rate("cuda:0", sk, torch,
                                                                         CSA_PREFILL_32K_BF16)}))
        return
    if args.only == "1m":
        print(json.dumps({"decode_1m_fp8": decode_1m_rate("cuda:0", sk, torch, gen),
                          "decode_1m_fp8_mxfp4_keys": decode_1m_rate("cuda:0", sk, torch, gen, fp4=True)}))
        return
    if args.only == "compress":
        print(json.dumps({"compress": compress_rates("cuda:0", sk, torch, gen)}))
        return
    if args.only == "stack":
        print(json.dumps({"prefill_hca_attend": prefill_hca_attend_rate("cuda:0", sk, torch, PAIR_DEC_128K_BF16),
                          "stack_prefill": stack_prefill_rate("cuda:0", sk, torch),
                          "stack_decode": stack_decode_rate("cuda:0", sk, torch)}))
        return

    wl = PAIR_DEC_128K_BF16 if args.batch is None else PAIR_DEC_128K_BF16.with_sizes(B=args.batch)
    dev = "cuda:0"
    sk.load()
    csa, hca = wl.layers
    B = wl.B
    t = wl.N - 1
    print(f"[bench] building caches: B={B} N={wl.N}", file=sys.stderr, flush=True)
    tb = time.time()
    fp4 = (not args.no_fp4 and args.only is None) or args.only == "fp4"
    c0, h0, tails, weights = build_caches(wl, dev, sk, torch, gen, tail=256, fp4_keys=fp4)
    reps = [(c0, h0)] + [({k: v.clone() for k, v in c0.items() if k != "keys_fp4"},
                          {k: v.clone() for k, v in h0.items()}) for _ in range(args.replicas - 1)]
    qc = gen.gpu_queries(wl, 0, B, dev)
    qh = gen.gpu_queries(wl, 1, B, dev)
    print(f"[bench] caches ready in {time.time() - tb:.1f} s", file=sys.stderr, flush=True)
    if args.only == "layer":
        print(json.dumps({"decode_layer": decode_layer_rate(dev, sk, torch, wl, c0, h0, weights)}), flush=True)
        return
    if args.only == "fp4":
        print(json.dumps({"decode_fp4_keys": decode_fp4_rate(dev, sk, torch, wl, c0, h0, qc, qh)}), flush=True)
        return

    pos = torch.full((B,), t, dtype=torch.int32, device=dev)
    rows = sk.RowSpec.decode(pos, t)
    idx = torch.empty(B, csa.k, dtype=torch.int32, device=dev)
    out_c = torch.empty(B, csa.H, csa.D, device=dev, dtype=torch.float32)
    out_h = torch.empty(B, hca.H, hca.D, device=dev, dtype=torch.float32)
    tau = 1.0 / math.sqrt(csa.d_h)
    ia = sk.index_args(rows, qc["qI"], qc["w"], c0["keys"], idx, m=csa.m, W=csa.W, k=csa.k)
    L = sk.load()
    import ctypes as C
    ws_idx = torch.empty(L.csa_index_topk_workspace_size(C.byref(ia)), dtype=torch.uint8, device=dev)
    cover = max(0, (t - csa.W) // csa.m)
    stride = (cover + 63) // 64 * 64
    scores = torch.empty(B, stride, device=dev)             # for timing the scoring kernel alone
    ws_c = sk.csa_attend(rows, qc["q"], c0["entries"], idx, c0["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau)
    ws_h = sk.hca_attend(rows, qh["q"], h0["entries"], h0["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau)

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        c, h = reps[i % len(reps)]
        if ev is not None:
            ev[0].record(stream)
        sk.csa_index_topk(rows, qc["qI"], qc["w"], c["keys"], idx, m=csa.m, W=csa.W, k=csa.k, workspace=ws_idx)
        if ev is not None:
            ev[1].record(stream)
        sk.csa_attend(rows, qc["q"], c["entries"], idx, c["win"], out_c, m=csa.m, W=csa.W, softmax_scale=tau,
                      workspace=ws_c)
        if ev is not None:
            ev[2].record(stream)
        sk.hca_attend(rows, qh["q"], h["entries"], h["win"], out_h, m=hca.m, W=hca.W, softmax_scale=tau,
                      workspace=ws_h)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # eager steps (each call marshals its arguments in Python)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    # per-kernel durations: the same steps with events between the launches
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    parts = {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
             for j, name in enumerate(["csa_index_topk", "csa_attend", "hca_attend"])}

    # the dominant kernel alone: back-to-back launches on the same stream between
    # two events (per-launch time without the event/launch gaps of the step)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(args.steps):
        c, _ = reps[i % len(reps)]
        sk.csa_index_score(rows, qc["qI"], qc["w"], c["keys"], scores, m=csa.m, W=csa.W, k=csa.k)
    s1.record(stream)
    torch.cuda.synchronize()
    score_ms = s0.elapsed_time(s1) / args.steps
    # timed region: K whole steps, each a replay of the step's HIP graph (the way a
    # serving loop launches it: no host work between the kernels)
    plan = step_graphs(torch, step, len(reps), args.steps)
    graph_ok = replay_matches_eager(torch, step, len(reps), plan, [idx, out_c, out_h])
    replay(plan)
    torch.cuda.synchronize()
    w0 = time.time()
    e0.record(stream)
    replay(plan)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.time() - w0
    ms = e0.elapsed_time(e1) / args.steps

    ab = algorithmic_bytes(wl)
    ctr = kernel_counters(STEP_COUNTERS)
    score_gbps = ab["score"] * B / (score_ms * 1e-3) / 1e9
    step_gbps = ab["step"] * B / (ms * 1e-3) / 1e9
    rec = {
        "metric": "CSA+HCA decode attention queries/s at 128K ctx; HBM GB/s as % of peak",
        "value": B / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "context": wl.N, "layers": "csa+hca", "heads": csa.H,
                   "latent": csa.D, "indexer": f"{csa.H_I}x{csa.D_I}", "top_k": csa.k, "window": csa.W,
                   "replicas": args.replicas},
        "step_hbm_GBps": step_gbps, "step_hbm_frac": step_gbps / PEAK_HBM_GBPS,
        "step_launch": "hip_graph_replay", "graph_replay_equals_eager": graph_ok, "eager_ms_per_step": eager_ms,
        "step_algorithmic_bytes": ab["step"] * B,
        "kernel_ms": parts,
        "roofline": {"bound": "hbm", "kernel": "index_score_decode", "launch_ms": score_ms, "achieved": score_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": score_gbps / PEAK_HBM_GBPS,
                     "traffic": ctr.get("index_score_decode", {}).get("traffic_B"),
                     "bytes_per_launch": ab["score"] * B},
        "kernel_traffic": ctr,
        "wall_s_timed": wall,
    }
    rd = hbm_read_reference(torch, dev)
    rec["hbm_read_reference"] = rd
    rec["step_frac_of_read"] = step_gbps / rd["GBps"]
    rec["roofline"]["frac_of_read"] = score_gbps / rd["GBps"]
    if not args.no_compress:
        print("[bench] bulk compressors (128K and 1M sequences)", file=sys.stderr, flush=True)
        rec["compress"] = compress_rates(dev, sk, torch, gen)
    if not args.no_append:
        print("[bench] steady-state decode with appends", file=sys.stderr, flush=True)
        rec["decode_append"] = decode_append_rate(dev, sk, torch, wl, c0, h0, tails, weights, qc, qh)
    del tails
    if fp4:
        print("[bench] decode step with MXFP4 indexer keys", file=sys.stderr, flush=True)
        rec["decode_fp4_keys"] = decode_fp4_rate(dev, sk, torch, wl, c0, h0, qc, qh)
    if not args.no_layer:
        print("[bench] whole decode layer step (projections in and out)", file=sys.stderr, flush=True)
        rec["decode_layer"] = decode_layer_rate(dev, sk, torch, wl, c0, h0, weights)
    if not args.no_prefill:
        print("[bench] prefill indexer scoring (32K causal rows)", file=sys.stderr, flush=True)
        del reps, c0, h0
        torch.cuda.empty_cache()
        rec["prefill_indexer"] = prefill_indexer_rate(dev, sk, torch, CSA_PREFILL_32K_BF16)
        torch.cuda.empty_cache()
        rec["prefill_indexer_fp4"] = prefill_indexer_rate(dev, sk, torch, CSA_PREFILL_32K_BF16, fp4=True)
        torch.cuda.empty_cache()
        rec["prefill_attend"] = prefill_attend_rate(dev, sk, torch, CSA_PREFILL_32K_BF16)
        torch.cuda.empty_cache()
        rec["prefill_projections"] = prefill_projection_rate(dev, sk, torch, CSA_PREFILL_32K_BF16)
    if not args.no_stack:
        print("[bench] HCA prefill attention and the layer stack (prefill, decode)", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        rec["prefill_hca_attend"] = prefill_hca_attend_rate(dev, sk, torch, wl)
        torch.cuda.empty_cache()
        rec["stack_prefill"] = stack_prefill_rate(dev, sk, torch)
        torch.cuda.empty_cache()
        rec["stack_decode"] = stack_decode_rate(dev, sk, torch)
    if not args.no_1m:
        print("[bench] 1M-context fp8 decode step", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        rec["decode_1m_fp8"] = decode_1m_rate(dev, sk, torch, gen)
        torch.cuda.empty_cache()
        rec["decode_1m_fp8_mxfp4_keys"] = decode_1m_rate(dev, sk, torch, gen, fp4=True)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

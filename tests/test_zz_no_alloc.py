"""The allocation-free index entry point (csa_index_topk_noalloc) against the one
that takes a workspace (csa_index_topk): two calls in a row on the library's
static scratch, the second smaller than the first, each bit for bit equal to the
workspace call on the same inputs; then rows that do not fit are refused."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, dev_i32

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("sequence_compressed_kv_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load()


def _inputs(seed, R, E_cap, HI=64, DI=128, keys="bf16"):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(R, HI, DI, device=DEV, generator=g).to(torch.bfloat16)
    w = torch.randn(R, HI, device=DEV, generator=g)
    kv = torch.randn(max(R, 1), E_cap, DI, device=DEV, generator=g)
    if keys == "e4m3":
        kv = kv.clamp(-448, 448).to(torch.float8_e4m3fn)
    else:
        kv = kv.to(torch.bfloat16)
    return q, w, sk.to_key_tiles(kv)


def _both(rows, q, w, keys, k):
    R = rows.R
    ref_i = torch.full((R, k), -7, device=DEV, dtype=torch.int32)
    ref_s = torch.zeros(R, k, device=DEV)
    got_i = torch.full((R, k), -9, device=DEV, dtype=torch.int32)
    got_s = torch.zeros(R, k, device=DEV)
    sk.csa_index_topk(rows, q, w, keys, ref_i, m=4, W=128, k=k, out_score=ref_s)
    sk.csa_index_topk_noalloc(rows, q, w, keys, got_i, m=4, W=128, k=k, out_score=got_s)
    torch.cuda.synchronize()
    return ref_i, ref_s, got_i, got_s


def _check(name, ref_i, ref_s, got_i, got_s):
    assert torch.equal(ref_i, got_i), f"{name}: indices differ from csa_index_topk"
    assert torch.equal(ref_s, got_s), f"{name}: scores differ from csa_index_topk"
    print(f"  {name}: {int((ref_i >= 0).sum())} kept entries equal", flush=True)


def test_noalloc_matches_workspace_call_twice_then_smaller():
    # call 1: one decode row at 1M context (262,111 visible entries, top-2048: the
    # many-block selection, about 3 MB of scratch)
    print("noalloc call 1: 1 row, 262144 entries, k=2048", flush=True)
    t1 = 1048575
    q, w, keys = _inputs(11, 1, 262144)
    rows = sk.RowSpec.decode(dev_i32([t1]), t1)
    _check("1M row", *_both(rows, q, w, keys, 2048))
    # call 2, smaller: five decode rows at different positions (one with nothing visible),
    # e4m3 keys; the scratch still holds call 1's scores beyond these rows
    print("noalloc call 2: 5 rows, 8192 entries, k=256", flush=True)
    pos = [32767, 20000, 4223, 300, 100]
    q, w, keys = _inputs(12, 5, 8192, keys="e4m3")
    rows = sk.RowSpec.decode(dev_i32(pos), max(pos))
    _check("5 decode rows", *_both(rows, q, w, keys, 256))
    # call 3: causal rows (prefill-style), 64 rows near position 16000
    print("noalloc call 3: 64 causal rows, k=128", flush=True)
    q, w, keys = _inputs(13, 64, 4096)
    q = q[:64].contiguous()
    rows = sk.RowSpec.causal(64, pos0=16000)
    _check("64 causal rows", *_both(rows, q, w, keys[:1].contiguous(), 128))


def test_noalloc_refuses_rows_beyond_its_scratch():
    print("noalloc: rows beyond the scratch are refused", flush=True)
    R = 2048
    q, w, keys = _inputs(14, 1, 8192)
    q = q.expand(R, -1, -1).contiguous()
    w = w.expand(R, -1).contiguous()
    rows = sk.RowSpec.causal(R, pos0=32000)
    out = torch.full((R, 64), -7, device=DEV, dtype=torch.int32)
    with pytest.raises(sk.SckvError) as e:
        sk.csa_index_topk_noalloc(rows, q, w, keys, out, m=4, W=128, k=64)
    assert e.value.status == 6 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == -7).all()), "a refused call wrote its output"

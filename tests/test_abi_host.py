"""The C ABI without a GPU: the library loads, exports every declared call, and
rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

import sequence_compressed_kv_amd as sk
from sequence_compressed_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only checks pass fake device pointers; run where no GPU is visible")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sk.lib_path()):
        from sequence_compressed_kv_amd import build       # nothing built yet: hipcc compiles without a GPU
        build.build()
    return sk.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "sckv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:sckv_status|size_t|const char\*|int32_t)\s+(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTS), decl
    for name in decl:
        assert hasattr(L, name), name
    assert L.sckv_abi_version() == 1


FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation fails first
FAKE_ODD = 0x10004


def pool(**kw):
    d = dict(val=FAKE, gate=FAKE, bpos=FAKE, out=FAKE, out_scale=None, E_cap=16, D=64, in_dtype=1, out_dtype=1,
             out_layout=0)
    d.update(kw)
    return _lib.PoolStream(**d)


def err(L):
    return L.sckv_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(val=None), 1), (dict(out=None), 1), (dict(in_dtype=2), 3), (dict(out_dtype=7), 3),
    (dict(D=48), 4), (dict(D=1024), 4), (dict(E_cap=3), 2), (dict(val=FAKE_ODD), 5),
    (dict(out_layout=1, E_cap=48), 2), (dict(out_layout=7), 2),
    # MXFP4 keys: tiles only, D >= 32, no out_scale (the scales sit in the tiles)
    (dict(out_dtype=3), 4), (dict(out_dtype=3, out_layout=1, E_cap=32, out_scale=FAKE), 4),
    (dict(out_dtype=3, out_layout=1, E_cap=32, D=16), 4),
])
def test_compress_validation(L, kw, status):
    p = pool(**kw)
    s = L.csa_compress(1, 64, 4, 4, 0, 16, C.byref(p), None, None)
    assert s == status, err(L)
    assert err(L)


def test_compress_token_range(L):
    p = pool()
    assert L.csa_compress(1, 63, 4, 4, 0, 16, C.byref(p), None, None) == 2     # entry 15 needs 64 tokens
    assert L.hca_compress(0, 64, 4, 0, 0, 1, C.byref(p), None) == 2             # B = 0
    assert L.hca_compress(1, 64, 0, 0, 0, 1, C.byref(p), None) == 2             # m = 0
    assert L.csa_compress(1, 64, 4, -1, 0, 1, C.byref(p), None, None) == 2      # o < 0
    assert L.csa_compress(1, 64, 4, 4, -1, 1, C.byref(p), None, None) == 2
    bad = pool(bpos=None)
    assert L.csa_compress(1, 64, 4, 4, 0, 16, C.byref(p), C.byref(bad), None) == 1
    assert L.csa_compress(1, 64, 4, 4, 0, 16, None, None, None) == 1


def app(**kw):
    d = dict(pos=FAKE, val=FAKE, gate=FAKE, val_ring=FAKE, gate_ring=FAKE, bpos=FAKE, out=FAKE, out_scale=None,
             E_cap=16, D=64, P=8, in_dtype=1, out_dtype=1, out_layout=0, reserved=0)
    d.update(kw)
    return _lib.AppendStream(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(pos=None), 1), (dict(gate_ring=None), 1), (dict(val_ring=None), 1), (dict(in_dtype=2), 3),
    (dict(out_dtype=9), 3), (dict(D=24), 4), (dict(P=7), 2), (dict(E_cap=0), 2),
    (dict(out_layout=1, E_cap=40), 2), (dict(gate_ring=FAKE_ODD), 5), (dict(out_scale=FAKE_ODD, out_dtype=2), 5),
    (dict(out_dtype=3), 4),
])
def test_append_validation(L, kw, status):
    a = app(**kw)
    assert L.csa_append(2, 4, 4, C.byref(a), None, None) == status, err(L)
    assert err(L)


def test_append_pool_and_counts(L):
    a = app()
    assert L.csa_append(0, 4, 4, C.byref(a), None, None) == 2                   # B = 0
    assert L.csa_append(2, 0, 4, C.byref(a), None, None) == 2                   # m = 0
    assert L.hca_append(2, 128, 0, C.byref(a), None) == 2                      # P = 8 < 128 ring slots
    bad_idx = app(bpos=None)
    assert L.csa_append(2, 4, 4, C.byref(a), C.byref(bad_idx), None) == 1       # the index stream is checked too
    assert L.csa_append(2, 4, 4, None, None, None) == 1
    assert L.hca_append(2, 128, 0, C.byref(app(P=127)), None) == 2
    assert L.hca_append(2, 128, 0, C.byref(app(P=128, val=None)), None) == 1


def idx_args(**kw):
    rows = kw.pop("rows", _lib.Rows(FAKE, 0, 2, 4095, 0, 0, 0))
    d = dict(rows=rows, q=FAKE, w=FAKE, keys=FAKE, out_idx=FAKE, out_score=None, E_cap=1024, B=2, H_I=64, D_I=128,
             q_dtype=1, key_dtype=1, m=4, W=128, k=64)
    d.update(kw)
    return _lib.IndexArgs(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out_idx=None), 1), (dict(k=0), 2), (dict(m=0), 2), (dict(E_cap=0), 2),
    (dict(q_dtype=0), 3), (dict(key_dtype=0), 3), (dict(H_I=48), 4), (dict(D_I=96), 4),
    (dict(q_dtype=0, key_dtype=0, H_I=128, D_I=128), 4), (dict(keys=FAKE_ODD), 5), (dict(E_cap=1000), 2),
    (dict(rows=_lib.Rows(None, 0, 2, 4095, 0, 0, 0)), 1), (dict(rows=_lib.Rows(FAKE, 0, 3, 4095, 0, 0, 0)), 2),
    (dict(rows=_lib.Rows(None, 1, 8, 0, 2, 0, 0)), 2), (dict(rows=_lib.Rows(None, 5, 8, 0, 0, 0, 0)), 2),
    # MXFP4 keys need bf16 queries and the MFMA shapes
    (dict(key_dtype=3, q_dtype=0), 3), (dict(key_dtype=3, D_I=96), 4),
])
def test_index_validation(L, kw, status):
    a = idx_args(**kw)
    assert L.csa_index_topk(C.byref(a), FAKE, 1 << 30, None) == status, err(L)
    if "out_idx" not in kw:                  # the size query does not need the output pointer
        assert L.csa_index_topk_workspace_size(C.byref(a)) == 0


def test_index_mxfp4_rows_accepted(L):
    """MXFP4 keys with bf16 queries pass validation for decode and causal rows."""
    for rows in (_lib.Rows(FAKE, 0, 2, 4095, 0, 0, 0), _lib.Rows(None, 1, 8, 0, 0, 100, 0)):
        a = idx_args(key_dtype=3, rows=rows)
        assert L.csa_index_topk_workspace_size(C.byref(a)) > 0, err(L)


def test_index_workspace(L):
    a = idx_args()
    n = L.csa_index_topk_workspace_size(C.byref(a))
    # scores of 2 rows x 991 visible entries (padded to 1024 floats)
    assert n >= 2 * 991 * 4
    assert L.csa_index_topk(C.byref(a), FAKE, n - 1, None) == 6
    assert L.csa_index_topk(C.byref(a), None, n, None) == 6
    assert L.csa_index_score(C.byref(a), None, 1024, None) == 1
    assert L.csa_index_score(C.byref(a), FAKE, 990, None) == 2          # stride below the visible count


def test_topk_plan_limits(L):
    # decode at t = 2^22 (1,048,544 visible entries, k = 4096): many blocks per row
    a = idx_args(rows=_lib.Rows(FAKE, 0, 1, 1 << 22, 0, 0, 0), E_cap=1 << 20, k=4096)
    assert L.csa_index_topk_workspace_size(C.byref(a)) > 1048544 * 4
    # t = 2^25 with 2^23 entries: more than 1024 blocks of 4096 per row, and slices
    # whose candidates exceed one block
    a = idx_args(rows=_lib.Rows(FAKE, 0, 1, 1 << 25, 0, 0, 0), E_cap=1 << 23, k=4096)
    assert L.csa_index_topk_workspace_size(C.byref(a)) == 0
    assert L.csa_index_topk(C.byref(a), FAKE, 1 << 40, None) == 4


def att_args(**kw):
    rows = kw.pop("rows", _lib.Rows(FAKE, 0, 4, 131071, 0, 0, 0))
    d = dict(rows=rows, q=FAKE, entries=FAKE, entry_scale=None, idx=FAKE, win=FAKE, out=FAKE, lse=None,
             E_cap=32768, R_w=128, B=4, H=64, D=512, q_dtype=1, entry_dtype=1, win_dtype=1, out_dtype=0, m=4,
             W=128, k=1024, softmax_scale=0.088, reserved=0)
    d.update(kw)
    return _lib.AttendArgs(**d)


@pytest.mark.parametrize("fn", ["csa_attend", "hca_attend"])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(win=None), 1), (dict(entry_dtype=2), 1), (dict(R_w=127), 2), (dict(W=0), 2),
    (dict(H=40), 4), (dict(D=96), 4), (dict(H=256), 4), (dict(q_dtype=0), 3), (dict(win_dtype=2), 3),
    (dict(out_dtype=2), 3), (dict(softmax_scale=float("nan")), 2), (dict(out=FAKE_ODD), 5),
    (dict(q_dtype=0, entry_dtype=0, win_dtype=0, H=64, D=128), 4),
])
def test_attend_validation(L, fn, kw, status):
    a = att_args(**kw)
    assert getattr(L, fn)(C.byref(a), FAKE, 1 << 30, None) == status, err(L)


def test_attend_csa_needs_idx_and_workspace(L):
    a = att_args(idx=None)
    assert L.csa_attend(C.byref(a), FAKE, 1 << 30, None) == 1
    a = att_args()
    n = L.csa_attend_workspace_size(C.byref(a))
    assert n > 0                                                          # split partials for 4 rows
    assert L.csa_attend(C.byref(a), FAKE, n - 1, None) == 6
    assert L.hca_attend_workspace_size(C.byref(att_args(rows=_lib.Rows(None, 1, 32768, 0, 0, 0, 0), B=1))) == 0


def qargs(**kw):
    d = dict(x=FAKE, W_q=FAKE, W_UK=FAKE, W_iq=FAKE, W_w=FAKE, q=FAKE, qI=FAKE, w=FAKE, R=32, d_model=4096, H=64,
             d_h=128, D=512, H_I=64, D_I=128, q_dtype=1)
    d.update(kw)
    return _lib.QueryArgs(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(q=None), 1), (dict(qI=None), 1), (dict(w=None), 1), (dict(R=0), 2),
    (dict(R=(1 << 21) + 1), 2),
    (dict(d_model=4000), 4), (dict(d_model=0), 4), (dict(q_dtype=2), 3), (dict(D=576), 4), (dict(D=8192), 4),
    (dict(d_h=120), 4),
    (dict(d_h=512), 4), (dict(W_UK=None), 2), (dict(W_q=FAKE_ODD), 5), (dict(w=FAKE_ODD), 5), (dict(H=0), 2),
])
def test_queries_validation(L, kw, status):
    a = qargs(**kw)
    assert L.layer_queries(C.byref(a), FAKE, 1 << 30, None) == status, err(L)


def test_queries_workspace(L):
    a = qargs()
    n = L.layer_queries_workspace_size(C.byref(a))
    # fp32 head queries before absorption, then the partial sums of W_w, whose
    # single column tile is cut in 16 parts of K beside the 256 tiles of W_q and W_iq
    assert n == 32 * 64 * 128 * 4 + 16 * 32 * 64 * 4
    assert L.layer_queries(C.byref(a), FAKE, n - 1, None) == 6
    assert L.layer_queries(C.byref(a), None, 0, None) == 6
    assert L.layer_queries_workspace_size(C.byref(qargs(W_UK=None, D=128))) == 16 * 32 * 64 * 4
    assert L.layer_queries_workspace_size(C.byref(qargs(W_UK=None, D=128, W_w=None))) == 0
    assert L.layer_queries_workspace_size(C.byref(qargs(R=0))) == 0


def sargs(**kw):
    d = dict(x=FAKE, W_c=FAKE, W_g=FAKE, W_cI=FAKE, W_gI=FAKE, v=FAKE, g=FAKE, vI=FAKE, gI=FAKE, R=32, d_model=4096,
             D=512, D_I=128, out_dtype=1, reserved=0)
    d.update(kw)
    return _lib.StreamArgs(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(v=None), 1), (dict(gI=None), 1), (dict(R=(1 << 21) + 1), 2), (dict(D=0), 2),
    (dict(D_I=0), 2), (dict(d_model=100), 4), (dict(out_dtype=2), 3), (dict(vI=FAKE_ODD), 5),
])
def test_streams_validation(L, kw, status):
    assert L.layer_streams(C.byref(sargs(**kw)), FAKE, 1 << 30, None) == status, err(L)


def test_streams_workspace(L):
    a = sargs()
    n = L.layer_streams_workspace_size(C.byref(a))
    # 1280 columns make 20 tiles of 64: K is cut in 16 parts, fp32 partial sums per part
    assert n == 16 * 32 * 1280 * 4
    assert L.layer_streams(C.byref(a), FAKE, n - 1, None) == 6
    assert L.layer_streams_workspace_size(C.byref(sargs(R=0))) == 0


def oargs(**kw):
    d = dict(o=FAKE, W_UV=FAKE, W_o=FAKE, y=FAKE, R=32, d_model=4096, H=64, d_h=128, D=512, y_dtype=1)
    d.update(kw)
    return _lib.OutputArgs(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(W_o=None), 1), (dict(y=None), 1), (dict(R=0), 2), (dict(d_model=0), 2),
    (dict(H=1, d_h=64), 4), (dict(D=192), 4), (dict(W_UV=None), 2), (dict(y_dtype=2), 3), (dict(y=FAKE_ODD), 5),
])
def test_output_validation(L, kw, status):
    assert L.layer_output(C.byref(oargs(**kw)), FAKE, 1 << 30, None) == status, err(L)


def test_output_workspace(L):
    a = oargs()
    n = L.layer_output_workspace_size(C.byref(a))
    heads = 32 * 64 * 128 * 2                                       # bf16 heads o_h = W_UV^h o~_h
    part = 4 * 32 * 4096 * 4                                        # W_o: 64 column tiles, K cut in 4 parts
    assert n == heads + part
    assert L.layer_output(C.byref(a), FAKE, n - 1, None) == 6
    assert L.layer_output_workspace_size(C.byref(oargs(W_UV=None, D=128))) == part


def test_inputs_validation_and_workspace(L):
    q, st = qargs(), sargs()
    n = L.layer_inputs_workspace_size(C.byref(q), C.byref(st))
    # fp32 head queries, then the partial sums of the products cut in 16 parts of K
    # beside the 256 column tiles of W_q and W_iq: W_w (64 columns) and the four streams
    assert n == 32 * 64 * 128 * 4 + 16 * 32 * (64 + 512 + 512 + 128 + 128) * 4
    assert L.layer_inputs(C.byref(q), C.byref(st), FAKE, n - 1, None) == 6
    assert L.layer_inputs(C.byref(q), C.byref(sargs(x=FAKE + 16)), FAKE, 1 << 30, None) == 2
    assert L.layer_inputs(C.byref(q), C.byref(sargs(R=31)), FAKE, 1 << 30, None) == 2
    assert L.layer_inputs(C.byref(qargs(q=None)), C.byref(st), FAKE, 1 << 30, None) == 1
    assert L.layer_inputs(C.byref(q), C.byref(sargs(out_dtype=2)), FAKE, 1 << 30, None) == 3


def test_mxfp4_key_tiles_layout():
    """mxfp4_pack / mxfp4_unpack follow the byte layout the header states: code byte
    (j/32) * 17 D + ((d/32) * 32 + j%32) * 16 + (d%32)/2 (even channel in the low
    nibble), scale byte (j/32) * 17 D + 16 D + (j%32) * (D/32) + d/32."""
    import torch
    rng = np.random.default_rng(5)
    for B, E, D in [(2, 70, 64), (1, 32, 128), (1, 5, 32)]:
        codes = rng.integers(0, 16, size=(B, E, D), dtype=np.uint8)
        scale = rng.integers(0, 255, size=(B, E, D // 32), dtype=np.uint8)
        keys = _lib.mxfp4_pack(torch.from_numpy(codes), torch.from_numpy(scale))
        t = keys.tiles.numpy()
        assert t.shape == (B, (E + 31) // 32, 17 * D) and keys.E_cap == (E + 31) // 32 * 32
        for b in range(B):
            for j in range(E):
                base = t[b, j // 32]
                for d in range(D):
                    byte = base[((d // 32) * 32 + j % 32) * 16 + (d % 32) // 2]
                    assert ((byte >> 4) if d % 2 else (byte & 15)) == codes[b, j, d]
                for blk in range(D // 32):
                    assert base[16 * D + (j % 32) * (D // 32) + blk] == scale[b, j, blk]
        c2, s2 = _lib.mxfp4_unpack(keys)
        assert np.array_equal(c2.numpy()[:, :E], codes) and np.array_equal(s2.numpy()[:, :E], scale)


# ---------------------------------------------------------------- the binding's own checks
# The C ABI sees bare pointers, so the Python binding refuses strided views, tensors on
# another device and shapes that disagree with the row count, head count or k before
# anything reaches the library (CPU tensors: the checks raise before any C call).
def _attend_inputs(R=2, H=16, D=64, B=2, E=32, Rw=128, k=8):
    q = torch.zeros(R, H, D, dtype=torch.bfloat16)
    ent = torch.zeros(B, E, D, dtype=torch.bfloat16)
    idx = torch.zeros(R, k, dtype=torch.int32)
    win = torch.zeros(B, Rw, D, dtype=torch.bfloat16)
    out = torch.zeros(R, H, D)
    pos = torch.full((R,), 200, dtype=torch.int32)
    return sk.RowSpec.decode(pos, 200), q, ent, idx, win, out


@pytest.mark.parametrize("bad", ["q_strided", "out_rows", "idx_dtype", "idx_rows", "win_dim", "lse_shape",
                                 "pos_rows", "ent_D"])
def test_binding_rejects_attend_tensors(bad):
    rows, q, ent, idx, win, out = _attend_inputs()
    lse = None
    if bad == "q_strided":
        q = torch.zeros(2, 16, 128, dtype=torch.bfloat16)[:, :, ::2]
    elif bad == "out_rows":
        out = torch.zeros(3, 16, 64)
    elif bad == "idx_dtype":
        idx = idx.to(torch.int64)
    elif bad == "idx_rows":
        idx = torch.zeros(1, 8, dtype=torch.int32)
    elif bad == "win_dim":
        win = torch.zeros(2, 128, 32, dtype=torch.bfloat16)
    elif bad == "lse_shape":
        lse = torch.zeros(2, 8)
    elif bad == "pos_rows":
        rows = sk.RowSpec(sk.ROWS_DECODE, 2, torch.zeros(3, dtype=torch.int32), 200)
    elif bad == "ent_D":
        ent = torch.zeros(2, 32, 128, dtype=torch.bfloat16)
    with pytest.raises(sk.SckvError):
        _lib.attend_args(rows, q, ent, win, out, m=4, W=128, softmax_scale=0.125, idx=idx, lse=lse)


@pytest.mark.parametrize("bad", ["w_shape", "q_strided", "out_k", "keys_tiles", "scores_rows"])
def test_binding_rejects_index_tensors(bad):
    R, HI, DI, B, E, k = 2, 32, 64, 2, 64, 16
    rows = sk.RowSpec.decode(torch.full((R,), 300, dtype=torch.int32), 300)
    q = torch.zeros(R, HI, DI, dtype=torch.bfloat16)
    w = torch.zeros(R, HI)
    keys = sk.key_tiles_empty(B, E, DI, torch.bfloat16, "cpu")
    out = torch.zeros(R, k, dtype=torch.int32)
    if bad == "w_shape":
        w = torch.zeros(R, HI + 1)
    elif bad == "q_strided":
        q = torch.zeros(R, DI, HI, dtype=torch.bfloat16).transpose(1, 2)
    elif bad == "out_k":
        out = torch.zeros(R, k + 1, dtype=torch.int32)
    elif bad == "keys_tiles":
        keys = torch.zeros(B, E // 32, DI // 8, 16, 16, dtype=torch.bfloat16)
    with pytest.raises(sk.SckvError):
        if bad == "scores_rows":
            sk.csa_index_score(rows, q, w, keys, torch.zeros(R + 1, 64), m=4, W=128, k=k)
        else:
            _lib.index_args(rows, q, w, keys, out, m=4, W=128, k=k)


@pytest.mark.parametrize("bad", ["gate_shape", "out_batch", "scale_shape", "ring_shape"])
def test_binding_rejects_pool_tensors(bad):
    B, N, D, E = 2, 64, 64, 16
    v = torch.zeros(B, N, D, dtype=torch.bfloat16)
    g = torch.zeros(B, N, D, dtype=torch.bfloat16)
    bp = torch.zeros(8, D)
    out = torch.zeros(B, E, D, dtype=torch.bfloat16)
    with pytest.raises(sk.SckvError):
        if bad == "gate_shape":
            sk.Pool(v, g[:, :32].contiguous(), bp, out).c()
        elif bad == "out_batch":
            sk.Pool(v, g, bp, torch.zeros(B + 1, E, D, dtype=torch.bfloat16)).c()
        elif bad == "scale_shape":
            sk.Pool(v, g, bp, out.to(torch.uint8), out_scale=torch.zeros(B, E + 1)).c()
        else:
            pos = torch.zeros(B, dtype=torch.int32)
            sk.Append(pos, v[:, 0].contiguous(), g[:, 0].contiguous(), torch.zeros(B, 16, D, dtype=torch.bfloat16),
                      torch.zeros(B, 8, D, dtype=torch.bfloat16), bp, out).c()


def test_binding_accepts_consistent_tensors():
    rows, q, ent, idx, win, out = _attend_inputs()
    a = _lib.attend_args(rows, q, ent, win, out, m=4, W=128, softmax_scale=0.125, idx=idx, lse=torch.zeros(2, 16))
    assert a.H == 16 and a.D == 64 and a.k == 8 and a.R_w == 128


def test_noalloc_index_rejects_rows_beyond_its_scratch(L):
    """csa_index_topk_noalloc refuses, before any HIP call, rows whose scores and
    selection need more than the static scratch holds."""
    # 4096 causal rows over 8192 visible entries: 4096 x 8192 fp32 scores = 128 MiB
    a = idx_args(rows=_lib.Rows(None, 1, 4096, 0, 0, 32900, 0), E_cap=8192, k=512)
    need = L.csa_index_topk_workspace_size(C.byref(a))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert L.csa_index_topk_noalloc(C.byref(a), None) == 6, err(L)
    assert "scratch" in err(L)
    # invalid arguments keep their own status
    bad = idx_args(k=0)
    assert L.csa_index_topk_noalloc(C.byref(bad), None) == 2


@pytest.mark.skipif(bool(os.environ.get("SCKV_LIB_PATH")), reason="this run already loads another build")
def test_host_checks_under_address_and_undefined_behaviour_sanitizers():
    """Every check above again, in a child process, against a host-only build of the
    library with AddressSanitizer and UndefinedBehaviorSanitizer (the runtime
    preloaded): the argument checks, plan arithmetic and error paths must neither
    touch memory they do not own nor hit undefined behaviour."""
    import subprocess
    import sys

    import sanitized_build
    lib = sanitized_build.build()
    env = dict(os.environ, LD_PRELOAD=sanitized_build.runtime(), SCKV_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.abspath(__file__), "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout

"""ctypes binding of libsckv.so: the same five calls (plus the two indexer halves),
taking torch device tensors and the current HIP stream.  Argument marshalling
only: every step runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

# SCKV_LIB_PATH names another build of the same library (the sanitized host build
# the host checks run against); by default the library next to this file
_LIB_PATH = os.environ.get("SCKV_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsckv.so")

F32, BF16, E4M3, MXFP4 = 0, 1, 2, 3
ROWS_DECODE, ROWS_CAUSAL = 0, 1
LAYOUT_ROWS, LAYOUT_KEY_TILES = 0, 1

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_UNSUPPORTED", 5: "ERR_ALIGN",
          6: "ERR_WORKSPACE", 7: "ERR_HIP"}


class SckvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


# ---------------------------------------------------------------- C structs (mirror include/sckv.h)
class Rows(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("kind", C.c_int32), ("R", C.c_int32), ("pos_max", C.c_int32),
                ("seq0", C.c_int32), ("pos0", C.c_int32), ("reserved", C.c_int32)]


class PoolStream(C.Structure):
    _fields_ = [("val", C.c_void_p), ("gate", C.c_void_p), ("bpos", C.c_void_p), ("out", C.c_void_p),
                ("out_scale", C.c_void_p), ("E_cap", C.c_int64), ("D", C.c_int32), ("in_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("out_layout", C.c_int32)]


class AppendStream(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("val", C.c_void_p), ("gate", C.c_void_p), ("val_ring", C.c_void_p),
                ("gate_ring", C.c_void_p), ("bpos", C.c_void_p), ("out", C.c_void_p), ("out_scale", C.c_void_p),
                ("E_cap", C.c_int64), ("D", C.c_int32), ("P", C.c_int32), ("in_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("out_layout", C.c_int32), ("reserved", C.c_int32)]


class IndexArgs(C.Structure):
    _fields_ = [("rows", Rows), ("q", C.c_void_p), ("w", C.c_void_p), ("keys", C.c_void_p),
                ("out_idx", C.c_void_p), ("out_score", C.c_void_p), ("E_cap", C.c_int64), ("B", C.c_int32),
                ("H_I", C.c_int32), ("D_I", C.c_int32), ("q_dtype", C.c_int32), ("key_dtype", C.c_int32),
                ("m", C.c_int32), ("W", C.c_int32), ("k", C.c_int32)]


class AttendArgs(C.Structure):
    _fields_ = [("rows", Rows), ("q", C.c_void_p), ("entries", C.c_void_p), ("entry_scale", C.c_void_p),
                ("idx", C.c_void_p), ("win", C.c_void_p), ("out", C.c_void_p), ("lse", C.c_void_p),
                ("E_cap", C.c_int64), ("R_w", C.c_int64), ("B", C.c_int32), ("H", C.c_int32), ("D", C.c_int32),
                ("q_dtype", C.c_int32), ("entry_dtype", C.c_int32), ("win_dtype", C.c_int32),
                ("out_dtype", C.c_int32), ("m", C.c_int32), ("W", C.c_int32), ("k", C.c_int32),
                ("softmax_scale", C.c_float), ("reserved", C.c_int32)]


class QueryArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("W_q", C.c_void_p), ("W_UK", C.c_void_p), ("W_iq", C.c_void_p),
                ("W_w", C.c_void_p), ("q", C.c_void_p), ("qI", C.c_void_p), ("w", C.c_void_p), ("R", C.c_int32),
                ("d_model", C.c_int32), ("H", C.c_int32), ("d_h", C.c_int32), ("D", C.c_int32), ("H_I", C.c_int32),
                ("D_I", C.c_int32), ("q_dtype", C.c_int32)]


class StreamArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("W_c", C.c_void_p), ("W_g", C.c_void_p), ("W_cI", C.c_void_p),
                ("W_gI", C.c_void_p), ("v", C.c_void_p), ("g", C.c_void_p), ("vI", C.c_void_p), ("gI", C.c_void_p),
                ("R", C.c_int32), ("d_model", C.c_int32), ("D", C.c_int32), ("D_I", C.c_int32),
                ("out_dtype", C.c_int32), ("reserved", C.c_int32)]


class OutputArgs(C.Structure):
    _fields_ = [("o", C.c_void_p), ("W_UV", C.c_void_p), ("W_o", C.c_void_p), ("y", C.c_void_p), ("R", C.c_int32),
                ("d_model", C.c_int32), ("H", C.c_int32), ("d_h", C.c_int32), ("D", C.c_int32),
                ("y_dtype", C.c_int32)]


EXPORTS = ["csa_compress", "hca_compress", "csa_append", "hca_append", "csa_index_topk_workspace_size", "csa_index_topk",
           "csa_index_topk_noalloc", "csa_index_score",
           "csa_topk_select_workspace_size", "csa_topk_select", "csa_attend_workspace_size",
           "hca_attend_workspace_size", "csa_attend", "hca_attend", "layer_queries_workspace_size", "layer_queries",
           "layer_streams_workspace_size", "layer_streams", "layer_inputs_workspace_size", "layer_inputs",
           "layer_output_workspace_size", "layer_output",
           "sckv_last_error", "sckv_abi_version"]

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> C.CDLL:
    """Loads libsckv.so (raises if it was not built: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(python -m sequence_compressed_kv_amd.build)")
    L = C.CDLL(_LIB_PATH)
    P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    L.csa_compress.argtypes = [i32, i64, i32, i32, i64, i64, C.POINTER(PoolStream), C.POINTER(PoolStream), P]
    L.hca_compress.argtypes = [i32, i64, i32, i32, i64, i64, C.POINTER(PoolStream), P]
    L.csa_append.argtypes = [i32, i32, i32, C.POINTER(AppendStream), C.POINTER(AppendStream), P]
    L.hca_append.argtypes = [i32, i32, i32, C.POINTER(AppendStream), P]
    L.csa_index_topk_workspace_size.argtypes = [C.POINTER(IndexArgs)]
    L.csa_index_topk_workspace_size.restype = sz
    L.csa_index_topk.argtypes = [C.POINTER(IndexArgs), P, sz, P]
    L.csa_index_topk_noalloc.argtypes = [C.POINTER(IndexArgs), P]
    L.csa_index_score.argtypes = [C.POINTER(IndexArgs), P, i64, P]
    L.csa_topk_select_workspace_size.argtypes = [C.POINTER(IndexArgs)]
    L.csa_topk_select_workspace_size.restype = sz
    L.csa_topk_select.argtypes = [C.POINTER(IndexArgs), P, i64, P, sz, P]
    for n in ("csa_attend_workspace_size", "hca_attend_workspace_size"):
        getattr(L, n).argtypes = [C.POINTER(AttendArgs)]
        getattr(L, n).restype = sz
    for n in ("csa_attend", "hca_attend"):
        getattr(L, n).argtypes = [C.POINTER(AttendArgs), P, sz, P]
    L.layer_queries_workspace_size.argtypes = [C.POINTER(QueryArgs)]
    L.layer_queries_workspace_size.restype = sz
    L.layer_queries.argtypes = [C.POINTER(QueryArgs), P, sz, P]
    L.layer_streams_workspace_size.argtypes = [C.POINTER(StreamArgs)]
    L.layer_streams_workspace_size.restype = sz
    L.layer_streams.argtypes = [C.POINTER(StreamArgs), P, sz, P]
    L.layer_inputs_workspace_size.argtypes = [C.POINTER(QueryArgs), C.POINTER(StreamArgs)]
    L.layer_inputs_workspace_size.restype = sz
    L.layer_inputs.argtypes = [C.POINTER(QueryArgs), C.POINTER(StreamArgs), P, sz, P]
    L.layer_output_workspace_size.argtypes = [C.POINTER(OutputArgs)]
    L.layer_output_workspace_size.restype = sz
    L.layer_output.argtypes = [C.POINTER(OutputArgs), P, sz, P]
    for n in ("csa_compress", "hca_compress", "csa_append", "hca_append", "csa_index_topk", "csa_index_topk_noalloc",
              "csa_index_score",
              "csa_topk_select", "csa_attend", "hca_attend", "layer_queries", "layer_streams", "layer_inputs", "layer_output"):
        getattr(L, n).restype = C.c_int
    L.sckv_last_error.restype = C.c_char_p
    L.sckv_abi_version.restype = C.c_int32
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise SckvError(status, load().sckv_last_error().decode())


# ---------------------------------------------------------------- helpers
def dtype_code(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return -1
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _fail(msg: str):
    raise SckvError(2, msg)


def _dense(device, **named):
    """Every named tensor (None skipped) must be contiguous and on `device`: the
    C ABI sees bare pointers, so a strided view or a tensor on another device
    would be read or written out of bounds."""
    for name, t in named.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            _fail(f"{name}: expected a tensor, got {type(t).__name__}")
        if not t.is_contiguous():
            _fail(f"{name}: tensor must be contiguous (shape {tuple(t.shape)}, strides {t.stride()})")
        if device is not None and t.device != device:
            _fail(f"{name}: on {t.device}, expected {device}")


def _shape(name: str, t: Optional[torch.Tensor], want):
    """t.shape must equal want (None entries match any size)."""
    if t is None:
        return
    got = t.shape
    ok = len(got) == len(want)
    if ok:
        for g, w in zip(got, want):
            if w is not None and g != w:
                ok = False
                break
    if not ok:
        _fail(f"{name}: shape {tuple(got)}, expected {tuple('*' if w is None else w for w in want)}")


def _int32(name: str, t: Optional[torch.Tensor]):
    if t is not None and t.dtype != torch.int32:
        _fail(f"{name}: dtype {t.dtype}, expected torch.int32")


def _rows_check(rows: "RowSpec", device):
    if rows.kind == ROWS_DECODE and rows.pos is not None:
        _dense(device, pos=rows.pos)
        _int32("pos", rows.pos)
        _shape("pos", rows.pos, (rows.R,))


_HAVE_GPU: Optional[bool] = None


def _stream(stream) -> Optional[int]:
    global _HAVE_GPU
    if stream is None:
        if _HAVE_GPU is None:
            _HAVE_GPU = torch.cuda.is_available()
        return torch.cuda.current_stream().cuda_stream if _HAVE_GPU else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


@dataclass
class RowSpec:
    """Query rows: decode (pos: int32 device tensor [R], one row per sequence) or causal
    (positions pos0 .. pos0 + R - 1 of sequence seq0)."""
    kind: int
    R: int
    pos: Optional[torch.Tensor] = None
    pos_max: int = 0
    seq0: int = 0
    pos0: int = 0

    @staticmethod
    def decode(pos: torch.Tensor, pos_max: int) -> "RowSpec":
        return RowSpec(ROWS_DECODE, int(pos.shape[0]), pos, int(pos_max))

    @staticmethod
    def causal(R: int, pos0: int = 0, seq0: int = 0) -> "RowSpec":
        return RowSpec(ROWS_CAUSAL, int(R), None, 0, int(seq0), int(pos0))

    def c(self) -> Rows:
        return Rows(_ptr(self.pos), self.kind, self.R, self.pos_max, self.seq0, self.pos0, 0)


@dataclass
class Mxfp4Keys:
    """An MXFP4 indexer key cache: tiles uint8 [B][E_cap/32][17 * D_I], per tile of 32
    keys the codes [D_I/32][32][16 bytes] (two e2m1 codes per byte, the even channel
    in the low nibble) then the E8M0 scale bytes [32][D_I/32]."""
    tiles: torch.Tensor
    D_I: int

    @staticmethod
    def empty(B: int, E_cap: int, D_I: int, device) -> "Mxfp4Keys":
        if E_cap % 32 or D_I % 32:
            raise ValueError("MXFP4 key tiles need E_cap % 32 == 0 and D_I % 32 == 0")
        return Mxfp4Keys(torch.empty(B, E_cap // 32, 17 * D_I, dtype=torch.uint8, device=device), D_I)

    @property
    def device(self):
        return self.tiles.device

    def clone(self) -> "Mxfp4Keys":
        return Mxfp4Keys(self.tiles.clone(), self.D_I)

    @property
    def E_cap(self) -> int:
        return int(self.tiles.shape[1]) * 32


def mxfp4_pack(codes: torch.Tensor, scale: torch.Tensor) -> Mxfp4Keys:
    """Row-major e2m1 codes [B][E][D] (uint8 0..15) and scale bytes [B][E][D/32] ->
    MXFP4 key tiles (E padded with zero keys to a multiple of 32).  Byte layout only."""
    B, E, D = codes.shape
    Ep = (E + 31) // 32 * 32
    if Ep != E:
        codes = torch.cat([codes, codes.new_zeros(B, Ep - E, D)], dim=1)
        scale = torch.cat([scale, scale.new_zeros(B, Ep - E, D // 32)], dim=1)
    T = Ep // 32
    c = codes.to(torch.uint8).reshape(B, T, 32, D // 32, 16, 2)
    byte = (c[..., 0] | (c[..., 1] << 4)).permute(0, 1, 3, 2, 4).reshape(B, T, 16 * D)
    sc = scale.to(torch.uint8).reshape(B, T, D)
    return Mxfp4Keys(torch.cat([byte, sc], dim=2).contiguous(), D)


def mxfp4_unpack(keys: Mxfp4Keys):
    """MXFP4 key tiles -> (codes [B][E_cap][D] uint8 0..15, scale bytes [B][E_cap][D/32])."""
    t, D = keys.tiles, keys.D_I
    B, T, _ = t.shape
    byte = t[:, :, :16 * D].reshape(B, T, D // 32, 32, 16).permute(0, 1, 3, 2, 4)    # [B][T][n][blk][16]
    codes = torch.stack([byte & 15, byte >> 4], dim=-1).reshape(B, T * 32, D)
    scale = t[:, :, 16 * D:].reshape(B, T * 32, D // 32)
    return codes, scale


def _out_code(out) -> int:
    return MXFP4 if isinstance(out, Mxfp4Keys) else dtype_code(out)


def _out_tensor(out) -> torch.Tensor:
    return out.tiles if isinstance(out, Mxfp4Keys) else out


@dataclass
class Pool:
    """One stream pair to pool: val, gate [B][N][D]; bpos [m+o][D] fp32;
    out [B][E_cap][D] (rows) or a key-tile cache made by key_tiles_empty();
    out_scale [B][E_cap] fp32 (scaled e4m3 output) or None."""
    val: torch.Tensor
    gate: torch.Tensor
    bpos: torch.Tensor
    out: torch.Tensor
    out_scale: Optional[torch.Tensor] = None
    layout: int = LAYOUT_ROWS

    def c(self) -> PoolStream:
        out = _out_tensor(self.out)
        _dense(self.val.device, val=self.val, gate=self.gate, bpos=self.bpos, out=out, out_scale=self.out_scale)
        if self.val.dim() != 3:
            _fail(f"val: shape {tuple(self.val.shape)}, expected [B][N][D]")
        B, N, D = (int(x) for x in self.val.shape)
        _shape("gate", self.gate, (B, N, D))
        _shape("bpos", self.bpos, (None, D))
        E_cap = int(out.shape[1]) if self.layout == LAYOUT_ROWS else int(out.shape[1]) * 32
        if int(out.shape[0]) != B:
            _fail(f"out: batch {int(out.shape[0])}, expected {B}")
        if self.layout == LAYOUT_ROWS:
            _shape("out", out, (B, E_cap, D))
        _shape("out_scale", self.out_scale, (B, E_cap))
        return PoolStream(_ptr(self.val), _ptr(self.gate), _ptr(self.bpos), _ptr(out), _ptr(self.out_scale),
                          E_cap, D, dtype_code(self.val), _out_code(self.out), self.layout)


@dataclass
class Append:
    """One stream's decode append: pos [B] int32 positions of the new tokens;
    val, gate [B][D] the new tokens; val_ring, gate_ring [B][P][D] the last P tokens
    (slot = position mod P; for the latent stream val_ring may be the window ring);
    bpos [m+o][D] fp32; out (+ out_scale) the entry cache as in Pool."""
    pos: torch.Tensor
    val: torch.Tensor
    gate: torch.Tensor
    val_ring: torch.Tensor
    gate_ring: torch.Tensor
    bpos: torch.Tensor
    out: torch.Tensor
    out_scale: Optional[torch.Tensor] = None
    layout: int = LAYOUT_ROWS

    def c(self) -> AppendStream:
        out = _out_tensor(self.out)
        _dense(self.val.device, pos=self.pos, val=self.val, gate=self.gate, val_ring=self.val_ring,
               gate_ring=self.gate_ring, bpos=self.bpos, out=out, out_scale=self.out_scale)
        if self.val.dim() != 2:
            _fail(f"val: shape {tuple(self.val.shape)}, expected [B][D]")
        B, D = (int(x) for x in self.val.shape)
        _int32("pos", self.pos)
        _shape("pos", self.pos, (B,))
        _shape("gate", self.gate, (B, D))
        _shape("val_ring", self.val_ring, (B, None, D))
        _shape("gate_ring", self.gate_ring, (B, int(self.val_ring.shape[1]), D))
        _shape("bpos", self.bpos, (None, D))
        E_cap = int(out.shape[1]) if self.layout == LAYOUT_ROWS else int(out.shape[1]) * 32
        if int(out.shape[0]) != B:
            _fail(f"out: batch {int(out.shape[0])}, expected {B}")
        if self.layout == LAYOUT_ROWS:
            _shape("out", out, (B, E_cap, D))
        _shape("out_scale", self.out_scale, (B, E_cap))
        return AppendStream(_ptr(self.pos), _ptr(self.val), _ptr(self.gate), _ptr(self.val_ring),
                            _ptr(self.gate_ring), _ptr(self.bpos), _ptr(out), _ptr(self.out_scale), E_cap, D,
                            int(self.val_ring.shape[1]), dtype_code(self.val), _out_code(self.out), self.layout, 0)


# ---------------------------------------------------------------- indexer key tiles
def key_tiles_empty(B: int, E_cap: int, D_I: int, dtype, device) -> torch.Tensor:
    """An indexer key cache in the tiled layout [B][E_cap/32][D_I/8][32][8]."""
    if E_cap % 32 or D_I % 8:
        raise ValueError("key tiles need E_cap % 32 == 0 and D_I % 8 == 0")
    return torch.empty(B, E_cap // 32, D_I // 8, 32, 8, dtype=dtype, device=device)


def to_key_tiles(keys: torch.Tensor) -> torch.Tensor:
    """[B][E][D_I] row-major keys -> tiled layout (E padded to a multiple of 32)."""
    f8 = keys.dtype == torch.float8_e4m3fn
    if f8:
        keys = keys.view(torch.uint8)
    B, E, D = keys.shape
    Ep = (E + 31) // 32 * 32
    if Ep != E:
        keys = torch.cat([keys, keys.new_zeros(B, Ep - E, D)], dim=1)
    t = keys.reshape(B, Ep // 32, 32, D // 8, 8).permute(0, 1, 3, 2, 4).contiguous()
    return t.view(torch.float8_e4m3fn) if f8 else t


def from_key_tiles(tiles: torch.Tensor) -> torch.Tensor:
    """Tiled keys -> [B][E_cap][D_I] row-major."""
    f8 = tiles.dtype == torch.float8_e4m3fn
    if f8:
        tiles = tiles.view(torch.uint8)
    B, T, DB, _, _ = tiles.shape
    r = tiles.permute(0, 1, 3, 2, 4).reshape(B, T * 32, DB * 8)
    return r.view(torch.float8_e4m3fn) if f8 else r


# ---------------------------------------------------------------- calls
def csa_compress(kv: Pool, index_keys: Optional[Pool] = None, *, m: int = 4, o: int = 4, e_begin: int = 0,
                 e_count: Optional[int] = None, stream=None):
    B, N = int(kv.val.shape[0]), int(kv.val.shape[1])
    e_count = (N // m - e_begin) if e_count is None else e_count
    a = kv.c()
    b = index_keys.c() if index_keys is not None else None
    _check(load().csa_compress(B, N, m, o, e_begin, e_count, C.byref(a), C.byref(b) if b is not None else None,
                               _stream(stream)))


def hca_compress(kv: Pool, *, m: int = 128, o: int = 0, e_begin: int = 0, e_count: Optional[int] = None,
                 stream=None):
    B, N = int(kv.val.shape[0]), int(kv.val.shape[1])
    e_count = (N // m - e_begin) if e_count is None else e_count
    a = kv.c()
    _check(load().hca_compress(B, N, m, o, e_begin, e_count, C.byref(a), _stream(stream)))


def csa_append(kv: Append, index_keys: Optional[Append] = None, *, m: int = 4, o: int = 4, stream=None):
    B = int(kv.val.shape[0])
    a = kv.c()
    b = index_keys.c() if index_keys is not None else None
    _check(load().csa_append(B, m, o, C.byref(a), C.byref(b) if b is not None else None, _stream(stream)))


def hca_append(kv: Append, *, m: int = 128, o: int = 0, stream=None):
    B = int(kv.val.shape[0])
    a = kv.c()
    _check(load().hca_append(B, m, o, C.byref(a), _stream(stream)))


def index_args(rows: RowSpec, q, w, keys, out_idx, *, m: int, W: int, k: int, out_score=None) -> IndexArgs:
    """keys: a tiled key cache [B][E_cap/32][D_I/8][32][8] (see key_tiles_empty) or Mxfp4Keys."""
    kt = keys.tiles if isinstance(keys, Mxfp4Keys) else keys
    _dense(kt.device, q=q, w=w, keys=kt, out_idx=out_idx, out_score=out_score)
    _rows_check(rows, kt.device)
    if q.dim() != 3:
        _fail(f"q: shape {tuple(q.shape)}, expected [R][H_I][D_I]")
    _shape("q", q, (rows.R, None, None))
    _shape("w", w, (rows.R, int(q.shape[1])))
    _int32("out_idx", out_idx)
    _shape("out_idx", out_idx, (rows.R, k))
    _shape("out_score", out_score, (rows.R, k))
    if isinstance(keys, Mxfp4Keys):
        _shape("keys", kt, (None, None, 17 * int(q.shape[2])))
        return IndexArgs(rows.c(), _ptr(q), _ptr(w), _ptr(keys.tiles), _ptr(out_idx), _ptr(out_score), keys.E_cap,
                         int(keys.tiles.shape[0]), int(q.shape[1]), int(q.shape[2]), dtype_code(q), MXFP4, m, W, k)
    if keys.dim() != 5:
        raise ValueError("indexer keys must be in the tiled layout [B][E_cap/32][D_I/8][32][8]")
    _shape("keys", keys, (None, None, int(q.shape[2]) // 8, 32, 8))
    return IndexArgs(rows.c(), _ptr(q), _ptr(w), _ptr(keys), _ptr(out_idx), _ptr(out_score),
                     int(keys.shape[1]) * 32, int(keys.shape[0]), int(q.shape[1]), int(q.shape[2]), dtype_code(q),
                     dtype_code(keys), m, W, k)


def _scores_check(scores, rows: RowSpec, keys):
    """A score matrix [R][stride] with unit stride along a row."""
    dev = (keys.tiles if isinstance(keys, Mxfp4Keys) else keys).device
    if scores.dim() != 2 or int(scores.shape[0]) != rows.R or scores.stride(1) != 1:
        _fail(f"scores: shape {tuple(scores.shape)} strides {scores.stride()}, expected [R][n] with unit row stride")
    if scores.device != dev or scores.dtype != torch.float32:
        _fail(f"scores: {scores.dtype} on {scores.device}, expected torch.float32 on {dev}")


def csa_index_topk_workspace_size(a: IndexArgs) -> int:
    return int(load().csa_index_topk_workspace_size(C.byref(a)))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return workspace
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise SckvError(6, f"workspace of {nbytes} bytes needed")
    return workspace


def csa_index_topk(rows: RowSpec, q, w, keys, out_idx, *, m: int = 4, W: int = 128, k: int, out_score=None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    a = index_args(rows, q, w, keys, out_idx, m=m, W=W, k=k, out_score=out_score)
    n = csa_index_topk_workspace_size(a)
    if n == 0:
        _check(load().csa_index_topk(C.byref(a), None, 0, _stream(stream)))
        return None
    ws = _workspace(n, keys.device, workspace)
    _check(load().csa_index_topk(C.byref(a), _ptr(ws), n, _stream(stream)))
    return ws


NOALLOC_SCRATCH_BYTES = 16 << 20


def csa_index_topk_noalloc(rows: RowSpec, q, w, keys, out_idx, *, m: int = 4, W: int = 128, k: int, out_score=None,
                           stream=None):
    """csa_index_topk with the library's static device scratch instead of a workspace
    (for callers that cannot allocate); calls that overlap on one device race."""
    a = index_args(rows, q, w, keys, out_idx, m=m, W=W, k=k, out_score=out_score)
    _check(load().csa_index_topk_noalloc(C.byref(a), _stream(stream)))


def csa_index_score(rows: RowSpec, q, w, keys, scores, *, m: int = 4, W: int = 128, k: int = 1, stream=None):
    a = index_args(rows, q, w, keys, None, m=m, W=W, k=k)
    _scores_check(scores, rows, keys)
    _check(load().csa_index_score(C.byref(a), _ptr(scores), int(scores.stride(0)), _stream(stream)))


def csa_topk_select(rows: RowSpec, scores, out_idx, *, keys_meta, m: int = 4, W: int = 128, k: int,
                    out_score=None, workspace=None, stream=None):
    """keys_meta: (q, w, keys) tensors describing the indexer (only shapes/dtypes are read)."""
    q, w, keys = keys_meta
    a = index_args(rows, q, w, keys, out_idx, m=m, W=W, k=k, out_score=out_score)
    _scores_check(scores, rows, keys)
    n = int(load().csa_topk_select_workspace_size(C.byref(a)))
    ws = _workspace(n, scores.device, workspace)
    _check(load().csa_topk_select(C.byref(a), _ptr(scores), int(scores.stride(0)), _ptr(ws), n, _stream(stream)))


def attend_args(rows: RowSpec, q, entries, win, out, *, m: int, W: int, softmax_scale: float, entry_scale=None,
                idx=None, lse=None) -> AttendArgs:
    _dense(entries.device, q=q, entries=entries, win=win, out=out, entry_scale=entry_scale, idx=idx, lse=lse)
    _rows_check(rows, entries.device)
    if q.dim() != 3 or entries.dim() != 3 or win.dim() != 3:
        _fail("q [R][H][D], entries [B][E_cap][D] and win [B][R_w][D] must be 3-dimensional")
    H, D = int(q.shape[1]), int(q.shape[2])
    B, E_cap = int(entries.shape[0]), int(entries.shape[1])
    _shape("q", q, (rows.R, H, D))
    _shape("entries", entries, (B, E_cap, D))
    _shape("win", win, (B, None, D))
    _shape("out", out, (rows.R, H, D))
    _shape("lse", lse, (rows.R, H))
    _shape("entry_scale", entry_scale, (B, E_cap))
    _int32("idx", idx)
    if idx is not None:
        _shape("idx", idx, (rows.R, None))
    k = int(idx.shape[1]) if idx is not None else 0
    return AttendArgs(rows.c(), _ptr(q), _ptr(entries), _ptr(entry_scale), _ptr(idx), _ptr(win), _ptr(out),
                      _ptr(lse), int(entries.shape[1]), int(win.shape[1]), int(entries.shape[0]), int(q.shape[1]),
                      int(q.shape[2]), dtype_code(q), dtype_code(entries), dtype_code(win), dtype_code(out), m, W, k,
                      float(softmax_scale), 0)


def _attend(fn: str, a: AttendArgs, device, workspace, stream):
    L = load()
    n = int(getattr(L, fn + "_workspace_size")(C.byref(a)))
    ws = _workspace(n, device, workspace)
    _check(getattr(L, fn)(C.byref(a), _ptr(ws), n, _stream(stream)))
    return ws


def csa_attend(rows: RowSpec, q, entries, idx, win, out, *, m: int = 4, W: int = 128, softmax_scale: float,
               entry_scale=None, lse=None, workspace=None, stream=None):
    a = attend_args(rows, q, entries, win, out, m=m, W=W, softmax_scale=softmax_scale, entry_scale=entry_scale,
                    idx=idx, lse=lse)
    return _attend("csa_attend", a, entries.device, workspace, stream)


def hca_attend(rows: RowSpec, q, entries, win, out, *, m: int = 128, W: int = 128, softmax_scale: float,
               entry_scale=None, lse=None, workspace=None, stream=None):
    a = attend_args(rows, q, entries, win, out, m=m, W=W, softmax_scale=softmax_scale, entry_scale=entry_scale,
                    lse=lse)
    return _attend("hca_attend", a, entries.device, workspace, stream)


# ---------------------------------------------------------------- projections
def query_args(x, W_q, q, *, W_UK=None, W_iq=None, qI=None, W_w=None, w=None) -> QueryArgs:
    """x [R][d_model], W_q [H*d_h][d_model], q [R][H][D]; W_UK [H][d_h][D] (absorption) or None;
    W_iq [H_I*D_I][d_model] -> qI [R][H_I][D_I]; W_w [H_I][d_model] -> w [R][H_I] (fp32)."""
    R, dm = int(x.shape[0]), int(x.shape[1])
    H, D = int(q.shape[1]), int(q.shape[2])
    d_h = int(W_q.shape[0]) // H
    H_I = int(qI.shape[1]) if qI is not None else (int(W_w.shape[0]) if W_w is not None else 0)
    D_I = int(qI.shape[2]) if qI is not None else (1 if W_w is not None else 0)
    return QueryArgs(_ptr(x), _ptr(W_q), _ptr(W_UK), _ptr(W_iq), _ptr(W_w), _ptr(q), _ptr(qI), _ptr(w), R, dm, H,
                     d_h, D, H_I, D_I, dtype_code(q))


def layer_queries(x, W_q, q, *, W_UK=None, W_iq=None, qI=None, W_w=None, w=None, workspace=None, stream=None):
    a = query_args(x, W_q, q, W_UK=W_UK, W_iq=W_iq, qI=qI, W_w=W_w, w=w)
    L = load()
    n = int(L.layer_queries_workspace_size(C.byref(a)))
    ws = _workspace(n, x.device, workspace)
    _check(L.layer_queries(C.byref(a), _ptr(ws), n, _stream(stream)))
    return ws


def stream_args(x, *, W_c=None, v=None, W_g=None, g=None, W_cI=None, vI=None, W_gI=None, gI=None) -> StreamArgs:
    R, dm = int(x.shape[0]), int(x.shape[1])
    D = int((W_c if W_c is not None else W_g).shape[0]) if (W_c is not None or W_g is not None) else 0
    D_I = int((W_cI if W_cI is not None else W_gI).shape[0]) if (W_cI is not None or W_gI is not None) else 0
    outs = [t for t in (v, g, vI, gI) if t is not None]
    return StreamArgs(_ptr(x), _ptr(W_c), _ptr(W_g), _ptr(W_cI), _ptr(W_gI), _ptr(v), _ptr(g), _ptr(vI), _ptr(gI), R,
                      dm, D, D_I, dtype_code(outs[0]) if outs else F32, 0)


def layer_inputs(x, W_q, q, *, W_UK=None, W_iq=None, qI=None, W_w=None, w=None, W_c=None, v=None, W_g=None, g=None,
                 W_cI=None, vI=None, W_gI=None, gI=None, workspace=None, stream=None):
    """layer_queries and layer_streams of the same rows x in one launch."""
    a = query_args(x, W_q, q, W_UK=W_UK, W_iq=W_iq, qI=qI, W_w=W_w, w=w)
    b = stream_args(x, W_c=W_c, v=v, W_g=W_g, g=g, W_cI=W_cI, vI=vI, W_gI=W_gI, gI=gI)
    L = load()
    n = int(L.layer_inputs_workspace_size(C.byref(a), C.byref(b)))
    ws = _workspace(n, x.device, workspace)
    _check(L.layer_inputs(C.byref(a), C.byref(b), _ptr(ws), n, _stream(stream)))
    return ws


def layer_streams(x, *, W_c=None, v=None, W_g=None, g=None, W_cI=None, vI=None, W_gI=None, gI=None, workspace=None,
                  stream=None):
    """x [R][d_model]; each given weight [n][d_model] writes its output [R][n] (v, g: n = D; vI, gI: n = D_I)."""
    a = stream_args(x, W_c=W_c, v=v, W_g=W_g, g=g, W_cI=W_cI, vI=vI, W_gI=W_gI, gI=gI)
    L = load()
    n = int(L.layer_streams_workspace_size(C.byref(a)))
    ws = _workspace(n, x.device, workspace)
    _check(L.layer_streams(C.byref(a), _ptr(ws), n, _stream(stream)))
    return ws


def output_args(o, W_o, y, *, W_UV=None) -> OutputArgs:
    """o [R][H][D] bf16, W_o [d_model][H*d_h], y [R][d_model]; W_UV [H][d_h][D] or None."""
    R, H, D = int(o.shape[0]), int(o.shape[1]), int(o.shape[2])
    return OutputArgs(_ptr(o), _ptr(W_UV), _ptr(W_o), _ptr(y), R, int(W_o.shape[0]), H, int(W_o.shape[1]) // H, D,
                      dtype_code(y))


def layer_output(o, W_o, y, *, W_UV=None, workspace=None, stream=None):
    a = output_args(o, W_o, y, W_UV=W_UV)
    L = load()
    n = int(L.layer_output_workspace_size(C.byref(a)))
    ws = _workspace(n, o.device, workspace)
    _check(L.layer_output(C.byref(a), _ptr(ws), n, _stream(stream)))
    return ws


def abi_version() -> int:
    return int(load().sckv_abi_version())

"""ctypes binding of libtwell (include/twell.h).  Argument marshalling only:
torch tensors become device pointers, the current torch stream becomes the
hipStream_t, and a non-zero status raises TwellError.  Every step of the
computation runs in the library's HIP kernels; nothing here computes."""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libtwell.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "twell.h")

TWELL_OK, TWELL_EINVAL, TWELL_EUNSUPPORTED, TWELL_EWORKSPACE, TWELL_EHIP = range(5)
TWELL_F32, TWELL_BF16 = 0, 1
R_TILE, C_TILE = 16, 64


class TwellError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libtwell status {status}: {msg}")
        self.status = status


class c_twell_mat(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("F", ctypes.c_int32), ("R", ctypes.c_int32), ("C", ctypes.c_int32),
                ("vdtype", ctypes.c_int), ("cnt", ctypes.c_void_p), ("width", ctypes.c_void_p),
                ("val", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("mask", ctypes.c_void_p)]


class c_twell_cmat(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("F", ctypes.c_int32), ("W", ctypes.c_int32),
                ("cnt", ctypes.c_void_p), ("width", ctypes.c_void_p), ("val", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("ovf", ctypes.c_void_p)]


class c_twell_ffn_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("F", ctypes.c_int32),
                ("in_dt", ctypes.c_int), ("out_dt", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtwell.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparse_feedforward_gate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.twell_mat_bytes.argtypes = [i32, i32, i32, i32, ctypes.c_int, P(sz)]
        L.twell_mat_bytes.restype = sz
        L.twell_pack.argtypes = [vp, ctypes.c_int, i64, P(c_twell_mat), vp]
        L.twell_unpack.argtypes = [P(c_twell_mat), vp, i64, vp]
        L.twell_ffn_fwd_workspace.argtypes = [P(c_twell_ffn_shape), i32]
        L.twell_ffn_fwd_workspace.restype = sz
        L.twell_ffn_fwd.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_mat), i32, vp, sz, vp]
        L.twell_ffn_bwd_workspace.argtypes = [P(c_twell_ffn_shape), i32]
        L.twell_ffn_bwd_workspace.restype = sz
        L.twell_ffn_bwd_hybrid.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_mat), i32,
                                           vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.twell_ffn_bwd_hybrid_l1.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_mat), i32,
                                              ctypes.c_float, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.twell_ffn_fwd_ex.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_mat), i32, vp, sz, vp,
                                       vp, i32]
        L.twell_gate_pack.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, P(c_twell_mat), vp]
        L.twell_sparse_up.argtypes = [P(c_twell_ffn_shape), vp, vp, P(c_twell_mat), vp, vp]
        L.twell_sparse_down.argtypes = [P(c_twell_ffn_shape), vp, vp, P(c_twell_mat), vp, vp]
        L.twell_ffn_dense_fwd_workspace.argtypes = [P(c_twell_ffn_shape)]
        L.twell_ffn_dense_fwd_workspace.restype = sz
        L.twell_ffn_dense_fwd.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.twell_relu_ffn_fwd_workspace.argtypes = [P(c_twell_ffn_shape)]
        L.twell_relu_ffn_fwd_workspace.restype = sz
        L.twell_relu_ffn_fwd.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, P(c_twell_mat), vp, sz, vp]
        L.twell_relu_ffn_dense_fwd_workspace.argtypes = [P(c_twell_ffn_shape)]
        L.twell_relu_ffn_dense_fwd_workspace.restype = sz
        L.twell_relu_ffn_dense_fwd.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, sz, vp]
        L.twell_ffn_dense_bwd_workspace.argtypes = [P(c_twell_ffn_shape)]
        L.twell_ffn_dense_bwd_workspace.restype = sz
        L.twell_ffn_dense_bwd.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          sz, vp]
        L.twell_cmat_bytes.argtypes = [i32, i32, i32, P(sz)]
        L.twell_cmat_bytes.restype = sz
        L.twell_compact.argtypes = [P(c_twell_mat), P(c_twell_cmat), vp]
        L.twell_expand.argtypes = [P(c_twell_cmat), P(c_twell_mat), vp]
        L.twell_ffn_bwd_compact_workspace.argtypes = [P(c_twell_ffn_shape), i32, i32]
        L.twell_ffn_bwd_compact_workspace.restype = sz
        L.twell_ffn_bwd_hybrid_compact.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_cmat),
                                                   i32, ctypes.c_float, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.twell_ffn_fwd_noalloc.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_mat), i32, vp]
        L.twell_ffn_fwd_compact_workspace.argtypes = [P(c_twell_ffn_shape), i32]
        L.twell_ffn_fwd_compact_workspace.restype = sz
        L.twell_ffn_fwd_compact.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, P(c_twell_cmat), i32, vp,
                                            sz, vp]
        L.twell_relu_ffn_fwd_bounded_workspace.argtypes = [P(c_twell_ffn_shape), i32, i32]
        L.twell_relu_ffn_fwd_bounded_workspace.restype = sz
        L.twell_relu_ffn_fwd_bounded.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, i32, i32, vp, vp, sz,
                                                 vp]
        L.twell_ffn_fwd_bounded_workspace.argtypes = [P(c_twell_ffn_shape), i32, i32]
        L.twell_ffn_fwd_bounded_workspace.restype = sz
        L.twell_ffn_fwd_bounded.argtypes = [P(c_twell_ffn_shape), vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.twell_status_string.argtypes = [ctypes.c_int]
        L.twell_status_string.restype = ctypes.c_char_p
        L.twell_last_error.argtypes = []
        L.twell_last_error.restype = ctypes.c_char_p
        for name in ("twell_pack", "twell_unpack", "twell_ffn_fwd", "twell_ffn_fwd_ex", "twell_ffn_bwd_hybrid",
                     "twell_ffn_bwd_hybrid_l1", "twell_compact", "twell_expand", "twell_ffn_bwd_hybrid_compact",
                     "twell_relu_ffn_fwd", "twell_relu_ffn_dense_fwd",
                     "twell_ffn_dense_fwd", "twell_ffn_dense_bwd",
                     "twell_gate_pack",
                     "twell_sparse_up", "twell_sparse_down", "twell_ffn_fwd_noalloc", "twell_ffn_fwd_bounded",
                     "twell_ffn_fwd_compact", "twell_relu_ffn_fwd_bounded"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/twell.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(twell_[a-z_0-9]+)\s*\(", txt)))


def _check(st: int):
    if st != TWELL_OK:
        raise TwellError(st, lib().twell_last_error().decode())


# ---------------------------------------------------------------- marshalling

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_obj(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dt(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.float32:
        return TWELL_F32
    if torch_dtype == torch.bfloat16:
        return TWELL_BF16
    raise TypeError(f"unsupported dtype {torch_dtype}")


@dataclass
class TwellMat:
    """Device arrays of one TwELL matrix (see twell_mat in include/twell.h)."""
    T: int
    F: int
    vdtype: int
    cnt: object
    width: object
    val: object
    idx: object
    mask: Optional[object]
    R: int = R_TILE
    C: int = C_TILE

    @property
    def NR(self) -> int:
        return -(-self.T // self.R)

    @property
    def NT(self) -> int:
        return -(-self.F // self.C)

    def c(self) -> c_twell_mat:
        return c_twell_mat(self.T, self.F, self.R, self.C, self.vdtype, _ptr(self.cnt), _ptr(self.width),
                           _ptr(self.val), _ptr(self.idx), _ptr(self.mask))


def alloc_twell_mat(T: int, F: int, vdtype: int = TWELL_F32, device="cuda", with_mask: bool = True) -> TwellMat:
    """Allocate the arrays of a T x F TwELL matrix with torch (plumbing only)."""
    import torch
    NR, NT = -(-T // R_TILE), -(-F // C_TILE)
    vt = torch.float32 if vdtype == TWELL_F32 else torch.bfloat16
    return TwellMat(
        T, F, vdtype,
        cnt=torch.empty((T, NT), dtype=torch.uint8, device=device),
        width=torch.empty((NR, NT), dtype=torch.uint8, device=device),
        val=torch.empty((NR, NT, C_TILE, R_TILE), dtype=vt, device=device),
        idx=torch.empty((NR, NT, C_TILE, R_TILE), dtype=torch.uint8, device=device),
        mask=torch.empty((T, NT), dtype=torch.int64, device=device) if with_mask else None,
    )


@dataclass
class TwellCMat:
    """Device arrays of one compact TwELL matrix (see twell_cmat in include/twell.h)."""
    T: int
    F: int
    W: int
    cnt: object
    width: object
    val: object
    idx: object
    mask: object
    ovf: object

    def c(self) -> c_twell_cmat:
        return c_twell_cmat(self.T, self.F, self.W, _ptr(self.cnt), _ptr(self.width), _ptr(self.val),
                            _ptr(self.idx), _ptr(self.mask), _ptr(self.ovf))


def alloc_twell_cmat(T: int, F: int, W: int, device="cuda") -> TwellCMat:
    """Allocate the arrays of a T x F compact TwELL matrix of capacity W with torch (plumbing only)."""
    import torch
    NR, NT = -(-T // R_TILE), -(-F // C_TILE)
    return TwellCMat(
        T, F, W,
        cnt=torch.empty((T, NT), dtype=torch.uint8, device=device),
        width=torch.empty((NR, NT), dtype=torch.uint8, device=device),
        val=torch.empty((NR, NT, W, R_TILE), dtype=torch.float32, device=device),
        idx=torch.empty((NR, NT, W, R_TILE), dtype=torch.uint8, device=device),
        mask=torch.empty((T, NT), dtype=torch.int64, device=device),
        ovf=torch.empty((T,), dtype=torch.uint8, device=device),
    )


def ffn_shape(T: int, d: int, F: int, in_dt: int, out_dt: int) -> c_twell_ffn_shape:
    return c_twell_ffn_shape(T, d, F, in_dt, out_dt)


# ---------------------------------------------------------------- entry points

def twell_mat_bytes(T: int, F: int, R: int = R_TILE, C: int = C_TILE, vdtype: int = TWELL_F32):
    parts = (ctypes.c_size_t * 5)()
    total = lib().twell_mat_bytes(T, F, R, C, vdtype, parts)
    return int(total), [int(p) for p in parts]


def twell_pack(G, out: TwellMat, stream=None) -> None:
    m = out.c()
    _check(lib().twell_pack(_ptr(G), _dt(G.dtype), G.stride(0), ctypes.byref(m), _stream(stream)))


def twell_unpack(m: TwellMat, H, stream=None) -> None:
    cm = m.c()
    _check(lib().twell_unpack(ctypes.byref(cm), _ptr(H), H.stride(0), _stream(stream)))


def twell_ffn_fwd_workspace(shape: c_twell_ffn_shape, training: bool = False) -> int:
    return int(lib().twell_ffn_fwd_workspace(ctypes.byref(shape), int(training)))


def twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, saved_h: Optional[TwellMat], dense_row_threshold: int,
                  ws, stream=None) -> None:
    sh = saved_h.c() if saved_h is not None else None
    _check(lib().twell_ffn_fwd(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd), _ptr(y),
                               ctypes.byref(sh) if sh is not None else None, dense_row_threshold,
                               _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                               _stream(stream)))


def twell_relu_ffn_fwd_bounded_workspace(shape: c_twell_ffn_shape, tile_cap: int, union_cap: int) -> int:
    return int(lib().twell_relu_ffn_fwd_bounded_workspace(ctypes.byref(shape), int(tile_cap), int(union_cap)))


def twell_relu_ffn_fwd_bounded(shape, x, W1T, b1, W2, y, tile_cap: int, union_cap: int, ws, n_over_blocks=None,
                               stream=None) -> None:
    """The capacity-bounded non-gated layer (see twell_ffn_fwd_bounded)."""
    _check(lib().twell_relu_ffn_fwd_bounded(ctypes.byref(shape), _ptr(x), _ptr(W1T), _ptr(b1), _ptr(W2), _ptr(y),
                                            int(tile_cap), int(union_cap), _ptr(n_over_blocks), _ptr(ws),
                                            ws.numel() * ws.element_size() if ws is not None else 0,
                                            _stream(stream)))


def twell_ffn_fwd_bounded_workspace(shape: c_twell_ffn_shape, tile_cap: int, union_cap: int) -> int:
    return int(lib().twell_ffn_fwd_bounded_workspace(ctypes.byref(shape), int(tile_cap), int(union_cap)))


def twell_ffn_fwd_bounded(shape, x, WgT, bg, WuT, Wd, y, tile_cap: int, union_cap: int, ws,
                          n_over_blocks=None, stream=None) -> None:
    """The capacity-bounded inference forward; n_over_blocks: optional device
    int32 tensor of one element that receives the blocks computed per pair."""
    _check(lib().twell_ffn_fwd_bounded(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                       _ptr(y), int(tile_cap), int(union_cap), _ptr(n_over_blocks), _ptr(ws),
                                       ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20        # TWELL_NOALLOC_SCRATCH_BYTES of include/twell.h


def twell_ffn_fwd_noalloc(shape, x, WgT, bg, WuT, Wd, y, saved_h: Optional[TwellMat], dense_row_threshold: int,
                          stream=None) -> None:
    """twell_ffn_fwd on the library's static scratch (no workspace argument)."""
    sh = saved_h.c() if saved_h is not None else None
    _check(lib().twell_ffn_fwd_noalloc(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                       _ptr(y), ctypes.byref(sh) if sh is not None else None, dense_row_threshold,
                                       _stream(stream)))


def twell_ffn_bwd_workspace(shape: c_twell_ffn_shape, dense_row_threshold: int) -> int:
    return int(lib().twell_ffn_bwd_workspace(ctypes.byref(shape), int(dense_row_threshold)))


def twell_ffn_bwd_hybrid(shape, x, WgT, bg, WuT, Wd, dY, saved_h: TwellMat, dense_row_threshold: int,
                         dX, dWgT, dWuT, dWd, dbg, n_dense_rows, ws, stream=None) -> None:
    hm = saved_h.c()
    _check(lib().twell_ffn_bwd_hybrid(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                      _ptr(dY), ctypes.byref(hm), int(dense_row_threshold), _ptr(dX), _ptr(dWgT),
                                      _ptr(dWuT), _ptr(dWd), _ptr(dbg), _ptr(n_dense_rows), _ptr(ws),
                                      ws.numel() * ws.element_size() if ws is not None else 0,
                                      _stream(stream)))


def twell_relu_ffn_fwd_workspace(shape) -> int:
    return int(lib().twell_relu_ffn_fwd_workspace(ctypes.byref(shape)))


def twell_relu_ffn_fwd(shape, x, W1T, b1, W2, y, saved_h: Optional[TwellMat], ws, stream=None) -> None:
    hm = saved_h.c() if saved_h is not None else None
    _check(lib().twell_relu_ffn_fwd(ctypes.byref(shape), _ptr(x), _ptr(W1T), _ptr(b1), _ptr(W2), _ptr(y),
                                    ctypes.byref(hm) if hm is not None else None, _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def twell_relu_ffn_dense_fwd_workspace(shape) -> int:
    return int(lib().twell_relu_ffn_dense_fwd_workspace(ctypes.byref(shape)))


def twell_relu_ffn_dense_fwd(shape, x, W1T, b1, W2, y, ws, stream=None) -> None:
    _check(lib().twell_relu_ffn_dense_fwd(ctypes.byref(shape), _ptr(x), _ptr(W1T), _ptr(b1), _ptr(W2), _ptr(y),
                                          _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                          _stream(stream)))


def twell_ffn_bwd_hybrid_l1(shape, x, WgT, bg, WuT, Wd, dY, saved_h: TwellMat, dense_row_threshold: int,
                            l1_lambda: float, l1_per_token_mean: bool, dX, dWgT, dWuT, dWd, dbg, n_dense_rows, ws,
                            stream=None) -> None:
    hm = saved_h.c()
    _check(lib().twell_ffn_bwd_hybrid_l1(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                         _ptr(dY), ctypes.byref(hm), int(dense_row_threshold), float(l1_lambda),
                                         int(bool(l1_per_token_mean)), _ptr(dX), _ptr(dWgT), _ptr(dWuT), _ptr(dWd),
                                         _ptr(dbg), _ptr(n_dense_rows), _ptr(ws),
                                         ws.numel() * ws.element_size() if ws is not None else 0,
                                         _stream(stream)))


def twell_cmat_bytes(T: int, F: int, W: int):
    parts = (ctypes.c_size_t * 6)()
    total = lib().twell_cmat_bytes(T, F, W, parts)
    return int(total), [int(p) for p in parts]


def twell_compact(full: TwellMat, out: TwellCMat, stream=None) -> None:
    fm, cm = full.c(), out.c()
    _check(lib().twell_compact(ctypes.byref(fm), ctypes.byref(cm), _stream(stream)))


def twell_expand(c: TwellCMat, full: TwellMat, stream=None) -> None:
    cm, fm = c.c(), full.c()
    _check(lib().twell_expand(ctypes.byref(cm), ctypes.byref(fm), _stream(stream)))


def twell_ffn_bwd_compact_workspace(shape: c_twell_ffn_shape, dense_row_threshold: int, W: int) -> int:
    return int(lib().twell_ffn_bwd_compact_workspace(ctypes.byref(shape), int(dense_row_threshold), int(W)))


def twell_ffn_fwd_compact_workspace(shape: c_twell_ffn_shape, W: int) -> int:
    return int(lib().twell_ffn_fwd_compact_workspace(ctypes.byref(shape), int(W)))


def twell_ffn_fwd_compact(shape, x, WgT, bg, WuT, Wd, y, saved: TwellCMat, dense_row_threshold: int, ws,
                          stream=None) -> None:
    """The hybrid training forward saving h straight into the compact form."""
    cm = saved.c()
    _check(lib().twell_ffn_fwd_compact(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                       _ptr(y), ctypes.byref(cm), int(dense_row_threshold), _ptr(ws),
                                       ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def twell_ffn_bwd_hybrid_compact(shape, x, WgT, bg, WuT, Wd, dY, saved: TwellCMat, dense_row_threshold: int,
                                 l1_lambda: float, l1_per_token_mean: bool, dX, dWgT, dWuT, dWd, dbg, n_dense_rows,
                                 ws, stream=None) -> None:
    cm = saved.c()
    _check(lib().twell_ffn_bwd_hybrid_compact(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT),
                                              _ptr(Wd), _ptr(dY), ctypes.byref(cm), int(dense_row_threshold),
                                              float(l1_lambda), int(bool(l1_per_token_mean)), _ptr(dX), _ptr(dWgT),
                                              _ptr(dWuT), _ptr(dWd), _ptr(dbg), _ptr(n_dense_rows), _ptr(ws),
                                              ws.numel() * ws.element_size() if ws is not None else 0,
                                              _stream(stream)))


def twell_ffn_fwd_ex(shape, x, WgT, bg, WuT, Wd, y, saved_h: Optional[TwellMat], dense_row_threshold: int,
                     ws, events, stream=None) -> None:
    """twell_ffn_fwd recording the torch.cuda.Event objects in `events` at the
    stage boundaries (see include/twell.h)."""
    sh = saved_h.c() if saved_h is not None else None
    for e in events:                 # torch creates the HIP event on its first record
        if not e.cuda_event:
            e.record(_stream_obj(stream))
    arr = (ctypes.c_void_p * max(1, len(events)))(*[e.cuda_event for e in events])
    _check(lib().twell_ffn_fwd_ex(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd), _ptr(y),
                                  ctypes.byref(sh) if sh is not None else None, dense_row_threshold,
                                  _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                  _stream(stream), arr, len(events)))


def twell_gate_pack(shape, x, WgT, bg, h: TwellMat, stream=None) -> None:
    hm = h.c()
    _check(lib().twell_gate_pack(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), ctypes.byref(hm),
                                 _stream(stream)))


def twell_sparse_up(shape, x, WuT, h: TwellMat, aval, stream=None) -> None:
    hm = h.c()
    _check(lib().twell_sparse_up(ctypes.byref(shape), _ptr(x), _ptr(WuT), ctypes.byref(hm), _ptr(aval),
                                 _stream(stream)))


def twell_sparse_down(shape, aval, Wd, pattern: TwellMat, y, stream=None) -> None:
    pm = pattern.c()
    _check(lib().twell_sparse_down(ctypes.byref(shape), _ptr(aval), _ptr(Wd), ctypes.byref(pm), _ptr(y),
                                   _stream(stream)))


def twell_ffn_dense_fwd_workspace(shape: c_twell_ffn_shape) -> int:
    return int(lib().twell_ffn_dense_fwd_workspace(ctypes.byref(shape)))


def twell_ffn_dense_fwd(shape, x, WgT, bg, WuT, Wd, y, ws, stream=None) -> None:
    _check(lib().twell_ffn_dense_fwd(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                     _ptr(y), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream(stream)))


def twell_ffn_dense_bwd_workspace(shape: c_twell_ffn_shape) -> int:
    return int(lib().twell_ffn_dense_bwd_workspace(ctypes.byref(shape)))


def twell_ffn_dense_bwd(shape, x, WgT, bg, WuT, Wd, dY, y, dX, dWgT, dWuT, dWd, dbg, ws, stream=None) -> None:
    _check(lib().twell_ffn_dense_bwd(ctypes.byref(shape), _ptr(x), _ptr(WgT), _ptr(bg), _ptr(WuT), _ptr(Wd),
                                     _ptr(dY), _ptr(y), _ptr(dX), _ptr(dWgT), _ptr(dWuT), _ptr(dWd), _ptr(dbg),
                                     _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream(stream)))


def twell_status_string(st: int) -> str:
    return lib().twell_status_string(st).decode()


def twell_last_error() -> str:
    return lib().twell_last_error().decode()

"""Host-side checks of libtwell that need no GPU: the library loads against
the installed ROCm runtime, exports every function include/twell.h declares,
and rejects bad arguments before launching anything."""
import ctypes
import os
import subprocess

import pytest

import activation_sparse_feedforward_gate_amd as tw
from activation_sparse_feedforward_gate_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_header_function():
    L = tw.lib()
    names = tw.header_functions()
    assert {"twell_pack", "twell_ffn_fwd", "twell_ffn_dense_fwd", "twell_unpack"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libtwell.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_header_is_plain_c():
    """The public header compiles as C (no torch, no C++ types in signatures)."""
    src = '#include "twell.h"\nint main(void){ twell_mat m; (void)m; return (int)TWELL_OK; }\n'
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_mat_bytes():
    total, parts = tw.twell_mat_bytes(33, 128, 16, 64, tw.TWELL_F32)
    NR, NT = 3, 2
    assert parts == [33 * NT, NR * NT, NR * NT * 64 * 16 * 4, NR * NT * 64 * 16, 33 * NT * 8]
    assert total == sum(parts)
    _, p16 = tw.twell_mat_bytes(33, 128, 16, 64, tw.TWELL_BF16)
    assert p16[2] == NR * NT * 64 * 16 * 2


def _call_fwd(shape, **kw):
    L = tw.lib()
    args = dict(x=16, WgT=32, bg=None, WuT=48, Wd=64, y=80, saved=None, thr=-1, ws=None, ws_bytes=0)
    args.update(kw)
    return L.twell_ffn_fwd(ctypes.byref(shape) if shape is not None else None, args["x"], args["WgT"], args["bg"],
                           args["WuT"], args["Wd"], args["y"], args["saved"], args["thr"], args["ws"],
                           args["ws_bytes"], None)


def test_fwd_argument_errors_are_synchronous():
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    assert _call_fwd(None) == tw.TWELL_EINVAL
    assert _call_fwd(sh, x=None) == tw.TWELL_EINVAL
    assert _call_fwd(tw.ffn_shape(64, 100, 512, tw.TWELL_BF16, tw.TWELL_F32)) == tw.TWELL_EUNSUPPORTED
    assert _call_fwd(tw.ffn_shape(64, 128, 500, tw.TWELL_BF16, tw.TWELL_F32)) == tw.TWELL_EUNSUPPORTED
    assert _call_fwd(tw.ffn_shape(-1, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)) == tw.TWELL_EINVAL
    assert _call_fwd(tw.ffn_shape(64, 128, 512, 7, tw.TWELL_F32)) == tw.TWELL_EINVAL
    assert _call_fwd(sh, x=16 + 2) == tw.TWELL_EINVAL         # misaligned
    need = tw.twell_ffn_fwd_workspace(sh)
    assert need > 0
    assert _call_fwd(sh, ws=4096, ws_bytes=need - 1) == tw.TWELL_EWORKSPACE
    assert b"workspace" in L.twell_last_error()
    # empty batch: nothing to do, nothing launched
    assert _call_fwd(tw.ffn_shape(0, 128, 512, tw.TWELL_BF16, tw.TWELL_F32), ws=4096,
                     ws_bytes=tw.twell_ffn_fwd_workspace(tw.ffn_shape(0, 128, 512, tw.TWELL_BF16, tw.TWELL_F32))) \
        == tw.TWELL_OK


def test_pack_argument_errors():
    L = tw.lib()
    m = tw.c_twell_mat(32, 128, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, None)
    assert L.twell_pack(None, tw.TWELL_F32, 128, ctypes.byref(m), None) == tw.TWELL_EINVAL
    assert L.twell_pack(64, tw.TWELL_BF16, 128, ctypes.byref(m), None) == tw.TWELL_EINVAL   # dtype mismatch
    assert L.twell_pack(64, tw.TWELL_F32, 64, ctypes.byref(m), None) == tw.TWELL_EINVAL     # ldg < F
    m8 = tw.c_twell_mat(32, 128, 8, 64, tw.TWELL_F32, 16, 16, 16, 16, None)
    assert L.twell_pack(64, tw.TWELL_F32, 128, ctypes.byref(m8), None) == tw.TWELL_EUNSUPPORTED
    m0 = tw.c_twell_mat(0, 128, 16, 64, tw.TWELL_F32, None, None, None, None, None)
    assert L.twell_pack(None, tw.TWELL_F32, 128, ctypes.byref(m0), None) == tw.TWELL_OK
    assert L.twell_pack(64, tw.TWELL_F32, 128, None, None) == tw.TWELL_EINVAL


def test_dense_baseline_argument_errors():
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_F32, tw.TWELL_F32)
    assert L.twell_ffn_dense_fwd(ctypes.byref(sh), 16, 16, None, 16, 16, 16, 16, 1 << 20, None) == tw.TWELL_EUNSUPPORTED
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    assert L.twell_ffn_dense_fwd(ctypes.byref(sh), 16, 16, None, 16, 16, 16, 16, 1, None) == tw.TWELL_EWORKSPACE


def test_dense_train_baseline_argument_errors():
    L = tw.lib()
    args = [16] * 13 + [1 << 30, None]      # x WgT bg WuT Wd dY y dX dWgT dWuT dWd dbg ws, ws_bytes, stream
    sh = tw.ffn_shape(64, 256, 512, tw.TWELL_F32, tw.TWELL_F32)
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *args) == tw.TWELL_EUNSUPPORTED        # fp32 inputs
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *args) == tw.TWELL_EUNSUPPORTED        # d % 256
    sh = tw.ffn_shape(100, 256, 512, tw.TWELL_BF16, tw.TWELL_F32)
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *args) == tw.TWELL_EUNSUPPORTED        # T % 64
    sh = tw.ffn_shape(64, 256, 512, tw.TWELL_BF16, tw.TWELL_F32)
    need = tw.twell_ffn_dense_bwd_workspace(sh)
    assert need >= 5 * 64 * 512 * 2
    small = [16] * 13 + [need - 1, None]
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *small) == tw.TWELL_EWORKSPACE
    bad = [16] * 8 + [None] + [16] * 4 + [need, None]                 # dWgT missing
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *bad) == tw.TWELL_EINVAL
    unaligned = [16] * 6 + [24] + [16] * 6 + [need, None]             # y misaligned
    assert L.twell_ffn_dense_bwd(ctypes.byref(sh), *unaligned) == tw.TWELL_EINVAL


def test_bwd_argument_errors():
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)
    need = tw.twell_ffn_bwd_workspace(sh, 51)
    assert need > 0
    assert tw.twell_ffn_bwd_workspace(sh, 51) < tw.twell_ffn_bwd_workspace(sh, 512)   # pair index sized by tau

    def call(shape=sh, hm=h, x=16, dY=16, dX=16, dW=16, ws=4096, ws_bytes=need, tau=51):
        return L.twell_ffn_bwd_hybrid(ctypes.byref(shape) if shape is not None else None, x, 16, None, 16, 16, dY,
                                      ctypes.byref(hm) if hm is not None else None, tau, dX, dW, dW, dW, None,
                                      None, ws, ws_bytes, None)
    assert call(shape=None) == tw.TWELL_EINVAL
    assert call(hm=None) == tw.TWELL_EINVAL
    assert call(dY=None) == tw.TWELL_EINVAL
    assert call(dW=None) == tw.TWELL_EINVAL
    assert call(x=24) == tw.TWELL_EINVAL                                       # misaligned
    assert call(ws_bytes=need - 1) == tw.TWELL_EWORKSPACE
    hb = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_BF16, 16, 16, 16, 16, 16)
    assert call(hm=hb) == tw.TWELL_EINVAL                                      # saved h must hold fp32
    hn = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, None)
    assert call(hm=hn) == tw.TWELL_EINVAL                                      # mask required
    h32 = tw.c_twell_mat(32, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)
    assert call(hm=h32) == tw.TWELL_EINVAL                                     # T mismatch
    assert call(shape=tw.ffn_shape(64, 100, 512, tw.TWELL_BF16, tw.TWELL_F32)) == tw.TWELL_EUNSUPPORTED


def test_bwd_l1_argument_errors():
    """The penalty's coefficient and normalisation flag are checked before any
    launch (so these calls need no GPU)."""
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)
    need = tw.twell_ffn_bwd_workspace(sh, 51)

    def call(lam, mean):
        return L.twell_ffn_bwd_hybrid_l1(ctypes.byref(sh), 16, 16, None, 16, 16, 16, ctypes.byref(h), 51,
                                         ctypes.c_float(lam), mean, 16, 16, 16, 16, None, None, 4096, need, None)
    assert call(-1e-5, 0) == tw.TWELL_EINVAL
    assert call(float("nan"), 0) == tw.TWELL_EINVAL
    assert call(float("inf"), 1) == tw.TWELL_EINVAL
    assert call(2e-5, 2) == tw.TWELL_EINVAL
    assert b"l1" in L.twell_last_error()


def test_cmat_bytes():
    total, parts = tw.twell_cmat_bytes(33, 128, 5)
    NR, NT = 3, 2
    assert parts == [33 * NT, NR * NT, NR * NT * 5 * 16 * 4, NR * NT * 5 * 16, 33 * NT * 8, 33]
    assert total == sum(parts)
    full, fparts = tw.twell_mat_bytes(33, 128)
    assert tw.twell_cmat_bytes(33, 128, 64)[1][:5] == fparts                   # W = 64 is the full layout
    for bad in ((33, 128, 0), (33, 128, 65), (33, 100, 4), (-1, 128, 4)):
        assert tw.twell_cmat_bytes(*bad)[0] == 0


def test_compact_argument_errors():
    """twell_compact / twell_expand check shapes, capacity and pointers
    before any launch (so these calls need no GPU)."""
    L = tw.lib()
    full = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)

    def cm(T=64, F=512, W=4, ovf=16, val=16):
        return tw.c_twell_cmat(T, F, W, 16, 16, val, 16, 16, ovf)

    for f in (L.twell_compact, L.twell_expand):
        def a(m, c, f=f):
            return (m, c) if f is L.twell_compact else (c, m)
        for c in (cm(W=0), cm(W=65), cm(T=32), cm(F=448), cm(ovf=None), cm(val=24)):
            x, y = a(ctypes.byref(full), ctypes.byref(c))
            assert f(x, y, None) == tw.TWELL_EINVAL, (f, c.T, c.F, c.W)
        x, y = a(None, ctypes.byref(cm()))
        assert f(x, y, None) == tw.TWELL_EINVAL
        bf = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_BF16, 16, 16, 16, 16, 16)
        x, y = a(ctypes.byref(bf), ctypes.byref(cm()))
        assert f(x, y, None) == tw.TWELL_EINVAL                                # fp32 values only
        nomask = tw.c_twell_mat(64, 512, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, None)
        x, y = a(ctypes.byref(nomask), ctypes.byref(cm()))
        assert f(x, y, None) == tw.TWELL_EINVAL
    empty_full = tw.c_twell_mat(0, 512, 16, 64, tw.TWELL_F32, None, None, None, None, None)
    empty = tw.c_twell_cmat(0, 512, 4, None, None, None, None, None, None)
    assert L.twell_compact(ctypes.byref(empty_full), ctypes.byref(empty), None) == tw.TWELL_OK


def test_bwd_compact_argument_errors():
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    c = tw.c_twell_cmat(64, 512, 4, 16, 16, 16, 16, 16, 16)
    need = tw.twell_ffn_bwd_compact_workspace(sh, 51, 4)
    # the three per-pair value arrays of the backward shrink from 64 to W slots per tile
    full = tw.twell_ffn_bwd_workspace(sh, 51)
    assert tw.twell_ffn_bwd_compact_workspace(sh, 51, 64) == full
    slots = 4 * 8 * 16 * 4                         # NR * NT * 16 rows, per slot of a tile, fp32
    # at most that much smaller (the sparse branch's buffers overlay the dense
    # branch's [T][3F] fp32-sized buffer, which may then set the size)
    assert 0 < full - need <= 3 * slots * (64 - 4) + 3 * 256
    assert need >= 64 * 3 * 512 * 4
    assert tw.twell_ffn_bwd_compact_workspace(sh, 51, 0) == 0
    assert tw.twell_ffn_bwd_compact_workspace(sh, 51, 65) == 0

    def call(cmat=c, lam=0.0, ws_bytes=need, dY=16):
        return L.twell_ffn_bwd_hybrid_compact(ctypes.byref(sh), 16, 16, None, 16, 16, dY,
                                              ctypes.byref(cmat) if cmat is not None else None, 51,
                                              ctypes.c_float(lam), 0, 16, 16, 16, 16, None, None, 4096, ws_bytes,
                                              None)
    assert call(cmat=None) == tw.TWELL_EINVAL
    assert call(cmat=tw.c_twell_cmat(64, 512, 4, 16, 16, 16, 16, 16, None)) == tw.TWELL_EINVAL   # ovf required
    assert call(cmat=tw.c_twell_cmat(64, 512, 70, 16, 16, 16, 16, 16, 16)) == tw.TWELL_EINVAL
    assert call(cmat=tw.c_twell_cmat(32, 512, 4, 16, 16, 16, 16, 16, 16)) == tw.TWELL_EINVAL
    assert call(lam=-1.0) == tw.TWELL_EINVAL
    assert call(dY=None) == tw.TWELL_EINVAL
    assert call(ws_bytes=need - 1) == tw.TWELL_EWORKSPACE


def test_hybrid_fwd_needs_saved_h():
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    need = tw.twell_ffn_fwd_workspace(sh, True)
    assert need >= tw.twell_ffn_fwd_workspace(sh, False)     # a training-sized workspace serves inference too
    assert _call_fwd(sh, thr=5, ws=4096, ws_bytes=need) == tw.TWELL_EINVAL


def test_status_strings():
    for st in range(5):
        assert tw.twell_status_string(st)


def test_shape_limits_of_32bit_offsets():
    """Shapes whose [T][d], [F][d] or [T][F] 16-bit matrices reach 2^31
    elements (the GEMM mainloops' 32-bit byte offsets) are refused before any
    launch, by every entry point that takes a shape; one element fewer passes
    the check (and then stops at the missing workspace)."""
    L = tw.lib()
    lim = 1 << 31
    cases = [
        (lim // 2048, 2048, 64),          # T*d == 2^31
        (64, 2048, lim // 2048),          # F*d == 2^31 (F = 2^20 > 65472 is refused anyway)
        (lim // 8192, 64, 8192),          # T*F == 2^31
    ]
    for T, d, F in cases:
        sh = tw.ffn_shape(T, d, F, tw.TWELL_BF16, tw.TWELL_F32)
        assert _call_fwd(sh, ws=4096, ws_bytes=1 << 40) == tw.TWELL_EUNSUPPORTED, (T, d, F)
        assert tw.twell_ffn_fwd_workspace(sh) == 0
        assert L.twell_ffn_dense_fwd(ctypes.byref(sh), 16, 16, None, 16, 16, 16, 4096, 1 << 40, None) \
            == tw.TWELL_EUNSUPPORTED
        assert L.twell_relu_ffn_fwd(ctypes.byref(sh), 16, 16, None, 16, 16, None, 4096, 1 << 40, None) \
            == tw.TWELL_EUNSUPPORTED
    # T*d one row below the limit: the shape passes, the call stops at the workspace
    sh = tw.ffn_shape(lim // 2048 - 1, 2048, 64, tw.TWELL_BF16, tw.TWELL_F32)
    assert _call_fwd(sh, ws=4096, ws_bytes=1) == tw.TWELL_EWORKSPACE
    # T*F one row below the limit
    sh = tw.ffn_shape(lim // 8192 - 1, 64, 8192, tw.TWELL_BF16, tw.TWELL_F32)
    assert _call_fwd(sh, ws=4096, ws_bytes=1) == tw.TWELL_EWORKSPACE


def test_bwd_shape_limit_of_dense_branch_buffer():
    """The backward also needs 3*T*F < 2^32 (its dense-branch fp32 buffer is
    read with 32-bit element offsets): T*F just under 2^31 passes the shape
    check but is refused here."""
    L = tw.lib()
    F = 8192
    T = (1 << 31) // F - 16                     # T*F < 2^31, 3*T*F > 2^32
    sh = tw.ffn_shape(T, 64, F, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.c_twell_mat(T, F, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)
    st = L.twell_ffn_bwd_hybrid(ctypes.byref(sh), 16, 16, None, 16, 16, 16, ctypes.byref(h), 10, 16, 16, 16, 16,
                                None, None, 4096, 1 << 40, None)
    assert st == tw.TWELL_EUNSUPPORTED
    assert b"3*T*F" in L.twell_last_error()
    T = ((1 << 32) // 3) // F - 16              # 3*T*F < 2^32: passes, stops at the workspace
    sh = tw.ffn_shape(T, 64, F, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.c_twell_mat(T, F, 16, 64, tw.TWELL_F32, 16, 16, 16, 16, 16)
    st = L.twell_ffn_bwd_hybrid(ctypes.byref(sh), 16, 16, None, 16, 16, 16, ctypes.byref(h), 10, 16, 16, 16, 16,
                                None, None, 4096, 1, None)
    assert st == tw.TWELL_EWORKSPACE


def _call_bounded(shape, **kw):
    L = tw.lib()
    args = dict(x=16, WgT=32, bg=None, WuT=48, Wd=64, y=80, W=8, U=256, cnt=None, ws=None, ws_bytes=0)
    args.update(kw)
    return L.twell_ffn_fwd_bounded(ctypes.byref(shape), args["x"], args["WgT"], args["bg"], args["WuT"], args["Wd"],
                                   args["y"], args["W"], args["U"], args["cnt"], args["ws"], args["ws_bytes"], None)


def test_bounded_fwd_workspace_and_argument_errors():
    T, d, F = 4096, 256, 1024
    sh = tw.ffn_shape(T, d, F, tw.TWELL_BF16, tw.TWELL_F32)
    full = tw.twell_ffn_fwd_workspace(sh)
    w8 = tw.twell_ffn_fwd_bounded_workspace(sh, 8, 256)
    w64 = tw.twell_ffn_fwd_bounded_workspace(sh, 64, F)
    # capacities at their maxima: the ordinary forward's buffers (plus the block flags)
    assert full <= w64 <= full + 1024
    # h shrinks by 5 * (64 - 8) / 64 bytes per (t, n) and a by 2 * (F - 256) bytes per token, to 256-byte rounding
    saved = 5 * T * F * (64 - 8) // 64 + 2 * T * (F - 256)
    assert abs((w64 - w8) - saved) <= 2048
    for W, U in [(0, 256), (3, 256), (6, 256), (68, 256), (8, 0), (8, 100), (8, F + 64)]:
        assert tw.twell_ffn_fwd_bounded_workspace(sh, W, U) == 0
        assert _call_bounded(sh, W=W, U=U, ws=256, ws_bytes=w8) == tw.TWELL_EINVAL
    assert tw.twell_ffn_fwd_bounded_workspace(tw.ffn_shape(T, d, F, tw.TWELL_F32, tw.TWELL_F32), 8, 256) == 0
    assert _call_bounded(tw.ffn_shape(T, d, F, tw.TWELL_F32, tw.TWELL_F32)) == tw.TWELL_EUNSUPPORTED
    assert _call_bounded(sh, x=None, ws=256, ws_bytes=w8) == tw.TWELL_EINVAL
    assert _call_bounded(sh, x=24, ws=256, ws_bytes=w8) == tw.TWELL_EINVAL          # misaligned
    assert _call_bounded(sh, ws=256, ws_bytes=w8 - 1) == tw.TWELL_EWORKSPACE
    assert _call_bounded(sh, ws=None, ws_bytes=w8) == tw.TWELL_EWORKSPACE
    # few tokens: the ordinary few-token workspace
    small = tw.ffn_shape(64, d, F, tw.TWELL_BF16, tw.TWELL_F32)
    assert tw.twell_ffn_fwd_bounded_workspace(small, 8, 256) == tw.twell_ffn_fwd_workspace(small)


def test_fwd_compact_argument_errors():
    L = tw.lib()
    sh = tw.ffn_shape(64, 128, 512, tw.TWELL_BF16, tw.TWELL_F32)
    c = tw.c_twell_cmat(64, 512, 4, 16, 16, 16, 16, 16, 16)
    need = tw.twell_ffn_fwd_compact_workspace(sh, 4)
    assert 0 < need < tw.twell_ffn_fwd_workspace(sh, True)     # no capacity-64 TwELL in it
    assert tw.twell_ffn_fwd_compact_workspace(sh, 0) == 0

    def call(cmat=c, thr=51, ws_bytes=need, x=16):
        return L.twell_ffn_fwd_compact(ctypes.byref(sh), x, 16, None, 16, 16, 16,
                                       ctypes.byref(cmat) if cmat is not None else None, thr, 4096, ws_bytes, None)
    assert call(cmat=None) == tw.TWELL_EINVAL
    assert call(cmat=tw.c_twell_cmat(64, 512, 4, 16, 16, 16, 16, 16, None)) == tw.TWELL_EINVAL   # ovf required
    assert call(cmat=tw.c_twell_cmat(64, 512, 0, 16, 16, 16, 16, 16, 16)) == tw.TWELL_EINVAL
    assert call(cmat=tw.c_twell_cmat(32, 512, 4, 16, 16, 16, 16, 16, 16)) == tw.TWELL_EINVAL
    assert call(thr=-1) == tw.TWELL_EINVAL
    assert call(x=None) == tw.TWELL_EINVAL
    assert call(x=24) == tw.TWELL_EINVAL
    assert call(ws_bytes=need - 1) == tw.TWELL_EWORKSPACE


def test_relu_bounded_workspace_and_errors():
    L = tw.lib()
    T, d, F = 4096, 256, 1024
    sh = tw.ffn_shape(T, d, F, tw.TWELL_BF16, tw.TWELL_F32)
    full = tw.twell_relu_ffn_fwd_workspace(sh)
    w8 = tw.twell_relu_ffn_fwd_bounded_workspace(sh, 8, 256)
    assert full <= tw.twell_relu_ffn_fwd_bounded_workspace(sh, 64, F) <= full + 1024
    assert abs((full - w8) - (5 * T * F * (64 - 8) // 64 + 2 * T * (F - 256))) <= 2048
    assert tw.twell_relu_ffn_fwd_bounded_workspace(sh, 6, 256) == 0
    assert tw.twell_relu_ffn_fwd_bounded_workspace(tw.ffn_shape(T, d, F, tw.TWELL_F32, tw.TWELL_F32), 8, 256) == 0

    def call(W=8, U=256, ws_bytes=w8, x=16, shape=sh):
        return L.twell_relu_ffn_fwd_bounded(ctypes.byref(shape), x, 32, None, 48, 64, W, U, None, 256, ws_bytes, None)
    assert call(W=2) == tw.TWELL_EINVAL
    assert call(U=100) == tw.TWELL_EINVAL
    assert call(x=None) == tw.TWELL_EINVAL
    assert call(ws_bytes=w8 - 1) == tw.TWELL_EWORKSPACE
    assert call(shape=tw.ffn_shape(T, d, F, tw.TWELL_F32, tw.TWELL_F32)) == tw.TWELL_EUNSUPPORTED

"""GPU parity of compact TwELL (capacity W slots per (row, tile)) and of the
hybrid backward that reads it.

twell_compact / twell_expand are byte work: they are compared bit for bit
with the oracle's twell_compact / twell_expand of the oracle's own pack of the
same seeded matrix G (the GPU side packs G with twell_pack, itself checked bit
for bit elsewhere).  twell_ffn_fwd_compact, which packs the gate GEMM's
output straight into the compact form, must save exactly twell_compact of the
full-capacity forward's h.  twell_ffn_bwd_hybrid_compact is compared with the float64
oracle's gradients within the hybrid backward's tolerance (relative Frobenius
1e-3 for bf16 inputs, 1e-5 for fp32), on the sparse and dense row sets
separately; the rows the dense branch took must be exactly those of the GPU's
own TwELL with a count above the threshold or a tile count above W.
"""
import numpy as np
import pytest

import oracle as O
from workloads import make_workload

from gpu_util import log, mat_to_numpy, oracle_val_bits, rel_fro, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-3, "f32": 1e-5}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a GPU"
    return _t


@pytest.fixture(scope="module")
def tw():
    import activation_sparse_feedforward_gate_amd as _tw
    _tw.lib()
    return _tw


def _gate_like(rng, T, F):
    """About 7% positive entries (about 4 per 64-wide tile row), a few rows
    far denser, one empty row: tile counts fall on both sides of small W."""
    G = (rng.standard_normal((T, F)) - 1.5).astype(np.float32)
    if T > 8:
        G[3] += 2.0
        G[T // 2] += 1.0
        G[7] = -1.0
    return G


def _cmat_to_numpy(c):
    return {"cnt": c.cnt.cpu().numpy().astype(np.int64), "width": c.width.cpu().numpy().astype(np.int64),
            "val_bits": c.val.cpu().numpy().view(np.uint32), "idx": c.idx.cpu().numpy(),
            "mask": c.mask.cpu().numpy().view(np.uint64), "ovf": c.ovf.cpu().numpy().astype(bool)}


def _compare_slots(got, ref_width, ref_val, ref_idx, what):
    vref = oracle_val_bits(ref_val, "f32")
    NR, NT = ref_width.shape
    for i in range(NR):
        for j in range(NT):
            w = int(ref_width[i, j])
            np.testing.assert_array_equal(got["idx"][i, j, :w], ref_idx[i, j, :w], err_msg=f"{what} idx {i},{j}")
            np.testing.assert_array_equal(got["val_bits"][i, j, :w], vref[i, j, :w], err_msg=f"{what} val {i},{j}")


@pytest.mark.parametrize("T,F,W", [(37, 128, 1), (300, 640, 4), (1000, 4096, 8), (50, 256, 64), (16, 64, 3)])
def test_compact_and_expand_bit_exact(torch, tw, T, F, W):
    log(f"[compact] T={T} F={F} W={W}")
    rng = np.random.default_rng(T * 31 + F + W)
    G = _gate_like(rng, T, F)
    full = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
    tw.twell_pack(to_dev(G, "f32"), full)
    c = tw.alloc_twell_cmat(T, F, W)
    c.ovf.fill_(0xAB)
    tw.twell_compact(full, c)
    back = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
    back.cnt.fill_(0xCD)
    back.width.fill_(0xCD)
    back.mask.fill_(-1)
    tw.twell_expand(c, back)
    torch.cuda.synchronize()

    ref_full = O.twell_pack(G, 16, 64)
    ref = O.twell_compact(ref_full, W)
    got = _cmat_to_numpy(c)
    np.testing.assert_array_equal(got["cnt"], ref.cnt, err_msg="cnt")
    np.testing.assert_array_equal(got["width"], ref.width, err_msg="width")
    np.testing.assert_array_equal(got["ovf"], ref.ovf, err_msg="ovf")
    np.testing.assert_array_equal(got["mask"], mat_to_numpy(full)["mask"], err_msg="mask")
    _compare_slots(got, ref.width, ref.val, ref.idx, "compact")
    n_ovf = int(ref.ovf.sum())
    log(f"   overflow rows {n_ovf} of {T}")
    if W < 8:
        assert 0 < n_ovf < T                      # both kinds of row are exercised

    ref_back = O.twell_expand(ref)
    gb = mat_to_numpy(back)
    np.testing.assert_array_equal(gb["cnt"], ref_back.cnt, err_msg="expanded cnt")
    np.testing.assert_array_equal(gb["width"], ref_back.width, err_msg="expanded width")
    np.testing.assert_array_equal(gb["mask"], got["mask"], err_msg="expanded mask")
    _compare_slots(gb, ref_back.width, ref_back.val, ref_back.idx, "expanded")


def test_compact_full_capacity_is_identity(torch, tw):
    """W = 64: nothing overflows and the compact arrays are the full ones."""
    T, F = 77, 320
    G = _gate_like(np.random.default_rng(9), T, F)
    full = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
    tw.twell_pack(to_dev(G, "f32"), full)
    c = tw.alloc_twell_cmat(T, F, 64)
    tw.twell_compact(full, c)
    torch.cuda.synchronize()
    got, f = _cmat_to_numpy(c), mat_to_numpy(full)
    assert not got["ovf"].any()
    for k in ("cnt", "width", "mask"):
        np.testing.assert_array_equal(got[k], f[k], err_msg=k)
    for i in range(f["width"].shape[0]):
        for j in range(f["width"].shape[1]):
            w = int(f["width"][i, j])
            np.testing.assert_array_equal(got["val_bits"][i, j, :w], f["val_bits"][i, j, :w])


def _run_compact_train(torch, tw, w, tau, W, l1=(0.0, False), bias=True, direct=False):
    """direct: the compact forward writes the saved state; else the full
    forward's saved h is compacted with twell_compact."""
    dt = w.cfg.dtype
    in_dt = tw.TWELL_BF16 if dt == "bf16" else tw.TWELL_F32
    x, WgT, WuT, Wd, dY = (to_dev(a, dt) for a in (w.x, w.WgT, w.WuT, w.Wd, w.dY))
    bg = to_dev(w.bg, dt) if bias else None
    T, d, F = w.T, w.d, w.f
    shape = tw.ffn_shape(T, d, F, in_dt, tw.TWELL_F32)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    c = tw.alloc_twell_cmat(T, F, W)
    if direct:
        c.val.fill_(float("nan"))
        c.idx.fill_(0xEE)
        wsf = torch.empty(max(1, tw.twell_ffn_fwd_compact_workspace(shape, W)), dtype=torch.uint8, device="cuda")
        wsf.fill_(0xFF)
        tw.twell_ffn_fwd_compact(shape, x, WgT, bg, WuT, Wd, y, c, tau, wsf)
        torch.cuda.synchronize()
        h_host = {"cnt": c.cnt.cpu().numpy().astype(np.int64)}
    else:
        h = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
        wsf = torch.empty(max(1, tw.twell_ffn_fwd_workspace(shape, True)), dtype=torch.uint8, device="cuda")
        tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, h, tau, wsf)
        tw.twell_compact(h, c)
        torch.cuda.synchronize()
        h_host = mat_to_numpy(h)
        # the full form is no longer needed: scribble over it so that a backward
        # that still read it would fail
        h.val.fill_(float("nan"))
        h.idx.fill_(0xEE)
    dX = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    dW = [torch.full((F, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    dbg = torch.full((F,), float("nan"), dtype=torch.float32, device="cuda")
    nD = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    wsb = torch.empty(max(1, tw.twell_ffn_bwd_compact_workspace(shape, tau, W)), dtype=torch.uint8, device="cuda")
    wsb.fill_(0xFF)
    tw.twell_ffn_bwd_hybrid_compact(shape, x, WgT, bg, WuT, Wd, dY, c, tau, l1[0], l1[1], dX, dW[0], dW[1], dW[2],
                                    dbg, nD, wsb)
    torch.cuda.synchronize()
    return {"y": y.cpu().numpy(), "dX": dX.cpu().numpy(), "dWgT": dW[0].cpu().numpy(), "dWuT": dW[1].cpu().numpy(),
            "dWd": dW[2].cpu().numpy(), "dbg": dbg.cpu().numpy(), "nD": int(nD.item()), "h": h_host,
            "ovf": c.ovf.cpu().numpy().astype(bool)}


def _check(w, got, tau, W, l1c=0.0, bias=True):
    tol = TOL[w.cfg.dtype]
    ref = O.ffn_dense_bwd(w.x, w.WgT, w.bg if bias else None, w.WuT, w.Wd, w.dY, l1=l1c)
    cnt = got["h"]["cnt"]
    ovf = (cnt > W).any(axis=1)
    np.testing.assert_array_equal(got["ovf"], ovf)
    dense = (cnt.sum(axis=1) > tau) | ovf
    log(f"   dense rows {got['nD']} of {w.T} ({int(ovf.sum())} overflow W={W})")
    assert got["nD"] == int(dense.sum()), (got["nD"], int(dense.sum()))
    for k, r in (("y", ref["fwd"]["y"]), ("dX", ref["dX"])):
        e = rel_fro(got[k], r)
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert e <= tol, (k, e)
        for name, sel in (("dense rows", dense), ("sparse rows", ~dense)):
            if sel.any():
                assert rel_fro(got[k][sel], r[sel]) <= tol, (k, name)
    for k in ("dWgT", "dWuT", "dWd", "dbg"):
        e = rel_fro(got[k], ref[k])
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert np.isfinite(got[k]).all(), k
        assert e <= tol, (k, e)
    return ovf


CASES = [
    ("hybrid", dict(T=520, d=256, f=1280), 2),
    ("hybrid", dict(T=333, d=128, f=640), 4),
    ("hybrid", dict(T=200, d=128, f=640), 64),
    ("hybrid", dict(T=130, d=128, f=640), 1),
    ("tiny_f32", dict(grad=True), 3),
]


@pytest.mark.parametrize("direct", [False, True], ids=["compacted", "direct"])
@pytest.mark.parametrize("name,kw,W", CASES, ids=["520-W2", "333-W4", "200-W64", "130-W1", "tiny_f32-W3"])
def test_bwd_compact(torch, tw, name, kw, W, direct):
    w = make_workload(name, **kw)
    log(f"[bwd compact] {name} T={w.T} d={w.d} f={w.f} tau={w.tau} W={W} direct={direct}")
    got = _run_compact_train(torch, tw, w, w.tau, W, direct=direct)
    ovf = _check(w, got, w.tau, W)
    if W == 64:
        assert not ovf.any()
    if W in (2, 4):
        assert ovf.any() and not ovf.all()


@pytest.mark.parametrize("direct", [False, True], ids=["compacted", "direct"])
def test_bwd_compact_l1_and_no_bias(torch, tw, direct):
    w = make_workload("hybrid", T=260, d=128, f=640)
    lam = 3e-3
    log(f"[bwd compact] l1 lambda={lam} mean, no bias, direct={direct}")
    got = _run_compact_train(torch, tw, w, w.tau, 3, l1=(lam, True), bias=False, direct=direct)
    _check(w, got, w.tau, 3, l1c=O.l1_coefficient(lam, w.T, True), bias=False)


@pytest.mark.parametrize("direct", [False, True], ids=["compacted", "direct"])
def test_bwd_compact_empty(torch, tw, direct):
    w = make_workload("hybrid", T=0, d=128, f=640)
    log(f"[bwd compact] T=0, direct={direct}")
    got = _run_compact_train(torch, tw, w, w.tau, 4, direct=direct)
    assert got["nD"] == 0
    for k in ("dWgT", "dWuT", "dWd", "dbg"):
        assert np.all(got[k] == 0), k


def test_bwd_compact_full_size_sampled(torch, tw):
    """The hybrid training workload at full size (T=16384, d=2048, F=5632)
    with the saved state in compact TwELL of capacity 8: the 30%-density rows
    overflow and take the dense branch, every 1% row fits.  Sampled tokens
    (y, dX) and neurons (weight gradients) against the oracle."""
    w = make_workload("hybrid")
    W = 8
    log(f"[bwd compact] full size T={w.T} d={w.d} f={w.f} tau={w.tau} W={W}, compact forward")
    got = _run_compact_train(torch, tw, w, w.tau, W, direct=True)
    cnt = got["h"]["cnt"]
    ovf = (cnt > W).any(axis=1)
    np.testing.assert_array_equal(got["ovf"], ovf)
    dense = (cnt.sum(axis=1) > w.tau) | ovf
    assert got["nD"] == int(dense.sum())
    log(f"   dense rows {got['nD']} ({int(ovf.sum())} overflow)")
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.choice(w.T, 192, replace=False), w.dense_rows[:32],
                                     np.arange(w.T - 16, w.T)]))
    neur = np.sort(rng.choice(w.f, 48, replace=False))
    ref = O.ffn_bwd_sampled(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY, toks, neur)
    for k, g, r in (("y", got["y"][toks], ref["y_rows"]), ("dX", got["dX"][toks], ref["dX_rows"]),
                    ("dWgT", got["dWgT"][neur], ref["dWgT_rows"]), ("dWuT", got["dWuT"][neur], ref["dWuT_rows"]),
                    ("dWd", got["dWd"][neur], ref["dWd_rows"]), ("dbg", got["dbg"][neur], ref["dbg_rows"])):
        e = rel_fro(g, r)
        log(f"   {k} rel-Frobenius {e:.3e} (sampled)")
        assert e <= TOL["bf16"], (k, e)
    for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
        assert np.isfinite(got[k]).all(), k


@pytest.mark.parametrize("name,kw,W", [("hybrid", dict(T=520, d=256, f=1280), 2),
                                       ("hybrid", dict(T=777, d=256, f=1280), 8),
                                       ("tiny_f32", dict(grad=True), 3),
                                       ("0.5b", dict(T=600, d=256, f=1024), 5)],
                         ids=["520-W2", "777-W8", "tiny_f32-W3", "0.5b-W5"])
def test_fwd_compact_saves_compact_of_full(torch, tw, name, kw, W):
    """The compact forward's saved state equals twell_compact of the full
    forward's saved h, byte for byte (counts, masks, clamped widths, overflow
    flags, the first min(width, W) slots of every tile); its y matches the
    oracle on the sparse and dense rows alike."""
    w = make_workload(name, **kw)
    dt = w.cfg.dtype
    in_dt = tw.TWELL_BF16 if dt == "bf16" else tw.TWELL_F32
    x, WgT, bg, WuT, Wd = (to_dev(a, dt) for a in (w.x, w.WgT, w.bg, w.WuT, w.Wd))
    T, d, F = w.T, w.d, w.f
    tau = w.tau if w.tau is not None else 64
    log(f"[fwd compact] {name} T={T} d={d} f={F} tau={tau} W={W}")
    shape = tw.ffn_shape(T, d, F, in_dt, tw.TWELL_F32)
    h = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
    y_full = torch.empty((T, d), dtype=torch.float32, device="cuda")
    wsf = torch.empty(max(1, tw.twell_ffn_fwd_workspace(shape, True)), dtype=torch.uint8, device="cuda")
    tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y_full, h, tau, wsf)
    ref_c = tw.alloc_twell_cmat(T, F, W)
    tw.twell_compact(h, ref_c)
    c = tw.alloc_twell_cmat(T, F, W)
    c.val.fill_(float("nan"))
    c.idx.fill_(0xEE)
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    wsc = torch.empty(max(1, tw.twell_ffn_fwd_compact_workspace(shape, W)), dtype=torch.uint8, device="cuda")
    wsc.fill_(0xFF)
    tw.twell_ffn_fwd_compact(shape, x, WgT, bg, WuT, Wd, y, c, tau, wsc)
    torch.cuda.synchronize()
    got, want = _cmat_to_numpy(c), _cmat_to_numpy(ref_c)
    for k in ("cnt", "width", "mask", "ovf"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    log(f"   overflow rows {int(got['ovf'].sum())} of {T}")
    NR, NT = want["width"].shape
    for i in range(NR):
        for j in range(NT):
            wd = int(want["width"][i, j])
            np.testing.assert_array_equal(got["idx"][i, j, :wd], want["idx"][i, j, :wd], err_msg=f"idx {i},{j}")
            np.testing.assert_array_equal(got["val_bits"][i, j, :wd], want["val_bits"][i, j, :wd],
                                          err_msg=f"val {i},{j}")
    ref = O.ffn_fwd_rows(w.x, w.WgT, w.bg, w.WuT, w.Wd, np.arange(T))
    yc = y.cpu().numpy()
    e = rel_fro(yc, ref["y"])
    log(f"   y rel-Frobenius {e:.3e}")
    assert e <= TOL[dt], e
    dense = (got["cnt"].sum(axis=1) > tau) | got["ovf"]
    for nm, sel in (("dense rows", dense), ("sparse rows", ~dense)):
        if sel.any():
            assert rel_fro(yc[sel], ref["y"][sel]) <= TOL[dt], nm

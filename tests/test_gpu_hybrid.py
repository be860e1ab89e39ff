"""GPU parity of the hybrid sparse/dense training path against the CPU oracle.

twell_ffn_fwd with a dense-row threshold (hybrid forward) and
twell_ffn_bwd_hybrid are compared with the float64 oracle run on the same
rounded inputs: y, dX, dWgT, dWuT, dWd and dbg within relative Frobenius error
1e-3 (bf16 inputs, fp32 accumulation) or 1e-5 (fp32 inputs), globally and on
the sparse and dense row sets separately.  The number of rows the dense branch
took must equal the count of rows of the GPU's own TwELL whose non-zero count
exceeds the threshold (the classification is integer work on a pattern that
is itself checked against the oracle's).  Full-size runs are checked on
sampled tokens (dX, y) and sampled neurons (weight gradients): a token's dX
depends on its own row only, a neuron's weight gradient on its own column of
g, u and dA only.
"""
import numpy as np
import pytest

import oracle as O
from workloads import make_workload, round_bf16

from gpu_util import log, mat_to_numpy, rel_fro, to_dev

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


def run_train(torch, tw, w, tau, with_dbg=True, bias=True, l1=None):
    """Hybrid forward then backward on the GPU; returns host arrays.  l1:
    None, or (lambda, per_token_mean) for the backward with the activation
    penalty."""
    dt = w.cfg.dtype
    in_dt = tw.TWELL_BF16 if dt == "bf16" else tw.TWELL_F32
    x, WgT, WuT, Wd, dY = (to_dev(a, dt) for a in (w.x, w.WgT, w.WuT, w.Wd, w.dY))
    bg = to_dev(w.bg, dt) if bias else None
    T, d, F = w.T, w.d, w.f
    shape = tw.ffn_shape(T, d, F, in_dt, tw.TWELL_F32)
    h = tw.alloc_twell_mat(T, F, tw.TWELL_F32)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    wsf = torch.empty(max(1, tw.twell_ffn_fwd_workspace(shape, True)), dtype=torch.uint8, device="cuda")
    tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, h, tau, wsf)
    dX = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    dW = [torch.full((F, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    dbg = torch.full((F,), float("nan"), dtype=torch.float32, device="cuda") if with_dbg else None
    nD = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    wsb = torch.empty(max(1, tw.twell_ffn_bwd_workspace(shape, tau)), dtype=torch.uint8, device="cuda")
    if l1 is None:
        tw.twell_ffn_bwd_hybrid(shape, x, WgT, bg, WuT, Wd, dY, h, tau, dX, dW[0], dW[1], dW[2], dbg, nD, wsb)
    else:
        tw.twell_ffn_bwd_hybrid_l1(shape, x, WgT, bg, WuT, Wd, dY, h, tau, l1[0], l1[1], dX, dW[0], dW[1], dW[2],
                                   dbg, nD, wsb)
    torch.cuda.synchronize()
    out = {"y": y.cpu().numpy(), "dX": dX.cpu().numpy(), "dWgT": dW[0].cpu().numpy(),
           "dWuT": dW[1].cpu().numpy(), "dWd": dW[2].cpu().numpy(), "nD": int(nD.item()),
           "h": mat_to_numpy(h)}
    if with_dbg:
        out["dbg"] = dbg.cpu().numpy()
    return out


def check_full(w, got, tau, bias=True, l1c=0.0):
    tol = TOL[w.cfg.dtype]
    bg = w.bg if bias else None
    ref = O.ffn_dense_bwd(w.x, w.WgT, bg, w.WuT, w.Wd, w.dY, l1=l1c)
    dense = got["h"]["cnt"].sum(axis=1) > tau
    assert got["nD"] == int(dense.sum()), (got["nD"], int(dense.sum()))
    log(f"   dense rows {got['nD']} of {w.T}")
    for k, r in (("y", ref["fwd"]["y"]), ("dX", ref["dX"])):
        e = rel_fro(got[k], r)
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert e <= tol, (k, e)
        for name, sel in (("dense rows", dense), ("sparse rows", ~dense)):
            if sel.any():
                es = rel_fro(got[k][sel], r[sel])
                assert es <= tol, (k, name, es)
    for k in ("dWgT", "dWuT", "dWd") + (("dbg",) if "dbg" in got else ()):
        e = rel_fro(got[k], ref[k])
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert np.isfinite(got[k]).all(), k
        assert e <= tol, (k, e)


SMALL = [
    ("hybrid", dict(T=520, d=256, f=1280)),
    ("hybrid", dict(T=333, d=128, f=640)),
    ("hybrid", dict(T=300, d=192, f=704)),
    ("0.5b", dict(T=300, d=256, f=1024, grad=True)),
    ("tiny_f32", dict(grad=True)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=["hybrid-520", "hybrid-333", "hybrid-d192-f704", "0.5b-300", "tiny_f32"])
def test_hybrid_small(torch, tw, name, kw):
    w = make_workload(name, **kw)
    log(f"[hybrid] {name} T={w.T} d={w.d} f={w.f} tau={w.tau}")
    got = run_train(torch, tw, w, w.tau)
    check_full(w, got, w.tau)


@pytest.mark.parametrize("tau_kind", ["all_dense", "all_sparse", "zero"])
def test_hybrid_threshold_limits(torch, tw, tau_kind):
    w = make_workload("hybrid", T=200, d=128, f=640)
    tau = {"all_dense": -1, "all_sparse": w.f, "zero": 0}[tau_kind]
    log(f"[hybrid] tau={tau}")
    got = run_train(torch, tw, w, tau)
    if tau_kind == "all_dense":
        assert got["nD"] == w.T
    if tau_kind == "all_sparse":
        assert got["nD"] == 0
    check_full(w, got, tau)


@pytest.mark.parametrize("T,d,f", [(1100, 128, 640), (2200, 128, 640), (2200, 256, 1280)],
                         ids=["1100-d128", "2200-d128", "2200-d256"])
def test_hybrid_all_dense_many_rows(torch, tw, T, d, f):
    """Every row dense with more than 1024 of them: the dense-row branch runs
    in two rounds of half the rows (640 + 460 at T = 1100; 1152 + 1048 at
    T = 2200, where each round's weight gradients run their K loop in two
    chunks of at most 1024 rows), the second adding its weight and bias
    gradients to the first's, on the 64x64 (d = 128) and the 256x256
    (d = 256, F = 1280) tiles."""
    w = make_workload("hybrid", T=T, d=d, f=f)
    log(f"[hybrid] all dense T={w.T} d={w.d} f={w.f}")
    got = run_train(torch, tw, w, -1)
    assert got["nD"] == w.T
    check_full(w, got, -1)


def test_hybrid_no_bias_no_dbg(torch, tw):
    """Without the gate bias about half the gate values are positive; a
    threshold at half the width sends about half the rows to each branch."""
    w = make_workload("hybrid", T=160, d=128, f=640)
    log("[hybrid] no bias, no dbg")
    got = run_train(torch, tw, w, 320, with_dbg=False, bias=False)
    assert 0 < got["nD"] < w.T
    check_full(w, got, 320, bias=False)


@pytest.mark.parametrize("T", [1, 17, 0])
def test_hybrid_ragged(torch, tw, T):
    w = make_workload("hybrid", T=T, d=128, f=640)
    log(f"[hybrid] ragged T={T}")
    got = run_train(torch, tw, w, w.tau)
    if T == 0:
        for k in ("dWgT", "dWuT", "dWd", "dbg"):
            assert not got[k].any(), k            # gradients are written even with no tokens
        assert got["nD"] == 0
        return
    check_full(w, got, w.tau)


def test_hybrid_deterministic(torch, tw):
    w = make_workload("hybrid", T=400, d=256, f=1280)
    log("[hybrid] determinism")
    a = run_train(torch, tw, w, w.tau)
    b = run_train(torch, tw, w, w.tau)
    for k in ("y", "dX", "dWgT", "dWuT", "dWd", "dbg"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_hybrid_full_size_sampled(torch, tw):
    """The hybrid training workload at full size: T=16384, d=2048, F=5632."""
    w = make_workload("hybrid")
    log(f"[hybrid] full size T={w.T} d={w.d} f={w.f} tau={w.tau}")
    got = run_train(torch, tw, w, w.tau)
    dense = got["h"]["cnt"].sum(axis=1) > w.tau
    assert got["nD"] == int(dense.sum())
    log(f"   dense rows {got['nD']} (drawn dense: {len(w.dense_rows)})")
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([rng.choice(w.T, 192, replace=False), w.dense_rows[:32],
                                     np.arange(w.T - 16, w.T)]))
    neur = np.sort(rng.choice(w.f, 48, replace=False))
    ref = O.ffn_bwd_sampled(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY, toks, neur)
    tol = TOL["bf16"]
    for k, g, r in (("y", got["y"][toks], ref["y_rows"]), ("dX", got["dX"][toks], ref["dX_rows"]),
                    ("dWgT", got["dWgT"][neur], ref["dWgT_rows"]), ("dWuT", got["dWuT"][neur], ref["dWuT_rows"]),
                    ("dWd", got["dWd"][neur], ref["dWd_rows"]), ("dbg", got["dbg"][neur], ref["dbg_rows"])):
        e = rel_fro(g, r)
        log(f"   {k} rel-Frobenius {e:.3e} (sampled)")
        assert e <= tol, (k, e)
    for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
        assert np.isfinite(got[k]).all(), k


@pytest.mark.parametrize("name,kw,mean", [("hybrid", dict(T=520, d=256, f=1280), False),
                                          ("hybrid", dict(T=520, d=256, f=1280), True),
                                          ("tiny_f32", dict(grad=True), False)],
                         ids=["hybrid-sum", "hybrid-mean", "tiny_f32-sum"])
def test_hybrid_l1_penalty(torch, tw, name, kw, mean):
    """Backward with the L1 activation penalty on both branches.  The
    coefficient is large enough that leaving the term out would fail the
    tolerance many times over."""
    w = make_workload(name, **kw)
    c = 0.05
    lam = c * w.T if mean else c
    assert O.l1_coefficient(lam, w.T, mean) == pytest.approx(c)
    log(f"[hybrid] L1 {'mean' if mean else 'sum'} lambda={lam} {name} T={w.T} tau={w.tau}")
    ref0 = O.ffn_dense_bwd(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY)
    ref1 = O.ffn_dense_bwd(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY, l1=O.l1_coefficient(lam, w.T, mean))
    for k in ("dX", "dWgT", "dbg"):
        assert rel_fro(ref0[k], ref1[k]) > 20 * TOL[w.cfg.dtype], k          # the term is visible
    got = run_train(torch, tw, w, w.tau, l1=(lam, mean))
    check_full(w, got, w.tau, l1c=O.l1_coefficient(lam, w.T, mean))
    if name == "hybrid":
        assert 0 < got["nD"] < w.T                                             # both branches ran


def test_hybrid_fwd_fp16_overflow_falls_back(torch, tw):
    """a = h*u beyond the fp16 range in the hybrid forward (x and the gate
    bias scaled up, which keeps the sign pattern): the union down-projection
    computes the sparse rows per stored pair in fp32 while the dense rows take
    their own branch; y and every gradient must still match."""
    w = make_workload("hybrid", T=520, d=256, f=1280)
    w.x[:] = round_bf16(np.asarray(w.x, dtype=np.float32) * np.float32(120.0))
    w.bg[:] = round_bf16(np.asarray(w.bg, dtype=np.float32) * np.float32(120.0))
    fwd = O.ffn_dense_fwd(w.x, w.WgT, w.bg, w.WuT, w.Wd)
    sparse = (fwd["h"] > 0).sum(axis=1) <= w.tau
    assert sparse.any() and (~sparse).any()
    assert np.abs(fwd["a"][sparse]).max() > 65504.0                # a sparse row really overflows fp16
    log("[hybrid] fp16 overflow in the forward")
    got = run_train(torch, tw, w, w.tau)
    check_full(w, got, w.tau)


def test_hybrid_fp16_overflow_falls_back(torch, tw):
    """dG or dU beyond the fp16 range (dY scaled up) makes the union dX GEMM
    stand down for the per-pair fp32 kernel; every gradient must still match."""
    w = make_workload("hybrid", T=520, d=256, f=1280)
    w.dY[:] = round_bf16(np.asarray(w.dY, dtype=np.float32) * np.float32(1.0e5))
    ref = O.ffn_dense_bwd(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY)
    dA = np.asarray(w.dY, dtype=np.float64) @ np.asarray(w.Wd, dtype=np.float64).T
    assert np.abs(dA * ref["fwd"]["u"]).max() > 65504.0           # the case really overflows fp16
    log("[hybrid] fp16 overflow in the backward")
    got = run_train(torch, tw, w, w.tau)
    check_full(w, got, w.tau)


def test_hybrid_all_dense_rounds_fp32(torch, tw):
    """fp32 inputs, every row dense, T = 1100: the register-staged dense-row
    kernels in two rounds (the weight and bias gradients of the second added
    to the first's)."""
    w = make_workload("tiny_f32", T=1100, d=128, f=512, grad=True)
    log(f"[hybrid] fp32 all dense T={w.T} d={w.d} f={w.f}")
    got = run_train(torch, tw, w, -1)
    assert got["nD"] == w.T
    check_full(w, got, -1)

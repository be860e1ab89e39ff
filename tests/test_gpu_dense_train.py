"""GPU parity of the library's dense training step (twell_ffn_dense_bwd), the
denominator of the hybrid training speedup, against the float64 oracle.

The baseline keeps h, u, a, dG and dU in bf16 between its GEMMs (the fastest
dense variant).  Each stored intermediate carries one or two bf16 roundings
(relative 2^-9 each, about 1.6e-3 rms for two), and the outputs are sums of
many such terms with independent rounding errors, so their relative Frobenius
error stays near 2e-3; the tests allow 5e-3.  The sparse path's own bound
(1e-3) is not claimed for this baseline.
"""
import numpy as np
import pytest

import oracle as O
from workloads import make_workload

from gpu_util import log, rel_fro, to_dev

pytestmark = pytest.mark.gpu
TOL = 5e-3


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


def run_dense_train(torch, tw, w, bias=True, with_dbg=True):
    x, WgT, WuT, Wd, dY = (to_dev(a, "bf16") for a in (w.x, w.WgT, w.WuT, w.Wd, w.dY))
    bg = to_dev(w.bg, "bf16") if bias else None
    T, d, F = w.T, w.d, w.f
    shape = tw.ffn_shape(T, d, F, tw.TWELL_BF16, tw.TWELL_F32)
    ws = torch.empty(max(1, tw.twell_ffn_dense_bwd_workspace(shape)), dtype=torch.uint8, device="cuda")
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    dX = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    dW = [torch.full((F, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    dbg = torch.full((F,), float("nan"), dtype=torch.float32, device="cuda") if with_dbg else None
    tw.twell_ffn_dense_bwd(shape, x, WgT, bg, WuT, Wd, dY, y, dX, dW[0], dW[1], dW[2], dbg, ws)
    torch.cuda.synchronize()
    out = {"y": y.cpu().numpy(), "dX": dX.cpu().numpy(), "dWgT": dW[0].cpu().numpy(),
           "dWuT": dW[1].cpu().numpy(), "dWd": dW[2].cpu().numpy()}
    if with_dbg:
        out["dbg"] = dbg.cpu().numpy()
    return out


@pytest.mark.parametrize("name,kw", [("hybrid", dict(T=512, d=256, f=1280)),
                                     ("hybrid", dict(T=320, d=512, f=768)),
                                     ("0.5b", dict(T=256, d=256, f=1024, grad=True))],
                         ids=["hybrid-512", "hybrid-320", "0.5b-256"])
def test_dense_train_matches_oracle(torch, tw, name, kw):
    w = make_workload(name, **kw)
    log(f"[dense train] {name} T={w.T} d={w.d} f={w.f}")
    got = run_dense_train(torch, tw, w)
    ref = O.ffn_dense_bwd(w.x, w.WgT, w.bg, w.WuT, w.Wd, w.dY)
    for k, r in (("y", ref["fwd"]["y"]), ("dX", ref["dX"]), ("dWgT", ref["dWgT"]), ("dWuT", ref["dWuT"]),
                 ("dWd", ref["dWd"]), ("dbg", ref["dbg"])):
        assert np.isfinite(got[k]).all(), k
        e = rel_fro(got[k], r)
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert e <= TOL, (k, e)


def test_dense_train_no_bias_no_dbg(torch, tw):
    w = make_workload("hybrid", T=256, d=256, f=768)
    got = run_dense_train(torch, tw, w, bias=False, with_dbg=False)
    ref = O.ffn_dense_bwd(w.x, w.WgT, None, w.WuT, w.Wd, w.dY)
    for k in ("dX", "dWgT", "dWuT", "dWd"):
        e = rel_fro(got[k], ref[k])
        log(f"   {k} rel-Frobenius {e:.3e}")
        assert e <= TOL, (k, e)


def test_dense_train_no_tokens(torch, tw):
    w = make_workload("hybrid", T=0, d=256, f=512)
    got = run_dense_train(torch, tw, w)
    for k in ("dWgT", "dWuT", "dWd", "dbg"):
        assert not got[k].any(), k

"""GPU parity of the non-gated ReLU FFN, y = ReLU(x.W1 + b1).W2, against the
CPU oracle: zero pattern equal to the oracle's except where |g| < 1e-4, y
within relative Frobenius error 1e-3 (bf16 inputs, fp32 accumulation) or 1e-5
(fp32 inputs); the dense baseline (bf16 act) within 5e-3.  The workloads'
gate weights and bias serve as W1 and b1, their down weights as W2.
"""
import numpy as np
import pytest

import oracle as O
from workloads import make_workload, round_bf16

from gpu_util import log, mat_to_numpy, masks_from_positive, rel_fro, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-3, "f32": 1e-5}
BAND = 1e-4


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


def run_relu(torch, tw, w, out_dt="f32", saved=True, dense=False):
    dt = w.cfg.dtype
    in_dt = tw.TWELL_BF16 if dt == "bf16" else tw.TWELL_F32
    od = tw.TWELL_BF16 if out_dt == "bf16" else tw.TWELL_F32
    x, W1T, b1, W2 = (to_dev(a, dt) for a in (w.x, w.WgT, w.bg, w.Wd))
    shape = tw.ffn_shape(w.T, w.d, w.f, in_dt, od)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16 if out_dt == "bf16" else torch.float32, device="cuda")
    m = None
    if dense:
        ws = torch.empty(max(1, tw.twell_relu_ffn_dense_fwd_workspace(shape)), dtype=torch.uint8, device="cuda")
        tw.twell_relu_ffn_dense_fwd(shape, x, W1T, b1, W2, y, ws)
    else:
        ws = torch.empty(max(1, tw.twell_relu_ffn_fwd_workspace(shape)), dtype=torch.uint8, device="cuda")
        m = tw.alloc_twell_mat(w.T, w.f, tw.TWELL_F32) if saved else None
        tw.twell_relu_ffn_fwd(shape, x, W1T, b1, W2, y, m, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), m


def check_relu(w, y, m, rows=None, out_dt="f32", tol=None):
    rows = np.arange(w.T) if rows is None else np.asarray(rows)
    ref = O.relu_ffn_dense_fwd(np.asarray(w.x)[rows], w.WgT, w.bg, w.Wd)
    tol = TOL[w.cfg.dtype] if tol is None else tol
    y_ref = ref["y"]
    if out_dt == "bf16":
        y_ref = round_bf16(y_ref.astype(np.float32)).astype(np.float64)
        tol = max(tol, 2 ** -8)
    err = rel_fro(y[rows], y_ref)
    log(f"   y rel-Frobenius error {err:.3e} (tol {tol:g}) over {len(rows)} rows")
    assert err <= tol, err
    if m is None:
        return
    got = mat_to_numpy(m)
    g = ref["g"]
    diff = got["mask"][rows] ^ masks_from_positive(g > 0)
    for t, j in zip(*np.nonzero(diff)):
        v = int(diff[t, j])
        while v:
            c = (v & -v).bit_length() - 1
            v &= v - 1
            assert abs(g[t, j * 64 + c]) < BAND, (rows[t], j * 64 + c, g[t, j * 64 + c])


SMALL = [
    ("tiny_f32", dict()),
    ("0.5b", dict(T=333, d=256, f=1024)),
    ("2b", dict(T=777, d=384, f=1536)),
    ("1.5b", dict(T=513, d=320, f=640)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] + "-" + str(s[1].get("T", "")) for s in SMALL])
def test_relu_ffn_small(torch, tw, name, kw):
    w = make_workload(name, **kw)
    log(f"[relu] {name} T={w.T} d={w.d} f={w.f} {w.cfg.dtype}")
    y, m = run_relu(torch, tw, w)
    check_relu(w, y, m)
    y2, _ = run_relu(torch, tw, w, saved=False)
    np.testing.assert_array_equal(y2, y)


@pytest.mark.parametrize("T", [1, 17, 129, 0])
def test_relu_ffn_ragged(torch, tw, T):
    w = make_workload("0.5b", T=T, d=128, f=256)
    log(f"[relu] ragged T={T}")
    y, m = run_relu(torch, tw, w)
    if T == 0:
        assert y.shape == (0, 128)
        return
    check_relu(w, y, m)


def test_relu_ffn_bf16_output(torch, tw):
    w = make_workload("0.5b", T=200, d=256, f=1024)
    y, m = run_relu(torch, tw, w, out_dt="bf16")
    check_relu(w, y, m, out_dt="bf16")


def test_relu_ffn_fp16_overflow_falls_back(torch, tw):
    """h beyond the fp16 range (inputs and bias scaled up) takes the per-pair
    fp32 path; y must still match the oracle."""
    w = make_workload("0.5b", T=300, d=256, f=1024)
    w.x[:] = round_bf16(w.x * np.float32(2.0e4))
    w.bg[:] = round_bf16(w.bg * np.float32(2.0e4))
    ref = O.relu_ffn_dense_fwd(w.x, w.WgT, w.bg, w.Wd)
    assert ref["h"].max() > 65504.0
    log("[relu] fp16 overflow fallback")
    y, m = run_relu(torch, tw, w)
    check_relu(w, y, m)


def test_relu_ffn_full_size_sampled(torch, tw):
    w = make_workload("1.5b")
    log(f"[relu] full size 1.5b T={w.T}")
    y, m = run_relu(torch, tw, w)
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(w.T, size=512, replace=False),
                                     np.arange(w.T - 40, w.T)]))
    check_relu(w, y, m, rows=rows)


@pytest.mark.parametrize("name,kw", [("0.5b", dict(T=333, d=256, f=1024)), ("2b", dict(T=600, d=384, f=1536))])
def test_relu_ffn_dense_baseline(torch, tw, name, kw):
    w = make_workload(name, **kw)
    log(f"[relu dense] {name} T={w.T}")
    y, _ = run_relu(torch, tw, w, dense=True)
    check_relu(w, y, None, tol=5e-3)


def run_relu_bounded(torch, tw, w, W, U):
    x, W1T, b1, W2 = (to_dev(a, "bf16") for a in (w.x, w.WgT, w.bg, w.Wd))
    shape = tw.ffn_shape(w.T, w.d, w.f, tw.TWELL_BF16, tw.TWELL_F32)
    nbytes = tw.twell_relu_ffn_fwd_bounded_workspace(shape, W, U)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tw.twell_relu_ffn_fwd_bounded(shape, x, W1T, b1, W2, y, W, U, ws, n_over_blocks=cnt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(cnt.item())


@pytest.mark.parametrize("W,U,kind", [(64, 1024, "fits"), (4, 1024, "tile"), (64, 64, "union")])
def test_relu_ffn_bounded(torch, tw, W, U, kind):
    """The capacity-bounded non-gated layer: with capacities every block fits,
    y equals twell_relu_ffn_fwd's bit for bit; over the tile capacity h comes
    from a GEMM of x with the union's W1T rows; over the union capacity the
    blocks go per pair.  y against the oracle in every case."""
    w = make_workload("0.5b", T=600, d=256, f=1024)
    g = w.x.astype(np.float64) @ w.WgT.astype(np.float64).T + w.bg.astype(np.float64)
    pos = g > 0
    tilemax = [int(pos[b:b + 128].reshape(-1, w.f // 64, 64).sum(axis=2).max()) for b in range(0, w.T, 128)]
    unions = [int(pos[b:b + 128].any(axis=0).sum()) for b in range(0, w.T, 128)]
    log(f"[relu bounded] {kind}: W={W} U={U}, max tile counts {tilemax}, unions {unions}")
    y, n_over = run_relu_bounded(torch, tw, w, W, U)
    if kind == "fits":
        assert n_over == 0
        y_full, _ = run_relu(torch, tw, w, saved=False)
        assert np.array_equal(y, y_full)
    elif kind == "tile":
        assert n_over >= sum(t >= 6 for t in tilemax)
    else:
        assert n_over == sum(u > U for u in unions) and n_over == len(unions)
    check_relu(w, y, None)

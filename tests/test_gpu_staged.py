"""GPU parity of the three staged forward calls (twell_gate_pack,
twell_sparse_up, twell_sparse_down), each against the CPU oracle:

* twell_gate_pack: zero pattern equal to the oracle's outside the 1e-4 band of
  the pre-activation, counts equal to the mask popcounts, widths and padding
  slots as the format defines them, stored values within the tolerance;
* twell_sparse_up: a = h * u at every stored slot within the tolerance of the
  oracle's a at the same (t, n) (slots of the pattern the GPU stored);
* twell_sparse_down: y from those a values within the tolerance of the
  oracle's y; chained, the three calls reproduce the layer.
Tolerances: relative Frobenius 1e-3 for bf16 inputs (fp32 accumulation),
1e-5 for fp32 inputs.
"""
import numpy as np
import pytest

import oracle as O
from workloads import make_workload

from gpu_util import log, mat_to_numpy, rel_fro, to_dev
from test_gpu_fwd import check_fwd, TOL, _bits

pytestmark = pytest.mark.gpu


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


CASES = [("tiny_f32", dict()), ("0.5b", dict(T=333, d=256, f=1024)), ("2b", dict(T=600, d=384, f=1536)),
         ("0.5b", dict(T=40, d=128, f=512))]


@pytest.mark.parametrize("name,kw", CASES, ids=["tiny_f32", "bf16-T333", "bf16-T600", "bf16-T40"])
def test_staged_forward(torch, tw, name, kw):
    w = make_workload(name, **kw)
    dt = w.cfg.dtype
    in_dt = tw.TWELL_BF16 if dt == "bf16" else tw.TWELL_F32
    log(f"[staged] {name} T={w.T} d={w.d} f={w.f} {dt}")
    x, WgT, bg, WuT, Wd = (to_dev(a, dt) for a in (w.x, w.WgT, w.bg, w.WuT, w.Wd))
    shape = tw.ffn_shape(w.T, w.d, w.f, in_dt, tw.TWELL_F32)
    h = tw.alloc_twell_mat(w.T, w.f, tw.TWELL_F32)
    tw.twell_gate_pack(shape, x, WgT, bg, h)
    torch.cuda.synchronize()
    hv0 = h.val.clone()
    aval = torch.zeros_like(h.val)
    tw.twell_sparse_up(shape, x, WuT, h, aval)
    y = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
    tw.twell_sparse_down(shape, aval, Wd, h, y)
    torch.cuda.synchronize()
    assert torch.equal(hv0.view(torch.int32), h.val.view(torch.int32))   # the pattern's values are not written

    # gate + pack, and the chained layer output
    check_fwd(w, y.cpu().numpy(), h)

    # a at every stored slot against the oracle's a at the same (t, n)
    ref = O.ffn_fwd_rows(w.x, w.WgT, w.bg, w.WuT, w.Wd, np.arange(w.T))
    got = mat_to_numpy(h)
    av = aval.cpu().numpy()
    a_gpu, a_ref = [], []
    for t in range(w.T):
        i, r = divmod(t, 16)
        for j in range(got["mask"].shape[1]):
            for s, c in enumerate(_bits(int(got["mask"][t, j]))):
                a_gpu.append(av[i, j, s, r])
                a_ref.append(ref["h"][t, j * 64 + c] * ref["u"][t, j * 64 + c])
    e = rel_fro(np.array(a_gpu), np.array(a_ref))
    log(f"   a at {len(a_ref)} stored slots: rel-Frobenius {e:.3e}")
    assert e <= TOL[dt]

    # down alone, fed the oracle's a at the GPU's slots: y within tolerance
    a_exact = np.zeros_like(av)
    k = 0
    for t in range(w.T):
        i, r = divmod(t, 16)
        for j in range(got["mask"].shape[1]):
            for s, c in enumerate(_bits(int(got["mask"][t, j]))):
                a_exact[i, j, s, r] = a_ref[k]
                k += 1
    y2 = torch.empty_like(y)
    tw.twell_sparse_down(shape, torch.from_numpy(a_exact.astype(np.float32)).cuda(), Wd, h, y2)
    torch.cuda.synchronize()
    e2 = rel_fro(y2.cpu().numpy(), ref["y"])
    log(f"   down-projection of the oracle's a: rel-Frobenius {e2:.3e}")
    assert e2 <= TOL[dt]


def test_staged_up_in_place(torch, tw):
    """aval may be h's own value array: a overwrites h slot by slot."""
    w = make_workload("0.5b", T=100, d=128, f=256)
    x, WgT, bg, WuT, Wd = (to_dev(a, "bf16") for a in (w.x, w.WgT, w.bg, w.WuT, w.Wd))
    shape = tw.ffn_shape(w.T, w.d, w.f, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.alloc_twell_mat(w.T, w.f, tw.TWELL_F32)
    tw.twell_gate_pack(shape, x, WgT, bg, h)
    aval = torch.zeros_like(h.val)
    tw.twell_sparse_up(shape, x, WuT, h, aval)
    tw.twell_sparse_up(shape, x, WuT, h, h.val)
    torch.cuda.synchronize()
    m = h.mask.cpu().numpy().view(np.uint64)
    cnt = h.cnt.cpu().numpy()
    a1, a2 = aval.cpu().numpy(), h.val.cpu().numpy()
    for t in range(w.T):
        i, r = divmod(t, 16)
        for j in range(m.shape[1]):
            n = int(cnt[t, j])
            np.testing.assert_array_equal(a1[i, j, :n, r], a2[i, j, :n, r])

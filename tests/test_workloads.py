"""Checks of the seeded synthetic workloads: shapes, dtype rounding, realised
gate density against the target, dead neurons, hybrid rows."""
import math

import numpy as np
import pytest

from workloads import CONFIGS, make_workload, round_bf16


def test_round_bf16_ties_and_exactness():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0], dtype=np.float32)
    r = round_bf16(a)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    np.testing.assert_array_equal(r, np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, -0.0], np.float32))
    assert (round_bf16(r) == r).all()


def test_deterministic():
    a = make_workload("0.5b", T=64, d=128, f=256)
    b = make_workload("0.5b", T=64, d=128, f=256)
    for k in ("x", "WgT", "bg", "WuT", "Wd"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))


@pytest.mark.parametrize("name", ["tiny_f32", "0.5b", "1.5b", "2b", "hybrid"])
def test_density_and_dead(name):
    cfg = CONFIGS[name]
    T = 4096 if name != "tiny_f32" else cfg.T
    d = min(cfg.d, 512)
    f = min(cfg.f, 2048)
    w = make_workload(name, T=T, d=d, f=f)
    if cfg.dtype == "bf16":
        for k in ("x", "WgT", "bg", "WuT", "Wd"):
            arr = getattr(w, k)
            np.testing.assert_array_equal(round_bf16(arr), arr)
    g = w.x.astype(np.float64) @ w.WgT.astype(np.float64).T + w.bg.astype(np.float64)
    act = g > 0
    assert not act[:, w.dead].any(), "dead neurons must never fire"
    if name == "hybrid":
        base = np.ones(T, bool)
        base[w.dense_rows] = False
        rho_base = act[base].mean()
        rho_dense = act[w.dense_rows].mean()
        assert abs(rho_base - 0.01) < 0.002, rho_base
        assert abs(rho_dense - 0.30) < 0.03, rho_dense
        assert w.tau == math.floor(0.10 * f)
        assert w.dY is not None and w.dY.shape == (T, d)
        return
    target = cfg.density
    rho = act.mean()
    n = act.size
    # 4-sigma band of a binomial proportion, widened for neuron-level correlation
    tol = 4 * math.sqrt(target * (1 - target) / n) + 0.1 * target
    assert abs(rho - target) < tol, (rho, target)
    # per-neuron realised rates follow the requested probabilities
    hot = np.argsort(-w.p)[:8]
    assert np.allclose(act[:, hot].mean(axis=0), w.p[hot], atol=0.05)


def test_decode_pass_shares_weights():
    full = make_workload("2b", T=32, d=256, f=512)
    dec = make_workload("2b", d=256, f=512, decode=True)
    assert dec.T == 64
    np.testing.assert_array_equal(full.WgT, dec.WgT)
    np.testing.assert_array_equal(full.bg, dec.bg)
    assert not np.array_equal(full.x[:32], dec.x[:32])

"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against a hand-derived worked example, a closed
form, an identity of the mathematics, brute-force enumeration, or central
finite differences, chosen so that a plausible mistake (a dropped bias, ReLU on
the wrong branch, a transposed weight, a wrong slot order, a wrong sign in the
gradient) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- worked example

def test_worked_example_forward_and_pack():
    ex = _load("worked_example_T2_d2_f4.json")
    arr = {k: np.array(ex[k], dtype=np.float64) for k in
           ("x", "WgT", "bg", "WuT", "Wd", "dY", "g", "h", "u", "a", "y")}
    fw = O.ffn_dense_fwd(arr["x"], arr["WgT"], arr["bg"], arr["WuT"], arr["Wd"])
    for k in ("g", "h", "u", "a", "y"):
        np.testing.assert_array_equal(fw[k], arr[k], err_msg=k)
    sp = O.ffn_sparse_fwd(arr["x"], arr["WgT"], arr["bg"], arr["WuT"], arr["Wd"], R=2, C=2)
    np.testing.assert_array_equal(sp["y"], arr["y"])
    loops = O.ffn_sparse_fwd_loops(arr["x"], arr["WgT"], arr["bg"], arr["WuT"], arr["Wd"], R=2, C=2)
    np.testing.assert_array_equal(loops, arr["y"])

    m = O.twell_pack(fw["g"], R=2, C=2)
    np.testing.assert_array_equal(m.cnt, ex["twell_cnt"])
    np.testing.assert_array_equal(m.width, ex["twell_width"])
    for j, key in enumerate(("tile0", "tile1")):
        w = int(m.width[0, j])
        np.testing.assert_array_equal(m.val[0, j, :w, :], ex["twell_val_slot_row"][key])
        np.testing.assert_array_equal(m.idx[0, j, :w, :], ex["twell_idx_slot_row"][key])


def test_worked_example_backward_and_hybrid():
    ex = _load("worked_example_T2_d2_f4.json")
    a = {k: np.array(ex[k], dtype=np.float64) for k in ("x", "WgT", "bg", "WuT", "Wd", "dY")}
    bw = O.ffn_dense_bwd(a["x"], a["WgT"], a["bg"], a["WuT"], a["Wd"], a["dY"])
    for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
        np.testing.assert_array_equal(bw[k], np.array(ex[k], dtype=np.float64), err_msg=k)
    for tau in (-1, 0, 1, 2, 3, 4):
        for fn in (O.hybrid_fwd_bwd, O.hybrid_fwd_bwd_loops):
            hy = fn(a["x"], a["WgT"], a["bg"], a["WuT"], a["Wd"], a["dY"], tau, R=2, C=2)
            np.testing.assert_array_equal(hy["nnz_row"], ex["nnz_row"])
            np.testing.assert_array_equal(hy["dense"], np.array(ex["nnz_row"]) > tau)
            np.testing.assert_array_equal(hy["y"], np.array(ex["y"], dtype=np.float64))
            for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
                np.testing.assert_array_equal(hy[k], np.array(ex[k], dtype=np.float64),
                                              err_msg=f"{fn.__name__} tau={tau} {k}")


# ---------------------------------------------------------------- closed forms

def test_identity_weights_closed_form():
    """Wg = Wu = Wd = I, b = 0: y_i = x_i^2 where x_i > 0, else 0."""
    rng = np.random.default_rng(1)
    d = 8
    x = rng.standard_normal((5, d))
    x[0, 3] = 0.0
    I = np.eye(d)
    y = O.ffn_dense_fwd(x, I, None, I, I)["y"]
    np.testing.assert_array_equal(y, np.where(x > 0, x * x, 0.0))
    ys = O.ffn_sparse_fwd(x, I, None, I, I, R=2, C=4)["y"]
    np.testing.assert_array_equal(ys, y)


def test_bias_only_gate_is_linear():
    """Wg = 0: the gate is the constant ReLU(b), so y is linear in x with the
    matrix WuT^T diag(ReLU(b)) Wd (assembled here column by column from unit
    inputs, not from the oracle's formula)."""
    rng = np.random.default_rng(2)
    T, d, f = 6, 5, 7
    WuT, Wd = rng.standard_normal((f, d)), rng.standard_normal((f, d))
    b = rng.standard_normal(f)
    x = rng.standard_normal((T, d))
    y = O.ffn_dense_fwd(x, np.zeros((f, d)), b, WuT, Wd)["y"]
    M = np.zeros((d, d))
    for k in range(d):
        e = np.zeros((1, d))
        e[0, k] = 1.0
        M[k] = O.ffn_dense_fwd(e, np.zeros((f, d)), b, WuT, Wd)["y"][0]
    np.testing.assert_allclose(y, x @ M, rtol=1e-12, atol=1e-12)
    # and the map uses only neurons with b > 0
    keep = b > 0
    M2 = WuT[keep].T @ (b[keep, None] * Wd[keep])
    np.testing.assert_allclose(M, M2, rtol=1e-12, atol=1e-12)


def test_odd_even_decomposition():
    """With b = 0: y(x) + y(-x) = ((x.Wg) * (x.Wu)).Wd and
    y(x) - y(-x) = (|x.Wg| * (x.Wu)).Wd.  A gate applied to the wrong factor,
    or a missing ReLU, breaks one of the two."""
    rng = np.random.default_rng(3)
    T, d, f = 9, 6, 11
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    yp = O.ffn_dense_fwd(x, WgT, None, WuT, Wd)["y"]
    ym = O.ffn_dense_fwd(-x, WgT, None, WuT, Wd)["y"]
    G = np.einsum("tk,nk->tn", x, WgT)
    U = np.einsum("tk,nk->tn", x, WuT)
    np.testing.assert_allclose(yp + ym, np.einsum("tn,nc->tc", G * U, Wd), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(yp - ym, np.einsum("tn,nc->tc", np.abs(G) * U, Wd), rtol=1e-10, atol=1e-10)


def test_permutation_equivariance():
    rng = np.random.default_rng(4)
    T, d, f = 7, 6, 13
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    b = rng.standard_normal(f)
    y = O.ffn_dense_fwd(x, WgT, b, WuT, Wd)["y"]
    pn = rng.permutation(f)
    pt = rng.permutation(T)
    y2 = O.ffn_dense_fwd(x[pt], WgT[pn], b[pn], WuT[pn], Wd[pn])["y"]
    np.testing.assert_allclose(y2, y[pt], rtol=1e-12, atol=1e-12)


def test_single_active_neuron_rank_one():
    """Exactly one neuron fires: y_t = h * u * Wd[n*] (integers, exact)."""
    x = np.array([[1.0, 2.0, 3.0]])
    WgT = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, -1.0]])
    b = np.array([-5.0, 1.0, 0.0])          # g = [-4, 3, -3]: only neuron 1
    WuT = np.array([[9.0, 9, 9], [1.0, 1, 1], [7.0, 7, 7]])   # u1 = 6
    Wd = np.array([[100.0, 100, 100], [1.0, -2, 4], [100.0, 100, 100]])
    y = O.ffn_dense_fwd(x, WgT, b, WuT, Wd)["y"]
    np.testing.assert_array_equal(y, [[18.0, -36.0, 72.0]])


# ---------------------------------------------------------------- TwELL pack

def _adversarial_G(rng, T, F):
    G = rng.standard_normal((T, F)).astype(np.float32)
    G[rng.random((T, F)) < 0.5] *= -1
    G[0, :] = -0.0                      # all -0 row
    G[1, :] = np.abs(G[1, :]) + 1       # all-positive row
    G[2, ::3] = 0.0
    G[3, 5] = np.float32(1e-45)         # positive denormal: kept
    G[3, 6] = np.float32(-1e-45)        # negative denormal: dropped
    G[4, 7] = np.nan                    # NaN is not > 0: dropped
    return G


@pytest.mark.parametrize("T,F,R,C", [(37, 130, 16, 64), (16, 64, 16, 64), (5, 9, 2, 4), (33, 200, 4, 8)])
def test_pack_invariants(T, F, R, C):
    rng = np.random.default_rng(T * 1000 + F)
    G = _adversarial_G(rng, T, F)
    m = O.twell_pack(G, R, C)
    # unpack(pack(G)) == ReLU(G), bit for bit (+0.0 everywhere else)
    H = O.twell_unpack(m)
    ref = np.where(G > 0, G, np.float32(0.0))
    np.testing.assert_array_equal(H.view(np.uint32), ref.view(np.uint32))
    # counts
    assert m.cnt.sum() == np.count_nonzero(G > 0)
    assert (m.cnt <= C).all()
    NR = -(-T // R)
    cnt_pad = np.zeros((NR * R, m.NT), dtype=np.int64)
    cnt_pad[:T] = m.cnt
    np.testing.assert_array_equal(m.width, cnt_pad.reshape(NR, R, m.NT).max(axis=1))
    # slots strictly ascending in column, padding is (+0.0, 0)
    for t in range(T):
        i, r = divmod(t, R)
        for j in range(m.NT):
            c = int(m.cnt[t, j])
            cols = m.idx[i, j, :c, r].astype(int)
            assert (np.diff(cols) > 0).all()
            w = int(m.width[i, j])
            assert (m.val[i, j, c:w, r].view(np.uint32) == 0).all()
            assert (m.idx[i, j, c:w, r] == 0).all()
    # explicit loops agree exactly
    m2 = O.twell_pack_loops(G, R, C)
    for k in ("cnt", "width", "idx"):
        np.testing.assert_array_equal(getattr(m, k), getattr(m2, k))
    np.testing.assert_array_equal(m.val.view(np.uint32), m2.val.view(np.uint32))


def test_pack_bruteforce_all_sign_patterns():
    """Every one of the 2^8 sign patterns of a 1 x 8 tile: the packed columns
    are the set bits of the pattern, lowest first (enumerated bit by bit)."""
    C = 8
    pats = np.arange(256)
    G = np.where(((pats[:, None] >> np.arange(C)[None, :]) & 1) == 1,
                 np.arange(1, C + 1, dtype=np.float64)[None, :] * 0.5, -1.0)
    m = O.twell_pack(G, R=1, C=C)
    for p in range(256):
        bits = [c for c in range(C) if (p >> c) & 1]
        assert m.cnt[p, 0] == len(bits) == bin(p).count("1")
        assert m.width[p, 0] == len(bits)
        assert list(m.idx[p, 0, : len(bits), 0]) == bits
        assert list(m.val[p, 0, : len(bits), 0]) == [0.5 * (c + 1) for c in bits]


def test_entries_sorted_and_complete():
    rng = np.random.default_rng(7)
    G = rng.standard_normal((21, 70))
    m = O.twell_pack(G, R=4, C=16)
    t, n, v = O.twell_entries(m)
    tt, nn = np.nonzero(G > 0)
    np.testing.assert_array_equal(t, tt)
    np.testing.assert_array_equal(n, nn)
    np.testing.assert_array_equal(v, G[tt, nn])


# ---------------------------------------------------------------- sparse == dense

def test_sparse_loops_equal_dense_loops_exactly():
    """Skipped terms are exact zeros, so with ascending sums the sparse result
    equals the dense one bit for bit."""
    rng = np.random.default_rng(8)
    T, d, f = 5, 6, 12
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    b = rng.standard_normal(f) - 0.5
    yd = O.ffn_dense_fwd_loops(x, WgT, b, WuT, Wd)
    ys = O.ffn_sparse_fwd_loops(x, WgT, b, WuT, Wd, R=2, C=4)
    np.testing.assert_array_equal(ys, yd)
    yv = O.ffn_sparse_fwd(x, WgT, b, WuT, Wd, R=2, C=4)["y"]
    np.testing.assert_allclose(yv, yd, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O.ffn_dense_fwd(x, WgT, b, WuT, Wd)["y"], yd, rtol=1e-13, atol=1e-13)


def test_sparse_degenerate_cases():
    rng = np.random.default_rng(9)
    T, d, f = 33, 16, 130
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    # nothing fires: y = 0 and the pack is empty
    sp = O.ffn_sparse_fwd(x, WgT, np.full(f, -1e6), WuT, Wd)
    assert sp["twell"].nnz == 0 and not sp["y"].any()
    # everything fires: y = ((x.Wg + b) * (x.Wu)).Wd
    b = np.full(f, 1e6)
    sp = O.ffn_sparse_fwd(x, WgT, b, WuT, Wd)
    assert sp["twell"].nnz == T * f
    G = x @ WgT.T + b
    np.testing.assert_allclose(sp["y"], (G * (x @ WuT.T)) @ Wd, rtol=1e-12)
    # empty batch
    sp = O.ffn_sparse_fwd(x[:0], WgT, None, WuT, Wd)
    assert sp["y"].shape == (0, d)


# ---------------------------------------------------------------- gradient

def _fd_inputs(seed, T=4, d=8, f=16):
    rng = np.random.default_rng(seed)
    while True:
        x = rng.standard_normal((T, d))
        WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
        b = rng.standard_normal(f)
        g = x @ WgT.T + b
        if np.abs(g).min() > 1e-2:          # away from the ReLU kink
            return x, WgT, b, WuT, Wd, rng.standard_normal((T, d))


@pytest.mark.parametrize("seed", [10, 11])
def test_backward_central_differences(seed):
    x, WgT, b, WuT, Wd, dY = _fd_inputs(seed)

    def L(x_, WgT_, b_, WuT_, Wd_):
        return float((O.ffn_dense_fwd(x_, WgT_, b_, WuT_, Wd_)["y"] * dY).sum())

    bw = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, dY)
    args = [x, WgT, b, WuT, Wd]
    names = ["dX", "dWgT", "dbg", "dWuT", "dWd"]
    eps = 1e-6
    for ai, name in enumerate(names):
        num = np.zeros_like(args[ai])
        it = np.nditer(args[ai], flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            p = [a.copy() for a in args]
            q = [a.copy() for a in args]
            p[ai][mi] += eps
            q[ai][mi] -= eps
            num[mi] = (L(*p) - L(*q)) / (2 * eps)
        err = np.abs(num - bw[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


def test_hybrid_limits_and_branch_agreement():
    """tau = -1 (all rows dense) and tau = f (all rows sparse) both give the
    dense gradient; so does every threshold in between."""
    rng = np.random.default_rng(12)
    T, d, f = 40, 16, 130
    x = rng.standard_normal((T, d))
    x[::7] *= 4.0                      # some rows far denser than others
    WgT, WuT, Wd = (rng.standard_normal((f, d)) / 4 for _ in range(3))
    b = rng.standard_normal(f) - 1.0
    dY = rng.standard_normal((T, d))
    ref = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, dY)
    nnz = (x @ WgT.T + b > 0).sum(axis=1)
    for tau in (-1, f, int(np.median(nnz))):
        hy = O.hybrid_fwd_bwd(x, WgT, b, WuT, Wd, dY, tau, R=16, C=64)
        assert hy["dense"].sum() == (nnz > tau).sum()
        np.testing.assert_allclose(hy["y"], ref["fwd"]["y"], rtol=1e-12, atol=1e-12)
        for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
            np.testing.assert_allclose(hy[k], ref[k], rtol=1e-12, atol=1e-12, err_msg=f"{tau} {k}")


def test_hybrid_loops_agree_on_tiny():
    rng = np.random.default_rng(13)
    T, d, f = 6, 4, 10
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    b = rng.standard_normal(f)
    dY = rng.standard_normal((T, d))
    a = O.hybrid_fwd_bwd(x, WgT, b, WuT, Wd, dY, 4, R=2, C=4)
    c = O.hybrid_fwd_bwd_loops(x, WgT, b, WuT, Wd, dY, 4, R=2, C=4)
    for k in ("y", "dX", "dWgT", "dWuT", "dWd", "dbg"):
        np.testing.assert_allclose(a[k], c[k], rtol=1e-12, atol=1e-12)


def test_sampled_backward_matches_full():
    rng = np.random.default_rng(14)
    T, d, f = 50, 12, 70
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    b = rng.standard_normal(f)
    dY = rng.standard_normal((T, d))
    full = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, dY)
    tr = np.array([0, 7, 49])
    nr = np.array([3, 69, 10])
    s = O.ffn_bwd_sampled(x, WgT, b, WuT, Wd, dY, tr, nr)
    np.testing.assert_allclose(s["dX_rows"], full["dX"][tr], rtol=1e-12)
    np.testing.assert_allclose(s["y_rows"], full["fwd"]["y"][tr], rtol=1e-12)
    for k in ("dWgT", "dWuT", "dWd"):
        np.testing.assert_allclose(s[k + "_rows"], full[k][nr], rtol=1e-12)
    np.testing.assert_allclose(s["dbg_rows"], full["dbg"][nr], rtol=1e-12)


def test_relu_exact_positive_zero():
    """ReLU gives +0.0 (bit pattern 0) for -0.0, 0.0, negatives and NaN."""
    g = np.array([-0.0, 0.0, -3.0, np.nan, 2.5, -np.inf, np.inf])
    h = O.relu(g)
    np.testing.assert_array_equal(h.view(np.uint64),
                                  np.array([0.0, 0.0, 0.0, 0.0, 2.5, 0.0, np.inf]).view(np.uint64))


# ------------------------------------------------------------------ L1 activation penalty

@pytest.mark.parametrize("seed", [20, 21])
def test_l1_backward_central_differences(seed):
    """With the penalty c * sum(h) added to L, every gradient matches central
    differences of the penalised loss (h computed here from its definition)."""
    x, WgT, b, WuT, Wd, dY = _fd_inputs(seed)
    c = 0.37

    def L(x_, WgT_, b_, WuT_, Wd_):
        g = x_ @ WgT_.T + b_[None, :]
        pen = c * np.maximum(g, 0.0).sum()
        return float((O.ffn_dense_fwd(x_, WgT_, b_, WuT_, Wd_)["y"] * dY).sum()) + pen

    bw = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, dY, l1=c)
    args = [x, WgT, b, WuT, Wd]
    eps = 1e-6
    for ai, name in enumerate(["dX", "dWgT", "dbg", "dWuT", "dWd"]):
        num = np.zeros_like(args[ai])
        it = np.nditer(args[ai], flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            p = [a.copy() for a in args]
            q = [a.copy() for a in args]
            p[ai][mi] += eps
            q[ai][mi] -= eps
            num[mi] = (L(*p) - L(*q)) / (2 * eps)
        err = np.abs(num - bw[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


def test_l1_alone_closed_form():
    """With dY = 0 only the penalty remains: dG is c on the active pairs, so
    dX = c * (active-count-weighted rows of WgT), dWgT[n] = c * sum of the x rows
    that activate n, dbg[n] = c * (tokens activating n), dWuT = dWd = 0."""
    rng = np.random.default_rng(22)
    T, d, f = 9, 5, 13
    x = rng.standard_normal((T, d))
    WgT, WuT, Wd = (rng.standard_normal((f, d)) for _ in range(3))
    b = rng.standard_normal(f)
    c = 1.5
    bw = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, np.zeros((T, d)), l1=c)
    active = [[n for n in range(f) if float(np.dot(x[t], WgT[n]) + b[n]) > 0] for t in range(T)]
    for t in range(T):
        want = sum((c * WgT[n] for n in active[t]), np.zeros(d))
        np.testing.assert_allclose(bw["dX"][t], want, rtol=1e-12, atol=1e-12)
    for n in range(f):
        toks = [t for t in range(T) if n in active[t]]
        np.testing.assert_allclose(bw["dWgT"][n], sum((c * x[t] for t in toks), np.zeros(d)), rtol=1e-12, atol=1e-12)
        assert bw["dbg"][n] == pytest.approx(c * len(toks), rel=1e-12)
    assert not bw["dWuT"].any() and not bw["dWd"].any()


def test_l1_hybrid_branch_agreement_and_loops():
    rng = np.random.default_rng(23)
    T, d, f = 40, 16, 130
    x = rng.standard_normal((T, d))
    x[::7] *= 4.0
    WgT, WuT, Wd = (rng.standard_normal((f, d)) / 4 for _ in range(3))
    b = rng.standard_normal(f) - 1.0
    dY = rng.standard_normal((T, d))
    c = O.l1_coefficient(0.8, T, per_token_mean=True)
    assert c == pytest.approx(0.8 / T)
    assert O.l1_coefficient(0.8, T, per_token_mean=False) == 0.8
    ref = O.ffn_dense_bwd(x, WgT, b, WuT, Wd, dY, l1=c)
    nnz = (x @ WgT.T + b > 0).sum(axis=1)
    for tau in (-1, f, int(np.median(nnz))):
        hy = O.hybrid_fwd_bwd(x, WgT, b, WuT, Wd, dY, tau, R=16, C=64, l1=c)
        for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
            np.testing.assert_allclose(hy[k], ref[k], rtol=1e-12, atol=1e-12, err_msg=f"{tau} {k}")
    a = O.hybrid_fwd_bwd(x[:6, :4], WgT[:10, :4], b[:10], WuT[:10, :4], Wd[:10, :4], dY[:6, :4], 4, R=2, C=4, l1=0.3)
    l = O.hybrid_fwd_bwd_loops(x[:6, :4], WgT[:10, :4], b[:10], WuT[:10, :4], Wd[:10, :4], dY[:6, :4], 4, R=2, C=4,
                               l1=0.3)
    for k in ("dX", "dWgT", "dWuT", "dWd", "dbg"):
        np.testing.assert_allclose(a[k], l[k], rtol=1e-12, atol=1e-12)
    s = O.ffn_bwd_sampled(x, WgT, b, WuT, Wd, dY, np.array([0, 39]), np.array([5, 129]), l1=c)
    np.testing.assert_allclose(s["dX_rows"], ref["dX"][[0, 39]], rtol=1e-12)
    np.testing.assert_allclose(s["dbg_rows"], ref["dbg"][[5, 129]], rtol=1e-12)


# ------------------------------------------------------------------ non-gated ReLU FFN

def test_relu_ffn_is_gated_ffn_with_unit_up_projection():
    """A gated FFN whose up-projection is 1 for every token (a constant input
    column and an up weight that reads only it) is the non-gated ReLU FFN."""
    rng = np.random.default_rng(30)
    T, d, f = 37, 12, 150
    x = rng.standard_normal((T, d))
    W1T, W2 = rng.standard_normal((f, d)), rng.standard_normal((f, d))
    b1 = rng.standard_normal(f) - 0.5
    xa = np.concatenate([x, np.ones((T, 1))], axis=1)
    W1a = np.concatenate([W1T, np.zeros((f, 1))], axis=1)
    WuA = np.concatenate([np.zeros((f, d)), np.ones((f, 1))], axis=1)
    W2a = W2                                                     # the output has d columns either way
    gated = O.ffn_dense_fwd(xa, W1a, b1, WuA, W2a)
    plain = O.relu_ffn_dense_fwd(x, W1T, b1, W2)
    np.testing.assert_allclose(gated["u"], 1.0, rtol=0, atol=0)
    np.testing.assert_allclose(plain["y"], gated["y"], rtol=1e-12, atol=1e-12)
    sparse = O.relu_ffn_sparse_fwd(x, W1T, b1, W2)
    np.testing.assert_allclose(sparse["y"], gated["y"], rtol=1e-12, atol=1e-12)


def test_relu_ffn_bias_only_closed_form():
    """With W1 = 0 the hidden layer is ReLU(b1) for every token, so every
    output row is sum_n max(b1[n], 0) * W2[n]."""
    rng = np.random.default_rng(31)
    T, d, f = 5, 7, 70
    W2 = rng.standard_normal((f, d))
    b1 = rng.standard_normal(f)
    want = sum(max(b1[n], 0.0) * W2[n] for n in range(f))
    for fn in (O.relu_ffn_dense_fwd, O.relu_ffn_sparse_fwd):
        y = fn(rng.standard_normal((T, d)), np.zeros((f, d)), b1, W2)["y"]
        for t in range(T):
            np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ compact TwELL

def test_compact_full_capacity_is_identity():
    rng = np.random.default_rng(40)
    G = rng.standard_normal((37, 200)) - 0.5
    m = O.twell_pack(G, R=16, C=64)
    c = O.twell_compact(m, 64)
    assert not c.ovf.any()
    e = O.twell_expand(c)
    np.testing.assert_array_equal(e.width, m.width)
    np.testing.assert_array_equal(e.val.view(np.uint64), m.val.view(np.uint64))
    np.testing.assert_array_equal(e.idx, m.idx)


@pytest.mark.parametrize("W", [2, 4, 8])
def test_compact_keeps_every_row_that_fits(W):
    """Rows flagged exactly when some tile holds more than W non-zeros; every
    other row's entries survive compact -> expand bit-exactly; the value
    arrays shrink by W / C."""
    rng = np.random.default_rng(41 + W)
    T, F = 70, 320
    G = rng.standard_normal((T, F)) - 2.3          # about 1% positive
    G[::9] += 2.2                                  # some much denser rows
    m = O.twell_pack(G, R=16, C=64)
    c = O.twell_compact(m, W)
    counts = np.array([[int((G[t, j * 64:(j + 1) * 64] > 0).sum()) for j in range(F // 64)] for t in range(T)])
    np.testing.assert_array_equal(c.ovf, (counts > W).any(axis=1))
    assert c.ovf.any() and not c.ovf.all()
    assert c.val.nbytes * 64 == m.val.nbytes * W
    keep = np.nonzero(~c.ovf)[0]
    t0, n0, v0 = O.twell_entries(m, rows=keep)
    t1, n1, v1 = O.twell_entries(O.twell_expand(c), rows=keep)
    np.testing.assert_array_equal(t0, t1)
    np.testing.assert_array_equal(n0, n1)
    np.testing.assert_array_equal(v0.view(np.uint64), v1.view(np.uint64))
    for t in keep:
        for j in range(F // 64):
            row = [G[t, j * 64 + c_] for c_ in range(64) if G[t, j * 64 + c_] > 0]
            assert len(row) == counts[t, j] <= W


def test_compact_bruteforce_overflow_flags():
    """All 2^8 sign patterns of a 1x8 tile (C = 8), capacity 3: the row is
    flagged iff more than 3 entries are positive."""
    for bits in range(256):
        G = np.array([[1.0 if (bits >> k) & 1 else -1.0 for k in range(8)]])
        c = O.twell_compact(O.twell_pack(G, R=1, C=8), 3)
        assert bool(c.ovf[0]) == (bin(bits).count("1") > 3)

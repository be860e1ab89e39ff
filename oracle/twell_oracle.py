"""CPU oracle of the TwELL ReLU-gated FFN (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  It shares no code,
tables or helpers with the HIP library.

Sources (the pages; cited by page and section):
  [IN]  intellectnews.ru article on Sakana AI + NVIDIA TwELL ("...twell-uskorenie-
        llm-do-20-procentov"), sections "Формат TwELL вместо классической
        sparse-упаковки" (TwELL format), "Слитые CUDA-ядра для инференса и гибрид
        для обучения" (fused inference kernel, hybrid training format),
        "Минимальные изменения в рецепте обучения" (ReLU gate), "Ограничения и
        открытые вопросы" (gated FFN).
  [GE]  gate.com/es post 20977915 (Sakana AI + NVIDIA, TwELL), paragraphs 1-4.
  [GI]  gate.com/id post 20978418 (same story in Indonesian), paragraphs 1-7.

What the method computes, as read from the pages:
  * The FFN is gated and its gate activation is ReLU, which makes the inactive
    gate values exact zeros ([IN] recipe and limitations sections).  With a gate
    bias b (a synthetic knob that sets the activation density):
        g = x.Wg + b,  h = ReLU(g),  u = x.Wu,  a = h * u,  y = a.Wd.
    Weights are stored neuron-major: WgT, WuT, Wd are [f, d], so neuron n's
    gate, up and down vectors are the rows WgT[n], WuT[n], Wd[n].
  * Only exact zeros are skipped, so the sparse result equals the dense one
    ([GE] paragraph 1 states no loss of precision).
  * TwELL ([IN] TwELL section; [GE] paragraph 3; [GI] paragraphs 4-5) is an
    ELLPACK layout applied per tile: the gate matrix is cut into R x C tiles and
    inside each tile every row keeps only its non-zero values, compacted, with
    their column index inside the tile; the tile is padded to the widest row
    (its ELL width).  Reading taken here: entries > 0 strictly are kept, in
    ascending column order; per (row, tile) a count; per tile a width; values
    and indices stored tile-major, slot-major, row-minor ([NR][NT][C][R]);
    padding slots below the width hold value +0.0 and index 0.
  * Training uses a hybrid format ([IN] fused/hybrid section): rows with few
    non-zeros take the sparse path, rows with many take a dense branch.
    Reading: a row is dense iff its non-zero count exceeds an integer
    threshold tau (ties go sparse).  Both branches compute the same gradient.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "relu", "ffn_dense_fwd", "ffn_dense_fwd_loops", "ffn_dense_bwd", "l1_coefficient",
    "TwellMat", "twell_pack", "twell_pack_loops", "twell_unpack", "twell_entries",
    "ffn_sparse_fwd", "ffn_sparse_fwd_loops", "classify_rows",
    "hybrid_fwd_bwd", "hybrid_fwd_bwd_loops", "ffn_fwd_rows", "ffn_bwd_sampled",
    "relu_ffn_dense_fwd", "relu_ffn_sparse_fwd",
    "CompactTwell", "twell_compact", "twell_expand",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def relu(g: np.ndarray) -> np.ndarray:
    """ReLU with exact zeros: v where v > 0, else +0.0 (also for -0.0 and NaN).

    [IN] "Минимальные изменения в рецепте обучения": the gate activation is
    ReLU so that inactive neurons give exact zeros.
    """
    g = np.asarray(g)
    return np.where(g > 0, g, np.zeros((), dtype=g.dtype))


# --------------------------------------------------------------------------
# Dense definition of the gated FFN and of its gradient
# --------------------------------------------------------------------------

def ffn_dense_fwd(x, WgT, bg, WuT, Wd) -> dict:
    """Dense ReLU-gated FFN in float64: y = (ReLU(x.Wg + b) * (x.Wu)) . Wd.

    [IN] recipe section (ReLU gate) and limitations section (gated FFN).
    Returns the intermediates g, h, u, a and the output y.
    """
    x, WgT, WuT, Wd = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd)
    g = x @ WgT.T
    if bg is not None:
        g = g + _f64(bg)[None, :]
    h = relu(g)
    u = x @ WuT.T
    a = h * u
    y = a @ Wd
    return {"g": g, "h": h, "u": u, "a": a, "y": y}


def ffn_dense_fwd_loops(x, WgT, bg, WuT, Wd) -> np.ndarray:
    """Same definition with scalar loops; every sum runs in ascending index order.
    For tiny inputs only."""
    x, WgT, WuT, Wd = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd)
    T, d = x.shape
    f = WgT.shape[0]
    b = np.zeros(f) if bg is None else _f64(bg)
    y = np.zeros((T, d))
    for t in range(T):
        a = np.zeros(f)
        for n in range(f):
            g = 0.0
            u = 0.0
            for k in range(d):
                g += x[t, k] * WgT[n, k]
                u += x[t, k] * WuT[n, k]
            g += b[n]
            h = g if g > 0 else 0.0
            a[n] = h * u
        for c in range(d):
            s = 0.0
            for n in range(f):
                s += a[n] * Wd[n, c]
            y[t, c] = s
    return y


def l1_coefficient(lam: float, T: int, per_token_mean: bool) -> float:
    """Coefficient c of the activation penalty's gradient, dL1/dg = c * 1[g > 0].

    [IN] section "Минимальные изменения в рецепте обучения" adds a small L1
    penalty on the activations (weight about 2e-5) to the training loss but
    does not say how it is normalised.  Readings: L1 = lam * sum_{t,n} h[t,n]
    (sum), or lam / T times that sum (mean over tokens).  h >= 0, so |h| = h
    and its derivative is 1[g > 0].
    """
    return float(lam) / T if (per_token_mean and T > 0) else float(lam)


def ffn_dense_bwd(x, WgT, bg, WuT, Wd, dY, l1: float = 0.0) -> dict:
    """Gradient of L = <y, dY> + l1 * sum(h) for the dense gated FFN (float64).

    ReLU'(g) is taken as 1[g > 0] (0 at g = 0); l1 is the coefficient c of
    l1_coefficient.  Returns dX, dWgT, dWuT, dWd, dbg and the forward dict
    under "fwd".
    """
    fw = ffn_dense_fwd(x, WgT, bg, WuT, Wd)
    x, WgT, WuT, Wd, dY = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd), _f64(dY)
    dA = dY @ Wd.T
    dG = np.where(fw["g"] > 0, dA * fw["u"] + l1, 0.0)
    dU = dA * fw["h"]
    return {
        "dX": dG @ WgT + dU @ WuT,
        "dWgT": dG.T @ x,
        "dWuT": dU.T @ x,
        "dWd": fw["a"].T @ dY,
        "dbg": dG.sum(axis=0),
        "fwd": fw,
    }


# --------------------------------------------------------------------------
# TwELL: tile-wise ELLPACK
# --------------------------------------------------------------------------

@dataclass
class TwellMat:
    """A [T, F] matrix of ReLU outputs in TwELL form.

    cnt   [T, NT]        non-zeros of row t inside column tile j
    width [NR, NT]       ELL width of tile (i, j): max cnt over its R rows
    val   [NR, NT, C, R] value of slot s of row r of tile (i, j)
    idx   [NR, NT, C, R] column of that value inside the tile (0..C-1)
    Slots s < cnt hold the row's non-zeros in ascending column order; slots
    cnt <= s < width hold value +0.0 and index 0; slots >= width are
    unspecified (zero here).  Row positions past T in the last row tile count
    as empty rows.
    """
    T: int
    F: int
    R: int
    C: int
    cnt: np.ndarray
    width: np.ndarray
    val: np.ndarray
    idx: np.ndarray

    @property
    def NR(self) -> int:
        return -(-self.T // self.R)

    @property
    def NT(self) -> int:
        return -(-self.F // self.C)

    @property
    def nnz(self) -> int:
        return int(self.cnt.sum())


def twell_pack(G: np.ndarray, R: int = 16, C: int = 64) -> TwellMat:
    """Pack the strictly positive entries of G into TwELL (vectorized numpy).

    [IN] TwELL section; [GE] paragraph 3; [GI] paragraphs 4-5: compaction of the
    useful values happens per tile.  Values are bit copies of G (same dtype).
    """
    G = np.asarray(G)
    T, F = G.shape
    NR, NT = -(-T // R), -(-F // C)
    Gp = np.zeros((NR * R, NT * C), dtype=G.dtype)
    Gp[:T, :F] = G
    act = (Gp > 0).reshape(NR, R, NT, C)
    cnt_full = act.sum(axis=3)                       # [NR, R, NT]
    width = cnt_full.max(axis=1).astype(np.int64)    # [NR, NT]
    cnt = cnt_full.reshape(NR * R, NT)[:T].astype(np.int64)
    slot = np.cumsum(act, axis=3) - 1                # slot of each active entry
    val = np.zeros((NR, NT, C, R), dtype=G.dtype)
    idx = np.zeros((NR, NT, C, R), dtype=np.uint8)
    i, r, j, c = np.nonzero(act)
    s = slot[i, r, j, c]
    val[i, j, s, r] = Gp.reshape(NR, R, NT, C)[i, r, j, c]
    idx[i, j, s, r] = c
    return TwellMat(T, F, R, C, cnt, width, val, idx)


def twell_pack_loops(G: np.ndarray, R: int = 16, C: int = 64) -> TwellMat:
    """TwELL pack with explicit loops over rows, tiles and columns (tiny inputs)."""
    G = np.asarray(G)
    T, F = G.shape
    NR, NT = -(-T // R), -(-F // C)
    cnt = np.zeros((T, NT), dtype=np.int64)
    width = np.zeros((NR, NT), dtype=np.int64)
    val = np.zeros((NR, NT, C, R), dtype=G.dtype)
    idx = np.zeros((NR, NT, C, R), dtype=np.uint8)
    for t in range(T):
        i, r = divmod(t, R)
        for j in range(NT):
            slot = 0
            for c in range(C):
                col = j * C + c
                if col < F and G[t, col] > 0:
                    val[i, j, slot, r] = G[t, col]
                    idx[i, j, slot, r] = c
                    slot += 1
            cnt[t, j] = slot
            width[i, j] = max(width[i, j], slot)
    return TwellMat(T, F, R, C, cnt, width, val, idx)


def twell_unpack(m: TwellMat) -> np.ndarray:
    """Dense [T, F] matrix from TwELL: the value of slot s < cnt goes to column
    j*C + idx; every other entry is +0.0."""
    H = np.zeros((m.T, m.F), dtype=m.val.dtype)
    for t in range(m.T):
        i, r = divmod(t, m.R)
        for j in range(m.NT):
            for s in range(int(m.cnt[t, j])):
                H[t, j * m.C + int(m.idx[i, j, s, r])] = m.val[i, j, s, r]
    return H


def twell_entries(m: TwellMat, rows: Optional[np.ndarray] = None):
    """All stored non-zeros as (t, n, value) arrays, sorted by (t, n)."""
    NR, NT, C, R = m.val.shape
    s_idx = np.arange(C)[None, None, :, None]
    t_of = (np.arange(NR)[:, None, None, None] * R + np.arange(R)[None, None, None, :])
    t_of = np.broadcast_to(t_of, (NR, NT, C, R))
    cnt_full = np.zeros((NR * R, NT), dtype=np.int64)
    cnt_full[: m.T] = m.cnt
    cnt4 = cnt_full.reshape(NR, R, NT).transpose(0, 2, 1)[:, :, None, :]   # [NR,NT,1,R]
    live = s_idx < cnt4
    if rows is not None:
        keep = np.zeros(NR * R, dtype=bool)
        keep[np.asarray(rows)] = True
        live = live & keep[t_of]
    i, j, s, r = np.nonzero(live)
    t = i * R + r
    n = j * C + m.idx[i, j, s, r].astype(np.int64)
    v = m.val[i, j, s, r]
    order = np.lexsort((n, t))
    return t[order], n[order], v[order]


# --------------------------------------------------------------------------
# Sparse forward through TwELL
# --------------------------------------------------------------------------

def ffn_sparse_fwd(x, WgT, bg, WuT, Wd, R: int = 16, C: int = 64,
                   chunk_rows: int = 256) -> dict:
    """Gated FFN that visits only the active neurons of each token (float64).

    [IN] fused-kernel section: the gate result is packed (TwELL) and the up and
    down projections then touch only the active neurons:
        u[t,n] = x_t . WuT[n],  a = h * u,  y_t = sum over active n of a * Wd[n].
    """
    x, WgT, WuT, Wd = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd)
    T, d = x.shape
    g = x @ WgT.T
    if bg is not None:
        g = g + _f64(bg)[None, :]
    m = twell_pack(g, R, C)
    t_all, n_all, h_all = twell_entries(m)
    y = np.zeros((T, d))
    bounds = np.searchsorted(t_all, np.arange(0, T + chunk_rows, chunk_rows))
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi <= lo:
            continue
        t, n, h = t_all[lo:hi], n_all[lo:hi], h_all[lo:hi]
        u = np.einsum("pk,pk->p", x[t], WuT[n])
        a = h * u
        np.add.at(y, t, a[:, None] * Wd[n])
    return {"y": y, "twell": m}


def ffn_sparse_fwd_loops(x, WgT, bg, WuT, Wd, R: int = 16, C: int = 64) -> np.ndarray:
    """Sparse forward with scalar loops, ascending sums (tiny inputs).  Equal to
    ffn_dense_fwd_loops bit for bit: skipped terms are exact zeros."""
    x, WgT, WuT, Wd = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd)
    T, d = x.shape
    f = WgT.shape[0]
    b = np.zeros(f) if bg is None else _f64(bg)
    G = np.zeros((T, f))
    for t in range(T):
        for n in range(f):
            s = 0.0
            for k in range(d):
                s += x[t, k] * WgT[n, k]
            G[t, n] = s + b[n]
    m = twell_pack_loops(G, R, C)
    y = np.zeros((T, d))
    for t in range(T):
        i, r = divmod(t, R)
        for j in range(m.NT):
            for s in range(int(m.cnt[t, j])):
                n = j * C + int(m.idx[i, j, s, r])
                h = m.val[i, j, s, r]
                u = 0.0
                for k in range(d):
                    u += x[t, k] * WuT[n, k]
                a = h * u
                for c in range(d):
                    y[t, c] += a * Wd[n, c]
    return y


# --------------------------------------------------------------------------
# Hybrid training step: row classification, sparse and dense branches
# --------------------------------------------------------------------------

def classify_rows(cnt: np.ndarray, tau: int) -> np.ndarray:
    """Dense-row mask: a row is dense iff its non-zero count exceeds tau.

    [IN] fused/hybrid section: rows with many active values go to the dense
    branch.  Reading: integer threshold, ties go sparse; tau < 0 sends every
    row dense, tau >= F sends every row sparse.
    """
    return np.asarray(cnt).sum(axis=1) > tau


def hybrid_fwd_bwd(x, WgT, bg, WuT, Wd, dY, tau: int, R: int = 16, C: int = 64,
                   chunk_rows: int = 256, l1: float = 0.0) -> dict:
    """Hybrid forward + backward (float64).

    Dense rows run the plain definition on the gathered rows; sparse rows run
    per active pair: u = x_t.WuT[n], a = h*u, y_t += a*Wd[n], da = dY_t.Wd[n],
    dg = da*u + l1 (g > 0 on every stored pair), du = da*h, dX_t += dg*WgT[n] +
    du*WuT[n], dWd[n] += a*dY_t, dWgT[n] += dg*x_t, dWuT[n] += du*x_t,
    dbg[n] += dg.  Weight gradients are the sum of both branches.
    """
    x, WgT, WuT, Wd, dY = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd), _f64(dY)
    T, d = x.shape
    f = WgT.shape[0]
    b = np.zeros(f) if bg is None else _f64(bg)
    g = x @ WgT.T + b[None, :]
    m = twell_pack(g, R, C)
    dense = classify_rows(m.cnt, tau)
    D = np.nonzero(dense)[0]
    S = np.nonzero(~dense)[0]

    y = np.zeros((T, d))
    dX = np.zeros((T, d))
    dWgT = np.zeros((f, d))
    dWuT = np.zeros((f, d))
    dWd = np.zeros((f, d))
    dbg = np.zeros(f)

    if D.size:
        gD = g[D]
        hD = relu(gD)
        uD = x[D] @ WuT.T
        aD = hD * uD
        y[D] = aD @ Wd
        dAD = dY[D] @ Wd.T
        dGD = np.where(gD > 0, dAD * uD + l1, 0.0)
        dUD = dAD * hD
        dX[D] = dGD @ WgT + dUD @ WuT
        dWd += aD.T @ dY[D]
        dWgT += dGD.T @ x[D]
        dWuT += dUD.T @ x[D]
        dbg += dGD.sum(axis=0)

    if S.size:
        t_all, n_all, h_all = twell_entries(m, rows=S)
        bounds = np.searchsorted(t_all, np.arange(0, T + chunk_rows, chunk_rows))
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            if hi <= lo:
                continue
            t, n, h = t_all[lo:hi], n_all[lo:hi], h_all[lo:hi]
            u = np.einsum("pk,pk->p", x[t], WuT[n])
            a = h * u
            da = np.einsum("pk,pk->p", dY[t], Wd[n])
            dg = da * u + l1
            du = da * h
            np.add.at(y, t, a[:, None] * Wd[n])
            np.add.at(dX, t, dg[:, None] * WgT[n] + du[:, None] * WuT[n])
            np.add.at(dWd, n, a[:, None] * dY[t])
            np.add.at(dWgT, n, dg[:, None] * x[t])
            np.add.at(dWuT, n, du[:, None] * x[t])
            np.add.at(dbg, n, dg)

    return {"y": y, "dX": dX, "dWgT": dWgT, "dWuT": dWuT, "dWd": dWd, "dbg": dbg,
            "dense": dense, "nnz_row": m.cnt.sum(axis=1), "twell": m}


def hybrid_fwd_bwd_loops(x, WgT, bg, WuT, Wd, dY, tau: int, R: int = 16,
                         C: int = 64, l1: float = 0.0) -> dict:
    """Hybrid forward + backward with scalar loops (tiny inputs)."""
    x, WgT, WuT, Wd, dY = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd), _f64(dY)
    T, d = x.shape
    f = WgT.shape[0]
    b = np.zeros(f) if bg is None else _f64(bg)
    G = np.zeros((T, f))
    for t in range(T):
        for n in range(f):
            G[t, n] = sum(x[t, k] * WgT[n, k] for k in range(d)) + b[n]
    m = twell_pack_loops(G, R, C)
    nnz_row = m.cnt.sum(axis=1)
    out = {k: np.zeros((T, d)) for k in ("y", "dX")}
    out.update({k: np.zeros((f, d)) for k in ("dWgT", "dWuT", "dWd")})
    out["dbg"] = np.zeros(f)
    for t in range(T):
        if nnz_row[t] > tau:                       # dense branch: every neuron
            pairs = [(n, G[t, n]) for n in range(f)]
        else:                                      # sparse branch: stored pairs
            i, r = divmod(t, R)
            pairs = [(j * C + int(m.idx[i, j, s, r]), float(m.val[i, j, s, r]))
                     for j in range(m.NT) for s in range(int(m.cnt[t, j]))]
        for n, gv in pairs:
            h = gv if gv > 0 else 0.0
            u = sum(x[t, k] * WuT[n, k] for k in range(d))
            a = h * u
            da = sum(dY[t, c] * Wd[n, c] for c in range(d))
            dg = da * u + l1 if gv > 0 else 0.0
            du = da * h
            for c in range(d):
                out["y"][t, c] += a * Wd[n, c]
                out["dX"][t, c] += dg * WgT[n, c] + du * WuT[n, c]
                out["dWd"][n, c] += a * dY[t, c]
                out["dWgT"][n, c] += dg * x[t, c]
                out["dWuT"][n, c] += du * x[t, c]
            out["dbg"][n] += dg
    out["dense"] = nnz_row > tau
    out["nnz_row"] = nnz_row
    return out


# --------------------------------------------------------------------------
# Sampled outputs for full-size parity (rows and neurons are independent)
# --------------------------------------------------------------------------

def ffn_fwd_rows(x, WgT, bg, WuT, Wd, rows) -> dict:
    """Forward of the listed token rows only (each output row depends on its own
    input row alone)."""
    rows = np.asarray(rows)
    return ffn_dense_fwd(np.asarray(x)[rows], WgT, bg, WuT, Wd)


def ffn_bwd_sampled(x, WgT, bg, WuT, Wd, dY, token_rows, neuron_rows, l1: float = 0.0) -> dict:
    """dX on the listed tokens and dWgT/dWuT/dWd/dbg on the listed neurons.

    dX_t needs only token t; the weight gradient of neuron n needs only column n
    of g, u and dA over all tokens.
    """
    x, WgT, WuT, Wd, dY = _f64(x), _f64(WgT), _f64(WuT), _f64(Wd), _f64(dY)
    f = WgT.shape[0]
    b = np.zeros(f) if bg is None else _f64(bg)
    tr = np.asarray(token_rows)
    nr = np.asarray(neuron_rows)
    # token rows
    gt = x[tr] @ WgT.T + b[None, :]
    ut = x[tr] @ WuT.T
    dAt = dY[tr] @ Wd.T
    dGt = np.where(gt > 0, dAt * ut + l1, 0.0)
    dUt = dAt * relu(gt)
    dX_rows = dGt @ WgT + dUt @ WuT
    y_rows = (relu(gt) * ut) @ Wd
    # neuron rows
    gn = x @ WgT[nr].T + b[nr][None, :]
    un = x @ WuT[nr].T
    hn = relu(gn)
    dAn = dY @ Wd[nr].T
    dGn = np.where(gn > 0, dAn * un + l1, 0.0)
    dUn = dAn * hn
    return {
        "y_rows": y_rows, "dX_rows": dX_rows,
        "dWd_rows": (hn * un).T @ dY,
        "dWgT_rows": dGn.T @ x,
        "dWuT_rows": dUn.T @ x,
        "dbg_rows": dGn.sum(axis=0),
    }


# --------------------------------------------------------------------------
# Non-gated ReLU FFN
# --------------------------------------------------------------------------

def relu_ffn_dense_fwd(x, W1T, b1, W2) -> dict:
    """Non-gated ReLU FFN in float64: y = ReLU(x.W1 + b1) . W2.

    [IN] section "Ограничения и открытые вопросы": the method targets gated
    FFNs; a plain ReLU FFN has the same exact zeros in ReLU(x.W1 + b1) but no
    up-projection to skip, so less to gain.  W1T and W2 are [f, d]
    (neuron-major, as for the gated layer).  Returns g, h and y.
    """
    x, W1T, W2 = _f64(x), _f64(W1T), _f64(W2)
    f = W1T.shape[0]
    b = np.zeros(f) if b1 is None else _f64(b1)
    g = x @ W1T.T + b[None, :]
    h = relu(g)
    return {"g": g, "h": h, "y": h @ W2}


def relu_ffn_sparse_fwd(x, W1T, b1, W2, R: int = 16, C: int = 64) -> dict:
    """The same layer through TwELL: pack ReLU(g), then y_t = sum over the
    stored (t, n) of h * W2[n], neurons ascending per token."""
    x, W1T, W2 = _f64(x), _f64(W1T), _f64(W2)
    T, d = x.shape
    f = W1T.shape[0]
    b = np.zeros(f) if b1 is None else _f64(b1)
    g = x @ W1T.T + b[None, :]
    m = twell_pack(g, R, C)
    t, n, h = twell_entries(m)
    y = np.zeros((T, W2.shape[1]))
    for tt in np.unique(t):
        sel = t == tt
        order = np.argsort(n[sel], kind="stable")
        y[tt] = (h[sel][order][:, None] * W2[n[sel][order]]).sum(axis=0)
    return {"y": y, "twell": m}


# --------------------------------------------------------------------------
# Compact TwELL: capacity W < C slots per (row, tile)
# --------------------------------------------------------------------------

@dataclass
class CompactTwell:
    """TwELL with capacity W slots per (row, tile) instead of C.

    [IN] section "Слитые CUDA-ядра для инференса и гибрид для обучения": in
    training, well-sparse rows are kept in a compact sparse matrix and rows
    with many active values go to a dense branch; [GE] paragraph 1 and [GI]
    paragraph 1 report reduced peak memory.  Reading: a fixed capacity W per
    (row, tile), so tile (i, j) sits at a fixed offset (i*NT + j)*W*R and needs
    no offset table; a row with more than W non-zeros in some tile cannot be
    stored whole and is flagged (ovf) for the dense branch.
    cnt [T, NT] true counts; width [NR, NT] = min(full width, W); val, idx
    [NR, NT, W, R] = the first W slots of the full form; ovf [T] bool.
    """
    T: int
    F: int
    R: int
    C: int
    W: int
    cnt: np.ndarray
    width: np.ndarray
    val: np.ndarray
    idx: np.ndarray
    ovf: np.ndarray


def twell_compact(m: TwellMat, W: int) -> CompactTwell:
    """Keep the first W slots of every (row, tile); flag the rows that have
    more than W non-zeros in some tile."""
    assert 1 <= W <= m.C
    ovf = (m.cnt > W).any(axis=1) if m.cnt.size else np.zeros(m.T, dtype=bool)
    return CompactTwell(m.T, m.F, m.R, m.C, W, m.cnt.copy(), np.minimum(m.width, W),
                        m.val[:, :, :W, :].copy(), m.idx[:, :, :W, :].copy(), ovf)


def twell_expand(c: CompactTwell) -> TwellMat:
    """Back to the capacity-C form: the stored slots in place, the others zero.
    Rows flagged in ovf keep their true counts but only W slots per tile."""
    NR, NT = c.width.shape
    val = np.zeros((NR, NT, c.C, c.R), dtype=c.val.dtype)
    idx = np.zeros((NR, NT, c.C, c.R), dtype=c.idx.dtype)
    val[:, :, :c.W, :] = c.val
    idx[:, :, :c.W, :] = c.idx
    return TwellMat(c.T, c.F, c.R, c.C, c.cnt.copy(), c.width.copy(), val, idx)

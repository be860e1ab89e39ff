#!/usr/bin/env python3
"""FFN-layer throughput of the TwELL ReLU-gated FFN on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2b]

One step is one pass of the whole hot path over the workload's token batch,
inputs already resident in HBM:
  forward workloads (0.5b, 1.5b, 2b, tiny_f32): twell_ffn_fwd = gate GEMM +
      bias + ReLU + TwELL pack in the epilogue, then the up- and down-
      projections over the active neurons;
  training workload (hybrid): twell_ffn_fwd with the dense-row threshold, then
      twell_ffn_bwd_hybrid (dX, dWgT, dWuT, dWd, dbg).
The library's own dense MFMA FFN (twell_ffn_dense_fwd) is timed on the same
inputs for the speedup (forward workloads).  Kernel and stage durations come
from HIP events recorded on the stream the kernels run on.  The CPU oracle is
timed on a bounded sample of the same workload.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FFN tokens/s @1 GPU (TwELL vs own dense); % HBM / MFMA roofline"
PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_vector_tflops": 157.3, "hbm_gbs": 8000.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed ones (the GPU clock takes a few hundred ms of work to settle)")
    ap.add_argument("--config", default="2b",
                    help="headline workload: 2b (T=32768, d=2304, F=9216, 0.93%% density) by default")
    ap.add_argument("--decode", action="store_true", help="use the workload's decode-shaped pass")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--no-bounded", action="store_true", help="skip the capacity-bounded forward")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extras", action="store_true", help="skip the short runs of the other workloads")
    ap.add_argument("--cold-iters", type=int, default=5,
                    help="steps timed one by one after a 512 MiB scratch write (cold cache); 0 skips")
    ap.add_argument("--compact-w", type=int, default=8,
                    help="training workloads: also time the step with the saved state in compact TwELL of this "
                         "capacity (twell_compact + twell_ffn_bwd_hybrid_compact); 0 skips it")
    ap.add_argument("--ffn", choices=["gated", "relu"], default="gated",
                    help="relu: the non-gated ReLU FFN y = ReLU(x.W1 + b1).W2 (the workload's gate weights and "
                         "bias as W1, b1, its down weights as W2)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the PMC byte counters)")
    return ap.parse_args()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, budget_s: float, training: bool) -> dict:
    """Time the CPU oracle (float64 numpy, as it stands) on leading token rows
    of the same workload for about budget_s seconds."""
    import oracle
    chunk = 128 if training else 256
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        rows = slice(done, min(done + chunk, w.T))
        if training:
            oracle.hybrid_fwd_bwd(w.x[rows], w.WgT, w.bg, w.WuT, w.Wd, w.dY[rows], w.tau)
        else:
            oracle.ffn_sparse_fwd(w.x[rows], w.WgT, w.bg, w.WuT, w.Wd)
        done = rows.stop
    dt = time.perf_counter() - t0
    what = ("hybrid forward + backward (row classification, dense and sparse branches)" if training
            else "sparse forward (gate GEMM, TwELL pack, per-pair up/down)")
    return {"value": done / dt, "unit": "tokens/s", "cores": blas_threads(), "host_cpu_count": os.cpu_count(),
            "kind": "oracle",
            "sample": f"first {done} of {w.T} token rows, float64 numpy {what}, {dt:.1f} s; cores = the BLAS "
                      f"threads the oracle ran on"}


# tokens per row block of the union up/down GEMMs (the library's row blocks)
UNION_BLOCK = 128

# kernels whose HBM traffic is recorded in profiles/hbm_traffic.json, with the
# source files that define each (a recorded figure is dropped once they change)
TRAFFIC_SOURCES = {
    "gate_gemm_twell_pack": ["twell_gate.hip", "gemm_core.hpp", "common.hpp"],
    "up_projection": ["twell_union.hip", "gemm_core.hpp", "common.hpp"],
    "down_projection": ["twell_union.hip", "gemm_core.hpp", "common.hpp"],
}
# the few-token (decode) path runs its own kernels
TRAFFIC_SOURCES_DECODE = {k: ["twell_decode.hip", "gemm_core.hpp", "common.hpp"]
                          for k in TRAFFIC_SOURCES}


def source_digest(files) -> str:
    import hashlib
    hsh = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "activation_sparse_feedforward_gate_amd", "csrc", f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def load_traffic(config: str) -> dict:
    """HBM bytes per launch from the recorded PMC runs (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-kernel calibration), for kernels unchanged since then."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    out = {}
    sources = TRAFFIC_SOURCES_DECODE if config.endswith("_decode") else TRAFFIC_SOURCES
    for k, files in sources.items():
        r = rec.get("kernels", {}).get(config, {}).get(k)
        if r and r.get("source_digest") == source_digest(files):
            out[k] = r["bytes_per_launch"]
    return out


def copy_calibration(steps: int) -> int:
    """A plain device copy of a known size, for scaling the PMC byte counters."""
    import torch
    n = 1 << 28                                         # 256 Mi floats = 1 GiB read + 1 GiB written
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": steps}))
    return 0


def relu_bench(args) -> int:
    """The non-gated ReLU FFN: whole-layer timing against its own dense
    baseline (no per-kernel events: the entry point records none)."""
    import numpy as np
    import torch

    import activation_sparse_feedforward_gate_amd as tw
    import oracle
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[args.config]
    if cfg.dtype != "bf16" or cfg.tau_frac is not None:
        print(json.dumps({"error": "--ffn relu runs the bf16 inference workloads (0.5b, 1.5b, 2b)"}))
        return 2
    w = make_workload(args.config, decode=args.decode)
    T, d, f = w.T, w.d, w.f
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dt(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)

    x, W1T, b1, W2 = dt(w.x), dt(w.WgT), dt(w.bg), dt(w.Wd)
    shape = tw.ffn_shape(T, d, f, tw.TWELL_BF16, tw.TWELL_F32)
    h = tw.alloc_twell_mat(T, f, tw.TWELL_F32, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, tw.twell_relu_ffn_fwd_workspace(shape)), dtype=torch.uint8, device=dev)
    wsd = torch.empty(max(1, tw.twell_relu_ffn_dense_fwd_workspace(shape)), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    ms = timed(lambda: tw.twell_relu_ffn_fwd(shape, x, W1T, b1, W2, y, h, ws, stream))
    nnz = int(h.cnt.to(torch.int64).sum().item())
    work = 2.0 * T * d * f + 2.0 * nnz * d              # gate GEMM + useful down-projection flops
    achieved = work / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes, densities and neuron-popularity structure of the workload)",
        "config": {"workload": cfg.description + " -- non-gated ReLU FFN (W1 = gate weights, W2 = down weights)",
                   "name": args.config, "ffn": "relu", "T": T, "d_model": d, "d_ff": f,
                   "realised_density": nnz / (T * f), "pass": "fwd"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK["bf16_mfma_tflops"], "unit": "TFLOP/s",
                     "frac": achieved / PEAK["bf16_mfma_tflops"], "traffic": None,
                     "kernel": "whole layer (gate GEMM + pack + union down-projection)"},
    }
    if not args.no_dense:
        dms = timed(lambda: tw.twell_relu_ffn_dense_fwd(shape, x, W1T, b1, W2, y, wsd, stream))
        out["dense_baseline"] = {"tokens_per_s": T / (dms * 1e-3), "ms_per_step": dms,
                                 "what": "dense ReLU FFN, bf16 act"}
        out["speedup_vs_dense"] = dms / ms
        out["workspace_bytes"] = {"twell": int(ws.numel()), "own_dense": int(wsd.numel())}
    caps = None if args.no_bounded else BOUNDED_CAPS.get(args.config)
    if caps and not args.decode:
        Wc, Uc = caps
        bws = tw.twell_relu_ffn_fwd_bounded_workspace(shape, Wc, Uc)
        wsb = torch.empty(bws, dtype=torch.uint8, device=dev)
        yb = torch.empty_like(y)
        nover = torch.zeros((1,), dtype=torch.int32, device=dev)
        bms = timed(lambda: tw.twell_relu_ffn_fwd_bounded(shape, x, W1T, b1, W2, yb, Wc, Uc, wsb, None, stream))
        tw.twell_relu_ffn_fwd_bounded(shape, x, W1T, b1, W2, yb, Wc, Uc, wsb, nover, stream)
        tw.twell_relu_ffn_fwd(shape, x, W1T, b1, W2, y, None, ws, stream)
        torch.cuda.synchronize()
        out["bounded_forward"] = {"tile_cap": Wc, "union_cap": Uc, "ms_per_step": bms, "workspace_bytes": int(bws),
                                  "over_capacity_blocks": int(nover.item()),
                                  "y_equals_full_forward": bool(torch.equal(yb, y))}
        if "dense_baseline" in out:
            out["bounded_forward"]["speedup_vs_dense"] = out["dense_baseline"]["ms_per_step"] / bms
            out["bounded_forward"]["workspace_vs_own_dense"] = bws / max(1, int(wsd.numel()))
    if not args.no_cpu:
        chunk, done, t0 = 256, 0, time.perf_counter()
        while done < T and time.perf_counter() - t0 < args.cpu_seconds:
            rows = slice(done, min(done + chunk, T))
            oracle.relu_ffn_dense_fwd(w.x[rows], w.WgT, w.bg, w.Wd)
            done = rows.stop
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                               "sample": f"first {done} of {T} token rows, float64 numpy dense ReLU FFN, {el:.1f} s"}
    print(json.dumps(out))
    return 0


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def _timed(fn, steps: int, warmup: int, stream, warm_s: float = 0.0) -> float:
    """Mean ms per call of fn over exactly `steps` calls after `warmup` untimed
    ones (and, with warm_s > 0, more untimed calls until warm_s seconds have
    passed), between two events on the launch stream, synchronized on both
    sides."""
    import time
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if warm_s > 0:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
    t0, t1 = _ev(), _ev()
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def cold_cache_ms(fn, iters: int, stream) -> float:
    """Median ms of fn over `iters` calls, each after a 512 MiB scratch write
    that evicts the 256 MB Infinity Cache and every L2, so the call reads its
    inputs from HBM."""
    import numpy as np
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ms = []
    for k in range(iters + 1):
        scratch.fill_(k & 0xff)
        e0, e1 = _ev(), _ev()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        if k:
            ms.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(ms))


def union_sizes(mask: "np.ndarray", T: int, live=None):
    """Union size of every UNION_BLOCK-token row block (live rows only)."""
    import numpy as np
    m = mask.copy()
    if live is not None:
        m[~live] = 0
    ub = UNION_BLOCK
    if T == 0:
        return np.zeros(0, dtype=np.int64)
    pad = (-T) % ub
    mm = np.concatenate([m, np.zeros((pad, m.shape[1]), np.uint64)]) if pad else m
    u = np.bitwise_or.reduce(mm.reshape(-1, ub, m.shape[1]), axis=1)
    return np.unpackbits(u.view(np.uint8), axis=1).sum(axis=1).astype(np.int64)


def measure(args, name: str, decode: bool, steps: int, warmup: int, full: bool, warm_s: float = 0.0) -> dict:
    """Time one workload: the TwELL step, the library's own dense step beside
    it, per-stage HIP events, and (full) the roofline of every forward kernel,
    a cold-cache figure and the workspace bytes of both paths."""
    import numpy as np
    import torch

    import activation_sparse_feedforward_gate_amd as tw
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[name]
    training = cfg.tau_frac is not None
    w = make_workload(name, decode=decode)
    T, d, f = w.T, w.d, w.f
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def dt(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return t.to(torch.bfloat16) if cfg.dtype == "bf16" else t

    x, WgT, bg, WuT, Wd = dt(w.x), dt(w.WgT), dt(w.bg), dt(w.WuT), dt(w.Wd)
    in_dt = tw.TWELL_BF16 if cfg.dtype == "bf16" else tw.TWELL_F32
    shape = tw.ffn_shape(T, d, f, in_dt, tw.TWELL_F32)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    tau = w.tau if training else -1
    ws_fwd_bytes = tw.twell_ffn_fwd_workspace(shape, training)
    wsf = torch.empty(max(1, ws_fwd_bytes), dtype=torch.uint8, device=dev)
    # inference keeps no TwELL for a backward pass: the step passes no saved_h
    # and the TwELL lives in the workspace; training saves h for the backward
    h = tw.alloc_twell_mat(T, f, tw.TWELL_F32, device=dev)
    saved = h if training else None
    if training:
        dY = dt(w.dY)
        dX = torch.empty((T, d), dtype=torch.float32, device=dev)
        dW = [torch.empty((f, d), dtype=torch.float32, device=dev) for _ in range(3)]
        dbg = torch.empty((f,), dtype=torch.float32, device=dev)
        nD = torch.empty((1,), dtype=torch.int32, device=dev)
        ws_bwd_bytes = tw.twell_ffn_bwd_workspace(shape, tau)
        # the forward's workspace is free once it returns: one buffer serves both calls
        if ws_bwd_bytes > ws_fwd_bytes:
            wsf = torch.empty(ws_bwd_bytes, dtype=torch.uint8, device=dev)
        wsb = wsf

    def step(evs=None):
        if evs is None:
            tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, saved, tau, wsf, stream)
        else:
            tw.twell_ffn_fwd_ex(shape, x, WgT, bg, WuT, Wd, y, saved, tau, wsf, evs[:7], stream)
        if training:
            if evs is not None:
                evs[7].record(stream)
            tw.twell_ffn_bwd_hybrid(shape, x, WgT, bg, WuT, Wd, dY, h, tau, dX, dW[0], dW[1], dW[2], dbg, nD, wsb,
                                    stream)
            if evs is not None:
                evs[8].record(stream)

    # timed region: exactly `steps` steps between two events, bracketed by synchronize
    ms_step = _timed(step, steps, warmup, stream, warm_s)

    # per-stage durations from events recorded between the kernel launches
    nst = 9 if training else 7
    recs = [[_ev() for _ in range(nst)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        step(recs[k])
    torch.cuda.synchronize()
    st = np.array([[r[i].elapsed_time(r[i + 1]) for i in range(nst - 1)] for r in recs]).mean(axis=0)
    stages = {"gate_gemm_twell_pack": st[0], "union_lists_wd_fp16": st[1], "up_projection": st[2],
              "down_projection": st[3]}
    if training:
        stages["dense_rows_fwd"] = st[5]
        stages["hybrid_bwd"] = st[7]
    if not training:
        # the TwELL of the step, for its statistics (one more call, untimed)
        tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, h, tau, wsf, stream)
        torch.cuda.synchronize()
    cnt = h.cnt.cpu().numpy().astype(np.int64)
    nnz = int(cnt.sum())
    mask = h.mask.cpu().numpy().view(np.uint64)

    out = {"ms_per_step": ms_step, "tokens_per_s": T / (ms_step * 1e-3),
           "workload": cfg.description + (" (decode pass)" if decode else ""), "name": name,
           "T": T, "d_model": d, "d_ff": f, "realised_density": nnz / max(1, T * f),
           "pass": "fwd+bwd" if training else "fwd",
           "stages_ms": {k: float(v) for k, v in stages.items()}}

    bf = cfg.dtype == "bf16"
    few_tokens = bf and not training and 0 < T <= 256
    live = None
    if training:
        live = cnt.sum(axis=1) <= tau                  # the union GEMMs cover the sparse rows only
        out["dense_rows"] = int((~live).sum())
    if bf and not few_tokens:
        nb = union_sizes(mask, T, live)
        out["mean_union_fraction"] = float(nb.mean() / f) if len(nb) else 0.0
    if few_tokens:
        n_union = int(np.unpackbits(np.bitwise_or.reduce(mask, axis=0).view(np.uint8)).sum())
        out["union_neurons"] = n_union
        out["stage_note"] = ("few-token kernels: gate_gemm_twell_pack is the K-split gate GEMM alone, "
                             "up_projection is the TwELL pack fused with the up-projection, "
                             "union_lists_wd_fp16 is empty (event overhead)")

    # the library's own dense step on the same inputs
    if not args.no_dense and bf:
        if training:
            dws = torch.empty(tw.twell_ffn_dense_bwd_workspace(shape), dtype=torch.uint8, device=dev)
            yd, dXd = torch.empty_like(y), torch.empty_like(dX)
            dWd_ = [torch.empty_like(t) for t in dW]
            dbgd = torch.empty_like(dbg)

            def dense_step():
                tw.twell_ffn_dense_bwd(shape, x, WgT, bg, WuT, Wd, dY, yd, dXd, dWd_[0], dWd_[1], dWd_[2], dbgd,
                                       dws, stream)
            dms = _timed(dense_step, steps, warmup, stream, warm_s)
            out["dense_baseline"] = {"tokens_per_s": T / (dms * 1e-3), "ms_per_step": dms,
                                     "tflops": 18.0 * T * d * f / (dms * 1e-3) / 1e12,
                                     "what": "dense forward + backward, bf16 intermediates"}
            dense_ws = tw.twell_ffn_dense_bwd_workspace(shape)
        else:
            dense_ws = tw.twell_ffn_dense_fwd_workspace(shape)
            dws = torch.empty(max(1, dense_ws), dtype=torch.uint8, device=dev)
            yd = torch.empty_like(y)

            def dense_step():
                tw.twell_ffn_dense_fwd(shape, x, WgT, bg, WuT, Wd, yd, dws, stream)
            dms = _timed(dense_step, steps, warmup, stream, warm_s)
            out["dense_baseline"] = {"tokens_per_s": T / (dms * 1e-3), "ms_per_step": dms,
                                     "tflops": 6.0 * T * d * f / (dms * 1e-3) / 1e12}
            out["dense_vs_sparse_rel_diff"] = (y - yd).norm().item() / max(yd.norm().item(), 1e-30)
        out["speedup_vs_dense"] = dms / ms_step
        # device memory the step needs beyond its inputs and outputs
        twell_ws = (max(ws_fwd_bytes, ws_bwd_bytes) + tw.twell_mat_bytes(T, f)[0]) if training else ws_fwd_bytes
        out["workspace_bytes"] = {"twell": int(twell_ws), "own_dense": int(dense_ws)}

    caps = None if args.no_bounded else BOUNDED_CAPS.get(name)
    if caps and bf and not training and not few_tokens:
        # the capacity-bounded forward on the same inputs: its workspace against
        # the full-capacity one and the own dense path's, and its time
        Wc, Uc = caps
        bws = tw.twell_ffn_fwd_bounded_workspace(shape, Wc, Uc)
        wsb_ = torch.empty(bws, dtype=torch.uint8, device=dev)
        yb = torch.empty_like(y)
        nover = torch.zeros((1,), dtype=torch.int32, device=dev)

        def bounded_step():
            tw.twell_ffn_fwd_bounded(shape, x, WgT, bg, WuT, Wd, yb, Wc, Uc, wsb_, None, stream)
        bms = _timed(bounded_step, steps, warmup, stream, warm_s)
        tw.twell_ffn_fwd_bounded(shape, x, WgT, bg, WuT, Wd, yb, Wc, Uc, wsb_, nover, stream)
        tw.twell_ffn_fwd(shape, x, WgT, bg, WuT, Wd, y, None, tau, wsf, stream)
        torch.cuda.synchronize()
        out["bounded_forward"] = {
            "tile_cap": Wc, "union_cap": Uc, "ms_per_step": bms, "tokens_per_s": T / (bms * 1e-3),
            "workspace_bytes": int(bws), "over_capacity_blocks": int(nover.item()),
            "y_equals_full_forward": bool(torch.equal(yb, y))}
        if "dense_baseline" in out:
            out["bounded_forward"]["speedup_vs_dense"] = out["dense_baseline"]["ms_per_step"] / bms
            out["bounded_forward"]["workspace_vs_own_dense"] = bws / max(1, out["workspace_bytes"]["own_dense"])
        del wsb_
    if training:
        # state a layer keeps between its forward and its backward: TwELL of h
        # (capacity 64, or compact with capacity W), against the own dense
        # step's (h, u) words and a (bf16 [T][F] each; x and the weights are
        # inputs either way)
        out["saved_state_bytes"] = {
            "twell_full": int(tw.twell_mat_bytes(T, f)[0]),
            f"twell_compact_W{args.compact_w or 8}": int(tw.twell_cmat_bytes(T, f, args.compact_w or 8)[0]),
            "own_dense_h_u_a_bf16": int(3 * T * f * 2)}
    if few_tokens and not full and args.cold_iters > 0 and not args.no_dense:
        out["cold_cache_ms_per_step"] = cold_cache_ms(step, args.cold_iters, stream)
        out["dense_baseline"]["cold_cache_ms_per_step"] = cold_cache_ms(dense_step, args.cold_iters, stream)
    if training and args.compact_w > 0:
        # the same step with the state saved between forward and backward in
        # compact TwELL of capacity W: the forward packs the gate output
        # straight into it, the backward reads it in place
        W = args.compact_w
        c = tw.alloc_twell_cmat(T, f, W, device=dev)
        fws = tw.twell_ffn_fwd_compact_workspace(shape, W)
        bws = tw.twell_ffn_bwd_compact_workspace(shape, tau, W)
        # the forward's workspace is free once it returns: one buffer serves both calls
        wsc = torch.empty(max(1, fws, bws), dtype=torch.uint8, device=dev)

        def compact_step():
            tw.twell_ffn_fwd_compact(shape, x, WgT, bg, WuT, Wd, y, c, tau, wsc, stream)
            tw.twell_ffn_bwd_hybrid_compact(shape, x, WgT, bg, WuT, Wd, dY, c, tau, 0.0, False, dX, dW[0], dW[1],
                                            dW[2], dbg, nD, wsc, stream)
        cms = _timed(compact_step, steps, warmup, stream, warm_s)
        saved_c = tw.twell_cmat_bytes(T, f, W)[0]
        out["compact_twell"] = {
            "W": W, "ms_per_step": cms, "tokens_per_s": T / (cms * 1e-3),
            "overflow_rows": int(c.ovf.to(torch.int64).sum().item()), "dense_rows": int(nD.item()),
            "saved_state_bytes": saved_c,
            "full_saved_state_bytes": tw.twell_mat_bytes(T, f)[0],
            "workspace_bytes": {"forward": int(fws), "backward": int(bws), "shared": int(max(fws, bws)),
                                "saved_state": int(saved_c), "peak": int(max(fws, bws) + saved_c)},
        }
        if "dense_baseline" in out:
            out["compact_twell"]["speedup_vs_dense"] = out["dense_baseline"]["ms_per_step"] / cms
            out["compact_twell"]["workspace_vs_own_dense"] = (max(fws, bws) + saved_c) / max(
                1, out["workspace_bytes"]["own_dense"])
        del wsc
    out["_workload"] = w
    if not full:
        return out

    # roofline of each forward kernel: algorithmic work per launch / its duration
    mma_peak = PEAK["bf16_mfma_tflops"] if bf else PEAK["fp32_vector_tflops"]
    gate_flops = 2.0 * T * d * f                       # 2 d F per token
    pair_flops = 2.0 * nnz * d                         # 2 d per stored (token, neuron) pair, each projection
    if training:
        pair_flops = 2.0 * float(cnt[live].sum()) * d  # the sparse rows' pairs
    lines = {
        "gate_gemm_twell_pack": {"bound": "mfma", "work": gate_flops, "ms": st[0]},
        "up_projection": {"bound": "mfma", "work": pair_flops, "ms": st[2]},
        "down_projection": {"bound": "mfma", "work": pair_flops, "ms": st[3]},
    }
    if few_tokens:
        # a few tokens make every phase a pass over weights: HBM-bound, with
        # algorithmic bytes Wg whole (+x), the union's Wu rows (+x), the
        # union's Wd rows (+y written)
        n_union = out["union_neurons"]
        lines["gate_gemm_twell_pack"].update(bound="hbm", work=2.0 * f * d + 2.0 * T * d)
        lines["up_projection"].update(bound="hbm", work=2.0 * n_union * d + 2.0 * T * d)
        lines["down_projection"].update(bound="hbm", work=2.0 * n_union * d + 4.0 * T * d)
    traffic = load_traffic(name + ("_decode" if decode else ""))
    for k, v in lines.items():
        if v["bound"] == "hbm":
            v["achieved"] = v["work"] / (v["ms"] * 1e-3) / 1e9
            v["peak"] = PEAK["hbm_gbs"]
            v["unit"] = "GB/s"
        else:
            v["achieved"] = v["work"] / (v["ms"] * 1e-3) / 1e12
            v["peak"] = mma_peak
            v["unit"] = "TFLOP/s"
        v["frac"] = v["achieved"] / v["peak"]
        v["traffic"] = traffic.get(k)
    if bf and not few_tokens:
        # MFMA work the union GEMMs execute (all union positions of every
        # row block, in whole tiles), beside the useful work above
        up_exec = 2.0 * float((-(-nb // 256) * 256).sum()) * UNION_BLOCK * d
        dn_exec = 2.0 * float((-(-nb // 64) * 64).sum()) * UNION_BLOCK * d
        for k, w_exec in (("up_projection", up_exec), ("down_projection", dn_exec)):
            lines[k]["executed_work"] = w_exec
            lines[k]["executed_tflops"] = w_exec / (lines[k]["ms"] * 1e-3) / 1e12
    dom = max(lines, key=lambda k: lines[k]["ms"])
    roof = {k2: lines[dom][k2] for k2 in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dom
    roof["launch_ms"] = float(lines[dom]["ms"])
    roof["work_per_launch"] = lines[dom]["work"]
    out["roofline"] = roof
    out["stage_roofline"] = {k: {k2: (float(v2) if isinstance(v2, (np.floating, float)) else v2)
                                 for k2, v2 in v.items()} for k, v in lines.items()}

    if args.cold_iters > 0:
        out["cold_cache_ms_per_step"] = cold_cache_ms(step, args.cold_iters, stream)
        if "dense_step" in locals():
            out["dense_baseline"]["cold_cache_ms_per_step"] = cold_cache_ms(dense_step, args.cold_iters, stream)

    if bf and not few_tokens and not training:
        # the library GEMM (hipBLASLt through torch.matmul) on the gate's shape,
        # without any epilogue: a practical MFMA ceiling measured on the same
        # box, beside the datasheet peak
        C = torch.empty((T, f), dtype=torch.bfloat16, device=dev)
        lib_ms = _timed(lambda: torch.matmul(x, WgT.t(), out=C), steps, warmup, stream)
        del C
        lib_tf = gate_flops / (lib_ms * 1e-3) / 1e12
        out["library_gemm"] = {"what": "torch.matmul (hipBLASLt) x.WgT^T, the gate's GEMM without epilogue",
                               "ms": lib_ms, "tflops": lib_tf, "frac_of_peak": lib_tf / PEAK["bf16_mfma_tflops"]}
        out["roofline"]["frac_of_library_gemm"] = float(lines["gate_gemm_twell_pack"]["achieved"]) / lib_tf

    return out


# capacities (tile_cap, union_cap) of the bounded forward per workload: the
# largest per-(row, tile) count of these inputs over every token is 8 (1.5b)
# and 7 (2b), the largest 128-token block union 43.8% and 27.3% of d_ff; the
# union capacity is that rounded up to a multiple of 64 with at least 1.5% of
# d_ff to spare
BOUNDED_CAPS = {"1.5b": (8, 2560), "2b": (8, 2816)}

# the workloads the default run reports beside the headline, as (name, decode)
EXTRA_WORKLOADS = [("1.5b", False), ("0.5b", False), ("2b", True), ("hybrid", False)]


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (the library has no multi-GPU path); "
                                   "use --gpus 1", "n_gpus": args.gpus}))
        return 2
    if args.copy_calibration:
        return copy_calibration(max(1, args.steps))
    if args.ffn == "relu":
        return relu_bench(args)
    from workloads import CONFIGS

    cfg = CONFIGS[args.config]
    training = cfg.tau_frac is not None
    r = measure(args, args.config, args.decode, args.steps, args.warmup, full=True)
    w = r.pop("_workload")
    out = {
        "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes, densities and neuron-popularity structure of the workload)",
        "config": {"workload": r["workload"], "name": args.config, "T": r["T"], "d_model": r["d_model"],
                   "d_ff": r["d_ff"], "tile": "16x64", "realised_density": r["realised_density"],
                   "pass": r["pass"]},
    }
    for k in ("mean_union_fraction", "union_neurons", "dense_rows"):
        if k in r:
            out["config"][k] = r[k]
    for k in ("stages_ms", "roofline", "stage_roofline", "dense_baseline", "speedup_vs_dense",
              "dense_vs_sparse_rel_diff", "workspace_bytes", "cold_cache_ms_per_step", "library_gemm",
              "saved_state_bytes", "compact_twell", "stage_note", "bounded_forward"):
        if k in r:
            out[k] = r[k]
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, training)
    del w
    if not args.no_extras:
        # the other workloads, each with a short timed run of its own
        ex = {}
        es, ew = max(1, min(args.steps, 10)), max(1, min(args.warmup, 10))
        # each extra workload follows seconds of host-side input generation with
        # the GPU idle: its warmup runs until 0.25 s of steps have passed
        for name, dec in EXTRA_WORKLOADS:
            if name == args.config and dec == args.decode:
                continue
            e = measure(args, name, dec, es, ew, full=False, warm_s=0.25)
            e.pop("_workload")
            e["steps"], e["warmup"], e["warmup_min_s"] = es, ew, 0.25
            ex[name + ("_decode" if dec else "")] = e
        out["extra_workloads"] = ex
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())

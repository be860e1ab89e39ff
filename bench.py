#!/usr/bin/env python3
"""FFN-layer throughput of the TwELL forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0.5b]

One step is one pass of the whole forward hot path over the workload's token
batch, inputs already resident in HBM:
    twell_gate_pack   gate GEMM + bias + ReLU + TwELL pack in the epilogue
    twell_sparse_up   a = h * (x . WuT^T) on the stored pairs
    twell_sparse_down y = a . Wd over the stored pairs
The library's own dense MFMA FFN (twell_ffn_dense_fwd) is timed on the same
inputs for the speedup.  Every kernel is timed with HIP events recorded on the
stream the kernels are launched on.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FFN tokens/s @1 GPU (TwELL vs own dense); % HBM / MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="0.5b")
    ap.add_argument("--decode", action="store_true", help="use the workload's decode-shaped pass")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def cpu_baseline(w, budget_s: float) -> dict:
    """Time the CPU oracle's sparse forward on a bounded sample of token rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    chunk = 256
    done = 0
    t0 = time.perf_counter()
    while done < w.T and time.perf_counter() - t0 < budget_s:
        rows = slice(done, min(done + chunk, w.T))
        oracle.ffn_sparse_fwd(w.x[rows], w.WgT, w.bg, w.WuT, w.Wd)
        done = rows.stop
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {done} of {w.T} token rows, float64 numpy sparse forward "
                      f"(gate GEMM, TwELL pack, per-pair up/down), {dt:.1f} s"}


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        return 2
    import numpy as np
    import torch

    import activation_sparse_feedforward_gate_amd as tw
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[args.config]
    w = make_workload(args.config, decode=args.decode)
    T, d, f = w.T, w.d, w.f
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dt(a):
        t = torch.from_numpy(a).to(dev)
        return t.to(torch.bfloat16) if cfg.dtype == "bf16" else t

    x, WgT, bg, WuT, Wd = dt(w.x), dt(w.WgT), dt(w.bg), dt(w.WuT), dt(w.Wd)
    in_dt = tw.TWELL_BF16 if cfg.dtype == "bf16" else tw.TWELL_F32
    shape = tw.ffn_shape(T, d, f, in_dt, tw.TWELL_F32)
    h = tw.alloc_twell_mat(T, f, tw.TWELL_F32, device=dev)
    aval = torch.empty_like(h.val)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(rec=None):
        if rec is not None:
            rec[0].record(stream)
        tw.twell_gate_pack(shape, x, WgT, bg, h, stream)
        if rec is not None:
            rec[1].record(stream)
        tw.twell_sparse_up(shape, x, WuT, h, aval, stream)
        if rec is not None:
            rec[2].record(stream)
        tw.twell_sparse_down(shape, aval, Wd, h, y, stream)
        if rec is not None:
            rec[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    t_start = ev()
    t_end = ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(recs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    stage = np.array([[r[i].elapsed_time(r[i + 1]) for i in range(3)] for r in recs])
    stage_ms = stage.mean(axis=0)
    ms_step = total_ms / args.steps
    nnz = int(h.cnt.to(torch.int64).sum().item())

    out = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.description + (" (decode pass)" if args.decode else ""),
                   "name": args.config, "T": T, "d_model": d, "d_ff": f, "tile": "16x64",
                   "realised_density": nnz / (T * f)},
        "stages_ms": {"gate_gemm_twell_pack": stage_ms[0], "sparse_up": stage_ms[1], "sparse_down": stage_ms[2]},
    }

    # roofline of each stage; the dominant one is reported as "roofline"
    gate_flops = 2.0 * T * d * f
    sparse_flops = 2.0 * nnz * d
    lines = {
        "gate_gemm_twell_pack": {"bound": "mfma", "achieved": gate_flops / (stage_ms[0] * 1e-3) / 1e12,
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"},
        "sparse_up": {"bound": "mfma", "achieved": sparse_flops / (stage_ms[1] * 1e-3) / 1e12,
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"},
        "sparse_down": {"bound": "mfma", "achieved": sparse_flops / (stage_ms[2] * 1e-3) / 1e12,
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"},
    }
    for v in lines.values():
        v["frac"] = v["achieved"] / v["peak"]
        v["traffic"] = None
    dom = max(lines, key=lambda k: out["stages_ms"][k])
    out["roofline"] = dict(lines[dom], kernel=dom)
    out["stage_roofline"] = lines

    if not args.no_dense and cfg.dtype == "bf16":
        dshape = tw.ffn_shape(T, d, f, tw.TWELL_BF16, tw.TWELL_F32)
        dws = torch.empty(tw.twell_ffn_dense_fwd_workspace(dshape), dtype=torch.uint8, device=dev)
        yd = torch.empty_like(y)
        for _ in range(args.warmup):
            tw.twell_ffn_dense_fwd(dshape, x, WgT, bg, WuT, Wd, yd, dws, stream)
        torch.cuda.synchronize()
        a0, a1 = ev(), ev()
        a0.record(stream)
        for _ in range(args.steps):
            tw.twell_ffn_dense_fwd(dshape, x, WgT, bg, WuT, Wd, yd, dws, stream)
        a1.record(stream)
        torch.cuda.synchronize()
        dms = a0.elapsed_time(a1) / args.steps
        out["dense_baseline"] = {"tokens_per_s": T / (dms * 1e-3), "ms_per_step": dms,
                                 "tflops": 6.0 * T * d * f / (dms * 1e-3) / 1e12}
        out["speedup_vs_dense"] = dms / ms_step
        diff = (y - yd).norm().item() / max(yd.norm().item(), 1e-30)
        out["dense_vs_sparse_rel_diff"] = diff

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())

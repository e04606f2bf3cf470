"""Benchmark of the selective-scan backward on one MI355X.

One step = one ``ssm_scan_bwd`` call (segment summaries, carries, the main
backward sweep, final reductions) over the mamba-370m-shaped workload
(batch 8, T 2048, d_inner 2048, d_state 16, float32), inputs resident in HBM.
Prints one JSON line.  Only one GPU is supported.

    python bench.py [--steps K] [--warmup W] [--workload mamba370m] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSM-bwd state-elements/s (B·T·d_inner·d_state) + HBM GB/s as % of MI355X peak"
HBM_PEAK_GBPS = 8000.0
# fp32 vector peak without packed instructions: 256 CUs x 64 lanes x 2 flop (FMA) x 2.4 GHz
VALU_PEAK_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
# algorithmic flops per state element of the backward's definition (mul, add, exp = 1 each):
# forward  a = exp(delta A) 2, h = a h + (delta u) B 3, y += C h 2             -> 7
# adjoint  g = dy C + a g 3, w = g (a h_prev) 1, d_delta += A w 2, d_A_log += delta w 2,
#          d_u's sum g B 2, d_B = sum_d g delta u 2, d_C = sum_d dy h 2        -> 14
FLOPS_PER_SE = 21


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba370m")
    ap.add_argument("--seg-len", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


class HipEvents:
    """Raw HIP events from the process's (torch's) HIP runtime."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def cpu_baseline(cfg, batches: int):
    """The fp64 oracle, single-threaded, on the first `batches` sequences of the workload."""
    from threadpoolctl import threadpool_limits

    from oracle import ssm as orc
    from synth import scan_inputs
    p = scan_inputs(batches, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, cfg.seed)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"], p["d_out"])
        dt = time.perf_counter() - t0
    se = batches * cfg.seqlen * cfg.d_inner * cfg.d_state
    return {"value": se / dt, "unit": "state-elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{batches} of {cfg.batch} sequences of the same workload ({se} state elements, "
                      f"{dt:.1f} s, fp64 NumPy, 1 thread)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding "
              "of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    import torch

    import selective_state_space_bwd_amd as ssm
    from synth import CONFIGS, scan_inputs

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    p = scan_inputs(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, cfg.seed)
    t = {k: (torch.from_numpy(v).to(dev) if k in ("A_log", "D") else torch.from_numpy(v).to(tdt).to(dev))
         for k, v in p.items()}
    del p
    out = {k: torch.empty_like(t["u"]) for k in ("d_u", "d_delta", "d_z")}
    out["d_B"] = torch.empty_like(t["B"])
    out["d_C"] = torch.empty_like(t["C"])
    out["d_A_log"] = torch.empty_like(t["A_log"])
    out["d_D"] = torch.empty_like(t["D"])
    dims = ssm.scan_dims(t["u"], t["B"], seg_len=args.seg_len)
    ws = torch.empty(ssm.ssm_scan_bwd_workspace_size(dims, tdt), dtype=torch.uint8, device=dev)

    def step(ev=None):
        ssm.ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"],
                         out=out, workspace=ws, seg_len=args.seg_len, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hip = HipEvents()
    evs = [hip.create(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = np.array([[hip.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for e in evs])
    hip.destroy([e for es in evs for e in es])

    ms_step = elapsed / args.steps * 1e3
    se = cfg.state_elements
    el = 4 if cfg.dtype == "f32" else 2
    rows = cfg.batch * cfg.seqlen
    alg_bytes = (7 * rows * cfg.d_inner + 4 * rows * cfg.d_state) * el + (2 * cfg.d_inner * (cfg.d_state + 1)) * 4
    main_ms = float(stages[:, 2].mean())
    # the main sweep reads u, delta, z, d_out, B, C and writes d_u, d_delta, d_z (d_B, d_C go out as partials)
    main_bytes = (7 * rows * cfg.d_inner + 2 * rows * cfg.d_state) * el
    main_gbps = main_bytes / (main_ms * 1e-3) / 1e9
    main_tflops = FLOPS_PER_SE * se / (main_ms * 1e-3) / 1e12
    hbm_frac = main_gbps / HBM_PEAK_GBPS
    alu_frac = main_tflops / VALU_PEAK_TFLOPS
    if alu_frac >= hbm_frac:
        roof = {"bound": "alu", "achieved": round(main_tflops, 3), "peak": round(VALU_PEAK_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(alu_frac, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(main_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(hbm_frac, 4)}
    roof["traffic"] = None
    roof["kernel"] = "scan_bwd_main"
    roof["kernel_ms"] = round(main_ms, 4)
    roof["hbm_frac"] = round(hbm_frac, 4)
    roof["alu_frac"] = round(alu_frac, 4)

    line = {
        "metric": METRIC,
        "value": se / (ms_step * 1e-3),
        "unit": "state-elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "d_inner": cfg.d_inner,
                   "d_state": cfg.d_state, "seg_len": args.seg_len or "auto",
                   "storage": cfg.dtype},
        "hbm": {"algorithmic_bytes": alg_bytes, "effective_GBps": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
                "frac_of_peak": round(alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "stages_ms": {"summary": round(float(stages[:, 0].mean()), 4), "carry": round(float(stages[:, 1].mean()), 4),
                      "main": round(main_ms, 4), "finalize": round(float(stages[:, 3].mean()), 4)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, batches=2 if cfg.seqlen * cfg.d_inner <= 2048 * 2048 else 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the selective-scan backward on one MI355X.

One step of the default workload = one ``ssm_scan_bwd`` call (segment
summaries, carries, the main backward sweep, final reductions) over the
mamba-370m-shaped problem (batch 8, T 2048, d_inner 2048, d_state 16, float32),
inputs resident in HBM.  The same run then times the other workloads of the
benchmark (mamba-130m-shaped and mamba-2.8b-shaped scans, the full layer; the
tiny case is parity-only) and reports them under ``configs``.  Prints one JSON
line.  Only one GPU is supported.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-configs]
                    [--copy-probe] [--ckpt] [--recompute] [--seg-len L]

``--workload`` times one other workload instead (mamba130m, mamba2p8b, layer,
backbone, revscan, tiny).  ``--copy-probe`` only copies a 1 GiB device buffer
``steps`` times: the plain copy of known size that calibrates the HBM byte
counters of rocprofv3.

The CPU baseline is the fp64 oracle (test infrastructure) run on the host's
cores, sharded over (batch, 256-channel block) in a process pool; it runs before
any GPU work, so the pool forks a process that has not touched the GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSM-bwd state-elements/s (B·T·d_inner·d_state) + HBM GB/s as % of MI355X peak"
HBM_PEAK_GBPS = 8000.0                 # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0         # dense bf16 matrix cores, published
FP32_VECTOR_PEAK_TFLOPS = 157.3        # published fp32 vector peak (packed FMA)
# the same vector units without packed instructions, which this library does not
# use: 256 CUs x 64 lanes x 2 flop (FMA) x 2.4 GHz
FP32_NONPACKED_CEILING_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12
# algorithmic flops per state element of the backward's definition (mul, add, exp = 1 each):
# forward  a = exp(delta A) 2, h = a h + (delta u) B 3, y += C h 2             -> 7
# adjoint  g = dy C + a g 3, w = g (a h_prev) 1, d_delta += A w 2, d_A_log += delta w 2,
#          d_u's sum g B 2, d_B = sum_d g delta u 2, d_C = sum_d dy h 2        -> 14
FLOPS_PER_SE = 21
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
CHANNEL_BLOCK = 1024  # most channels per CPU-baseline shard (the oracle's own block size)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload, DEFAULT_STEPS)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps before them (default: per workload)")
    ap.add_argument("--workload", default="mamba370m")
    ap.add_argument("--seg-len", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the named workload (skip the other workloads' summary)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--recompute", action="store_true",
                    help="backbone: keep only the layer inputs (SSM_KEEP_INPUTS); the backward reruns each layer's "
                         "forward")
    ap.add_argument("--recompute-inputs", action="store_true",
                    help="layer and backbone: the forward keeps y instead of the products' inputs (gated, u, xn) "
                         "and the backward recomputes the gate, the conv + SiLU and the RMSNorm forward")
    ap.add_argument("--ckpt", action="store_true",
                    help="time the backward that takes the scan's state before every 8-step chunk from the "
                         "forward (scan workloads: ssm_scan_bwd_ckpt after one ssm_scan_fwd; layer and backbone: "
                         "the forward keeps them) instead of rebuilding the states")
    return ap.parse_args()


class HipEvents:
    """Raw HIP events from the process's (torch's) HIP runtime, recorded by the library on its stream."""

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


# the sources each profiled kernel (or whole call) is compiled from
KERNEL_SOURCES = {"scan_bwd_main": ("scan.hip", "common.hpp"), "ssm_scan_bwd": ("scan.hip", "common.hpp")}


def code_text(src: str) -> str:
    """C++ source without its comments, whitespace runs collapsed to one space: what the compiler sees."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, copied through its closing quote
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_digest(kernel: str) -> str:
    """Digest of a kernel's sources (code only: comments and layout do not count), so that recorded
    counter totals are used only with the code they came from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_bwd_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + code_text(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` (or per call, kernel "ssm_scan_bwd") from the committed counter
    summary, if it was taken on the current sources: lines `traffic <workload> <kernel> <bytes> <digest>`."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = source_digest(kernel)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = re.match(r"^traffic\s+(\S+)\s+(\S+)\s+(\d+)\s+([0-9a-f]+)\s*$", line.strip())
            if m and m.group(1) == workload and m.group(2) == kernel and m.group(4) == digest:
                return int(m.group(3))
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host's cores (fork pool, before any GPU use)

_POOL_INPUTS: dict = {}


def _pool_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _scan_shard(task):
    """The oracle on one (batch element, channel block) shard; returns its partial sums."""
    from oracle import ssm as orc
    b, d0, d1 = task
    p = _POOL_INPUTS
    t0 = time.process_time()
    r = orc.ssm_scan_bwd(p["u"][b:b + 1, :, d0:d1], p["delta"][b:b + 1, :, d0:d1], p["A_log"][d0:d1],
                         p["B"][b:b + 1], p["C"][b:b + 1], p["D"][d0:d1], p["z"][b:b + 1, :, d0:d1],
                         p["d_out"][b:b + 1, :, d0:d1])
    return task, r["d_B"][0], r["d_C"][0], r["d_A_log"], r["d_D"], time.process_time() - t0


def _layer_shard(b):
    from oracle import layer as orc
    p = _POOL_INPUTS
    q = {k: (v[b:b + 1] if k in ("x", "d_out") else v) for k, v in p.items() if not k.startswith("_")}
    t0 = time.process_time()
    r = orc.layer_bwd(q, q["d_out"], p["_d_state"], p["_dt_rank"])
    return b, {k: v for k, v in r.items() if k != "d_x"}, time.process_time() - t0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_workers() -> int:
    # the host share of one GPU is 16 cores at most on the GPU hosts
    return max(1, min(len(os.sched_getaffinity(0)), 16))


MIN_CPU_SECONDS = 10.0


def _channel_block(cfg, n: int) -> int:
    """Channels per CPU-baseline shard: at most CHANNEL_BLOCK, a multiple of 256, and small enough
    that each of the n workers gets at least two shards when the shape allows."""
    per_b = -(-2 * n // cfg.batch)  # channel blocks per batch element for 2n shards
    return max(256, min(CHANNEL_BLOCK, cfg.d_inner // per_b // 256 * 256))


def cpu_baseline_scan(cfg):
    """The fp64 oracle over the whole workload, sharded over (batch element, channel block) on a
    fork pool of all host cores (BLAS threads 1 per worker).  The shards' partial sums of d_B, d_C
    (over channel blocks) and d_A_log, d_D (over batch) are added in shard order.  The whole workload
    is repeated until the workers have spent MIN_CPU_SECONDS of CPU time."""
    import multiprocessing as mp

    from synth import scan_inputs
    global _POOL_INPUTS
    _POOL_INPUTS = scan_inputs(cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dtype, cfg.seed)
    n = _pool_workers()
    blk = _channel_block(cfg, n)
    tasks = [(b, d0, min(d0 + blk, cfg.d_inner)) for b in range(cfg.batch) for d0 in range(0, cfg.d_inner, blk)]
    passes, wall, cpu = 0, 0.0, 0.0
    with mp.get_context("fork").Pool(n, initializer=_pool_init) as pool:
        while cpu < MIN_CPU_SECONDS and passes < 8:
            t0 = time.perf_counter()
            res = pool.map(_scan_shard, tasks, chunksize=1)
            d_B = np.zeros((cfg.batch, cfg.seqlen, cfg.d_state))
            d_C = np.zeros_like(d_B)
            d_A = np.zeros((cfg.d_inner, cfg.d_state))
            d_D = np.zeros(cfg.d_inner)
            for (b, d0, d1), pb, pc, pa, pd, _ in res:      # fixed order: batch, then channel block
                d_B[b] += pb
                d_C[b] += pc
                d_A[d0:d1] += pa
                d_D[d0:d1] += pd
            wall += time.perf_counter() - t0
            cpu += sum(r[-1] for r in res)
            passes += 1
    _POOL_INPUTS = {}
    se = passes * cfg.state_elements
    return {"value": se / wall, "unit": "state-elements/s", "cores": n, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"the whole workload x {passes} ({se} state elements) as {len(tasks)} shards of "
                      f"(batch element, {blk} channels) on {n} worker processes, fp64 NumPy, "
                      f"1 BLAS thread each; {wall:.2f} s wall, {cpu:.1f} s CPU"}


def cpu_baseline_layer(cfg):
    """The fp64 oracle's whole-layer forward + backward, one sequence per task on a fork pool of all host
    cores, until the workers have spent MIN_CPU_SECONDS of CPU time or the batch is done; parameter
    gradients summed over the sequences in order."""
    import multiprocessing as mp

    from synth import layer_inputs
    global _POOL_INPUTS
    p = layer_inputs(cfg.batch, cfg.seqlen, cfg.d_model, cfg.d_inner, cfg.d_state, cfg.dt_rank, cfg.d_conv,
                     cfg.dtype, cfg.seed)
    p["_d_state"], p["_dt_rank"] = cfg.d_state, cfg.dt_rank
    _POOL_INPUTS = p
    n = _pool_workers()
    with mp.get_context("fork").Pool(n, initializer=_pool_init) as pool:
        t0 = time.perf_counter()
        res = pool.map(_layer_shard, list(range(min(cfg.batch, n))), chunksize=1)
        wall = time.perf_counter() - t0
    tot = {}
    for _, g, _ in sorted(res, key=lambda r: r[0]):
        for k, v in g.items():
            tot[k] = tot.get(k, 0) + v
    cpu = sum(r[-1] for r in res)
    _POOL_INPUTS = {}
    done = len(res)
    se = done * cfg.seqlen * cfg.d_inner * cfg.d_state
    return {"value": se / wall, "unit": "state-elements/s", "cores": n, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{done} of {cfg.batch} sequences of the same workload, one per worker process ({se} state "
                      f"elements), fp64 NumPy forward + backward, 1 BLAS thread each; {wall:.2f} s wall, "
                      f"{cpu:.1f} s CPU"}


# ---------------------------------------------------------------------------
# timing

STAGE_SAMPLES = 4  # timed steps that also record the per-stage HIP events
ROTATE = 3         # copies of each workload's tensors that the steps take in turn (Infinity Cache)


def timed(step, n_events: int, steps: int, warmup: int):
    """Wall time per step over exactly `steps` steps after `warmup` untimed ones,
    and the per-stage times (HIP events the library records between its kernels
    on its stream).  An event record between two kernels costs a few
    microseconds of idle GPU, so only STAGE_SAMPLES evenly spaced steps of the
    timed region carry the events; the others run as a caller would."""
    import torch
    # the events are created before the warm-up, so that the GPU goes from the warm-up steps to the
    # timed ones with no host-side work between them but the synchronisation
    hip = HipEvents()
    every = max(1, steps // STAGE_SAMPLES)
    sampled = [k for k in range(steps) if k % every == every - 1][:STAGE_SAMPLES]
    evs = {k: hip.create(n_events) for k in sampled}
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs.get(k))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = np.array([[hip.elapsed_ms(e[i], e[i + 1]) for i in range(n_events - 1)] for e in evs.values()])
    hip.destroy([e for es in evs.values() for e in es])
    return elapsed / steps * 1e3, stages


def step_stats(step, steps: int):
    """Per-step times of `steps` more steps, each bracketed by events on the stream the library
    runs on (torch's current stream): median, 10th and 90th percentile in ms.  A separate pass
    after the timed one, so the timed region carries no per-step event records."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        step(None)
        ev[k + 1].record()
    torch.cuda.synchronize()
    ms = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    return {"ms_median": round(float(np.median(ms)), 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
            "ms_p90": round(float(np.percentile(ms, 90)), 4), "steps": steps,
            "note": "per-step HIP events in a second pass of the same length after the timed region; "
                    f"steps take {ROTATE} copies of their input and output tensors in turn, so no step finds "
                    "its tensors in the Infinity Cache from the step before"}


# ---------------------------------------------------------------------------
# scan workloads

def scan_bytes(cfg, ckpt: bool):
    el = 4 if cfg.dtype == "f32" else 2
    rows = cfg.batch * cfg.seqlen
    # with given chunk states, the float32 states before every 8-step chunk are one more input
    ckpt_bytes = 4 * cfg.batch * ((cfg.seqlen + 7) // 8) * cfg.d_state * cfg.d_inner if ckpt else 0
    call = ((7 * rows * cfg.d_inner + 4 * rows * cfg.d_state) * el + (2 * cfg.d_inner * (cfg.d_state + 1)) * 4
            + ckpt_bytes)
    # the main sweep reads u, delta, z, d_out, B, C (and the given chunk states) and writes d_u, d_delta,
    # d_z (d_B, d_C go out as partials)
    main = (7 * rows * cfg.d_inner + 2 * rows * cfg.d_state) * el + ckpt_bytes
    return call, main


def scan_roofline(cfg, main_ms, ms_step, main_bytes, call_bytes, traffic_main, traffic_call):
    """Roofline of the main sweep against the published HBM peak (the metric's bound), with its
    arithmetic against the published fp32 vector peak and the non-packed issue ceiling beside it."""
    se = cfg.state_elements
    gbps = main_bytes / (main_ms * 1e-3) / 1e9
    tflops = FLOPS_PER_SE * se / (main_ms * 1e-3) / 1e12
    return {
        "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_main,
        "traffic_GBps": round(traffic_main / (main_ms * 1e-3) / 1e9, 1) if traffic_main else None,
        "traffic_frac_of_peak": round(traffic_main / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) if traffic_main else None,
        "kernel": "scan_bwd_main", "kernel_ms": round(main_ms, 4), "algorithmic_bytes": main_bytes,
        "alu": {"flops_per_state_element": FLOPS_PER_SE, "achieved_TFLOPs": round(tflops, 3),
                "published_fp32_peak_TFLOPs": FP32_VECTOR_PEAK_TFLOPS,
                "frac_of_published_peak": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 4),
                "nonpacked_issue_ceiling_TFLOPs": round(FP32_NONPACKED_CEILING_TFLOPS, 1),
                "frac_of_nonpacked_ceiling": round(tflops / FP32_NONPACKED_CEILING_TFLOPS, 4)},
        "step": {"algorithmic_bytes": call_bytes,
                 "frac_of_hbm_peak": round(call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 "counted_bytes": traffic_call,
                 "counted_GBps": round(traffic_call / (ms_step * 1e-3) / 1e9, 1) if traffic_call else None,
                 "counted_frac_of_peak": round(traffic_call / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                 if traffic_call else None,
                 "counted_over_algorithmic": round(traffic_call / call_bytes, 3) if traffic_call else None},
    }


def prepare_scan(args, cfg):
    """Upload one scan workload's seeded inputs and outputs; returns its step function."""
    import torch

    import selective_state_space_bwd_amd as ssm
    from synth import scan_inputs
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
    # ROTATE copies of the inputs and outputs, used in turn: a step finds none of its
    # tensors in the Infinity Cache from the step before
    sets = [(t, out)] + [({k: v.clone() for k, v in t.items()}, {k: torch.empty_like(v) for k, v in out.items()})
                         for _ in range(ROTATE - 1)]
    turn = [0]

    def next_set():
        i = turn[0]
        turn[0] = (i + 1) % ROTATE
        return sets[i]
    if args.ckpt:
        h_ckpts = [ssm.ssm_scan_fwd(ti["u"], ti["delta"], ti["A_log"], ti["B"], ti["C"], ti["D"], want_y=False,
                                    want_out=False, ckpt_every=8)["h_ckpt"] for ti, _ in sets]
        ws = torch.empty(ssm.ssm_scan_bwd_ckpt_workspace_size(dims, tdt), dtype=torch.uint8, device=dev)

        def step(ev):
            i = turn[0]
            ti, oi = next_set()
            ssm.ssm_scan_bwd_ckpt(ti["u"], ti["delta"], ti["A_log"], ti["B"], ti["C"], ti["D"], ti["z"],
                                  ti["d_out"], h_ckpts[i], out=oi, workspace=ws, seg_len=args.seg_len,
                                  stage_events=ev)
    else:
        ws = torch.empty(ssm.ssm_scan_bwd_workspace_size(dims, tdt), dtype=torch.uint8, device=dev)

        def step(ev):
            ti, oi = next_set()
            ssm.ssm_scan_bwd(ti["u"], ti["delta"], ti["A_log"], ti["B"], ti["C"], ti["D"], ti["z"], ti["d_out"],
                             out=oi, workspace=ws, seg_len=args.seg_len, stage_events=ev)
    return step


def measure_scan(args, cfg, steps, warmup, want_stats=True, step=None):
    import torch
    step = step or prepare_scan(args, cfg)
    ms_step, stages = timed(step, 5, steps, warmup)
    stats = step_stats(step, steps) if want_stats else None
    del step
    torch.cuda.empty_cache()
    return ms_step, stages, stats


def run_scan(args, cfg, step=None):
    ms_step, stages, stats = measure_scan(args, cfg, args.steps, args.warmup, step=step)
    se = cfg.state_elements
    call_bytes, main_bytes = scan_bytes(cfg, args.ckpt)
    main_ms = float(stages[:, 2].mean())
    roof = scan_roofline(cfg, main_ms, ms_step, main_bytes, call_bytes,
                         None if args.ckpt else recorded_traffic(args.workload, "scan_bwd_main"),
                         None if args.ckpt else recorded_traffic(args.workload, "ssm_scan_bwd"))
    line = {
        "metric": METRIC, "value": se / (ms_step * 1e-3), "unit": "state-elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "d_inner": cfg.d_inner,
                   "d_state": cfg.d_state, "seg_len": args.seg_len or "auto", "storage": cfg.dtype,
                   "chunk_states": "given by the forward" if args.ckpt else "rebuilt"},
        "hbm": {"algorithmic_bytes": call_bytes, "effective_GBps": round(call_bytes / (ms_step * 1e-3) / 1e9, 1),
                "frac_of_peak": round(call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "timing": stats,
        "stages_ms": {"summary": round(float(stages[:, 0].mean()), 4), "carry": round(float(stages[:, 1].mean()), 4),
                      "main": round(main_ms, 4), "finalize": round(float(stages[:, 3].mean()), 4)},
        "roofline": roof,
    }
    return line


def config_entry_scan(args, key, cfg, warmup, step=None):
    """One other scan workload of the benchmark, timed in the same run."""
    ms_step, stages, stats = measure_scan(args, cfg, args.steps, warmup, step=step)
    call_bytes, main_bytes = scan_bytes(cfg, False)
    main_ms = float(stages[:, 2].mean())
    med = stats["ms_median"]
    roof = scan_roofline(cfg, main_ms, med, main_bytes, call_bytes, recorded_traffic(key, "scan_bwd_main"),
                         recorded_traffic(key, "ssm_scan_bwd"))
    return {"workload": cfg.name, "dtype": cfg.dtype, "steps": args.steps, "warmup": warmup,
            "ms_per_step": round(ms_step, 4), **{k: stats[k] for k in ("ms_median", "ms_p10", "ms_p90")},
            "state_elements_per_s": round(cfg.state_elements / (med * 1e-3), 1),
            "hbm_effective_frac": round(call_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "stages_ms": {"summary": round(float(stages[:, 0].mean()), 4),
                          "carry": round(float(stages[:, 1].mean()), 4), "main": round(main_ms, 4),
                          "finalize": round(float(stages[:, 3].mean()), 4)},
            "dominant_kernel": roof}


# ---------------------------------------------------------------------------
# layer

LAYER_STAGES = ("gate_fwd", "out_proj", "conv_silu_fwd", "scan_bwd", "dt_proj", "x_proj", "conv_bwd",
                "rmsnorm_fwd", "in_proj", "rmsnorm_bwd")


# what the layer forward keeps for the backward: the products' inputs (gated, u, xn, as the page's
# MambaLayerFlat keeps gated, u and post_norm), or only y (the backward recomputes the gate, the conv + SiLU
# and the RMSNorm forward, 0.25 GB less activation memory per layer of the full layer shape)
LAYER_SAVED_KEPT = "xz, xdbl, delta and the products' inputs gated, u, xn (the page's acts keep gated, u, post_norm)"
LAYER_SAVED_LEAN = "xz, xdbl, delta, y; the gate, conv + SiLU and RMSNorm forward recomputed in the backward"


def measure_layer(args, cfg, steps, warmup, want_stats=True, keep_inputs=True, scan_states=None):
    import torch

    import selective_state_space_bwd_amd as ssm
    from synth import layer_inputs
    dev = torch.device("cuda:0")
    p = layer_inputs(cfg.batch, cfg.seqlen, cfg.d_model, cfg.d_inner, cfg.d_state, cfg.dt_rank, cfg.d_conv,
                     cfg.dtype, cfg.seed)
    bf = ("x", "d_out", "W_in", "W_x", "W_dt", "W_out")
    t = {k: (torch.from_numpy(v).to(torch.bfloat16) if k in bf else torch.from_numpy(v)).to(dev) for k, v in p.items()}
    del p
    W = {k: t[k] for k in ssm.LAYER_WEIGHTS}
    # ROTATE copies of the input, the upstream gradient and the saved activations, used in turn
    xs = [t["x"]] + [t["x"].clone() for _ in range(ROTATE - 1)]
    gs = [t["d_out"]] + [t["d_out"].clone() for _ in range(ROTATE - 1)]
    keep_states = args.ckpt if scan_states is None else scan_states
    saves = [ssm.mamba_layer_fwd(x, W, seg_len=args.seg_len, keep_scan_states=keep_states,
                                 keep_gemm_inputs=keep_inputs)[1] for x in xs]
    ws = torch.empty(ssm.mamba_layer_bwd_workspace_size(t["x"], W, seg_len=args.seg_len), dtype=torch.uint8,
                     device=dev)
    out = ssm.mamba_layer_bwd(xs[0], W, saves[0], gs[0], workspace=ws, seg_len=args.seg_len)
    turn = [0]

    def step(ev):
        i = turn[0]
        turn[0] = (i + 1) % ROTATE
        ssm.mamba_layer_bwd(xs[i], W, saves[i], gs[i], workspace=ws, out=out, seg_len=args.seg_len,
                            stage_events=ev)

    ms_step, stages = timed(step, 11, steps, warmup)
    stats = step_stats(step, steps) if want_stats else None
    del t, W, xs, gs, saves, ws, out
    torch.cuda.empty_cache()
    return ms_step, {name: float(stages[:, i].mean()) for i, name in enumerate(LAYER_STAGES)}, stats


def layer_gemm_flops(cfg):
    M = cfg.batch * cfg.seqlen
    dm, di, R2 = cfg.d_model, cfg.d_inner, cfg.dt_rank + 2 * cfg.d_state
    return {"out_proj": 4 * M * dm * di, "dt_proj": 4 * M * di * cfg.dt_rank, "x_proj": 4 * M * di * R2,
            "in_proj": 4 * M * 2 * di * dm}


def layer_scan_bytes(cfg):
    """Algorithmic bytes of the layer's scan stage (bf16 activations: u, delta, z, d_out read, d_u, d_delta
    written, d_z written; B, C read and d_B, d_C written; A_log, D and their gradients)."""
    rows = cfg.batch * cfg.seqlen
    return (7 * rows * cfg.d_inner + 4 * rows * cfg.d_state) * 2 + 2 * cfg.d_inner * (cfg.d_state + 1) * 4


def run_layer(args, cfg):
    keep = not args.recompute_inputs
    ms_step, st, stats = measure_layer(args, cfg, args.steps, args.warmup, keep_inputs=keep)
    gemm_flops = layer_gemm_flops(cfg)
    in_tf = gemm_flops["in_proj"] / (st["in_proj"] * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(in_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(in_tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "kernel": "gemm_pair_kernel, in_proj dX + dW in one launch, then the split-k sum of dW",
            "kernel_ms": round(st["in_proj"], 4)}
    gemm_ms = sum(st[k] for k in gemm_flops)
    line = {
        "metric": METRIC, "value": cfg.state_elements / (ms_step * 1e-3), "unit": "state-elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "d_model": cfg.d_model,
                   "d_inner": cfg.d_inner, "d_state": cfg.d_state, "dt_rank": cfg.dt_rank, "d_conv": cfg.d_conv,
                   "seg_len": args.seg_len or "auto", "storage": "bf16",
                   "scan_states": "kept by the forward" if args.ckpt else "rebuilt",
                   "saved": LAYER_SAVED_KEPT if keep else LAYER_SAVED_LEAN},
        "timing": stats,
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "gemm": {"TFLOP": round(sum(gemm_flops.values()) / 1e12, 4), "ms": round(gemm_ms, 4),
                 "TFLOPs": round(sum(gemm_flops.values()) / (gemm_ms * 1e-3) / 1e12, 1),
                 "per_stage_TFLOPs": {k: round(v / (st[k] * 1e-3) / 1e12, 1) for k, v in gemm_flops.items()}},
        "roofline": roof,
    }
    return line


def config_entry_layer(args, cfg, warmup):
    ms_step, st, stats = measure_layer(args, cfg, args.steps, warmup)
    lean_ms, lean_st, lean_stats = measure_layer(args, cfg, args.steps, warmup, keep_inputs=False)
    ck_ms, ck_st, ck_stats = measure_layer(args, cfg, args.steps, warmup, scan_states=True)
    gemm_flops = layer_gemm_flops(cfg)
    med = stats["ms_median"]
    dom = max(st, key=st.get)
    if dom in gemm_flops:
        tf = gemm_flops[dom] / (st[dom] * 1e-3) / 1e12
        droof = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        nbytes = layer_scan_bytes(cfg) if dom == "scan_bwd" else None
        gbps = nbytes / (st[dom] * 1e-3) / 1e9 if nbytes else None
        droof = {"bound": "hbm", "achieved": round(gbps, 1) if gbps else None, "peak": HBM_PEAK_GBPS,
                 "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4) if gbps else None,
                 "algorithmic_bytes": nbytes}
    droof.update({"kernel": f"{dom} stage" + (" (summary, carry, main sweep, finalize)" if dom == "scan_bwd" else ""),
                  "kernel_ms": round(st[dom], 4)})
    return {"workload": cfg.name, "dtype": "bf16", "steps": args.steps, "warmup": warmup, "saved": LAYER_SAVED_KEPT,
            "ms_per_step": round(ms_step, 4), **{k: stats[k] for k in ("ms_median", "ms_p10", "ms_p90")},
            "state_elements_per_s": round(cfg.state_elements / (med * 1e-3), 1),
            "stages_ms": {k: round(v, 4) for k, v in st.items()},
            "gemm_TFLOPs": {k: round(v / (st[k] * 1e-3) / 1e12, 1) for k, v in gemm_flops.items()},
            "dominant_kernel": droof,
            "recompute_inputs": {"saved": LAYER_SAVED_LEAN, "ms_per_step": round(lean_ms, 4),
                                 **{k: lean_stats[k] for k in ("ms_median", "ms_p10", "ms_p90")},
                                 "stages_ms": {k: round(v, 4) for k, v in lean_st.items()}},
            "chunk_states_kept": {"saved": LAYER_SAVED_KEPT + ", and the scan's state before every 8-step chunk "
                                           "(written by the forward; the backward does not rebuild them)",
                                  "ms_per_step": round(ck_ms, 4),
                                  **{k: ck_stats[k] for k in ("ms_median", "ms_p10", "ms_p90")},
                                  "stages_ms": {k: round(v, 4) for k, v in ck_st.items()}}}


def config_entry_tiny(args, cfg, warmup, step=None):
    ms_step, _, stats = measure_scan(args, cfg, args.steps, warmup, step=step)
    return {"workload": cfg.name, "dtype": cfg.dtype, "steps": args.steps, "warmup": warmup,
            "role": "parity case (checked against the fp64 oracle and finite differences by the tests); "
                    "launch-bound, timed here only for completeness",
            "ms_per_step": round(ms_step, 4), **{k: stats[k] for k in ("ms_median", "ms_p10", "ms_p90")}}


def run_configs(args, keys, steps=None):
    """The benchmark's other workloads, timed in this run with the same number of timed steps; each
    warms up for the run's warm-up steps or its own default, whichever is more (the two small ones run
    before the headline, so this also brings the clocks up before the headline's warm-up).  `steps`
    may hold step functions of scan workloads whose inputs are already on the GPU."""
    from synth import CONFIGS
    out = {}
    steps = steps or {}
    for key in keys:
        if key == args.workload:
            continue
        cfg = CONFIGS[key]
        warmup = max(args.warmup, DEFAULT_STEPS[key][0])
        print(f"bench: timing {cfg.name}", file=sys.stderr, flush=True)
        if key == "tiny":
            out[key] = config_entry_tiny(args, cfg, warmup, step=steps.pop(key, None))
        elif key == "layer":
            out[key] = config_entry_layer(args, cfg, warmup)
        else:
            out[key] = config_entry_scan(args, key, cfg, warmup, step=steps.pop(key, None))
    return out


# ---------------------------------------------------------------------------
# reverse linear recurrence

def cpu_baseline_recurrence(cfg):
    """The fp64 oracle, single-threaded, one whole sequence at a time until 10 s have passed."""
    from threadpoolctl import threadpool_limits

    from oracle import recurrence as orc
    from synth import recurrence_inputs
    p = recurrence_inputs(cfg.batch, cfg.seqlen, cfg.channels, cfg.dtype, seed=cfg.seed, decay="ssm")
    dt, done = 0.0, 0
    with threadpool_limits(1):
        while done < cfg.batch and dt < MIN_CPU_SECONDS:
            t0 = time.perf_counter()
            orc.reverse_linear_scan(p["a"][done:done + 1], p["b"][done:done + 1])
            dt += time.perf_counter() - t0
            done += 1
    n = done * cfg.seqlen * cfg.channels
    return {"value": n / dt, "unit": "elements/s", "cores": 1, "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{done} of {cfg.batch} sequences of the same workload, one at a time ({n} elements, "
                      f"{dt:.1f} s, fp64 NumPy, 1 thread)"}


def run_recurrence(args, cfg):
    """reverse_linear_scan on [B, T, C]: the decayed sweep (the value) and the a = 1 cumsum backward."""
    import torch

    import selective_state_space_bwd_amd as ssm
    from synth import recurrence_inputs
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    p = recurrence_inputs(cfg.batch, cfg.seqlen, cfg.channels, cfg.dtype, seed=cfg.seed, decay="ssm")
    a = torch.from_numpy(p["a"]).to(tdt).to(dev)
    b = torch.from_numpy(p["b"]).to(tdt).to(dev)
    x = torch.empty_like(b)
    ws = torch.empty(max(1, ssm.lib().reverse_linear_scan_workspace_size(cfg.batch, cfg.seqlen, cfg.channels, 1)),
                     dtype=torch.uint8, device=dev)

    def run(decayed):
        for _ in range(args.warmup):
            ssm.reverse_linear_scan(a if decayed else None, b, x=x, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            ssm.reverse_linear_scan(a if decayed else None, b, x=x, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = run(True)
    ms_unit = run(False)
    el = 4 if cfg.dtype == "f32" else 2
    alg = 3 * cfg.elements * el          # a, b read, x written
    gbps = alg / (ms * 1e-3) / 1e9
    return {
        "metric": "reverse linear scan elements/s (B·T·C)", "value": cfg.elements / (ms * 1e-3),
        "unit": "elements/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen": cfg.seqlen, "channels": cfg.channels,
                   "decay": "exp(-softplus(N(-2, 0.5)))"},
        "unit_decay_ms": round(ms_unit, 4),
        "unit_decay_GBps": round(2 * cfg.elements * el / (ms_unit * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "reverse_linear_scan (summary + carry + final sweep, one call)",
                     "kernel_ms": round(ms, 4), "algorithmic_bytes": alg},
    }


# ---------------------------------------------------------------------------
# backbone

def cpu_baseline_backbone(cfg, steps: int = 0):
    """The fp64 oracle's backbone forward + backward, single-threaded, on the first `steps` steps (default: all)
    of one sequence."""
    steps = steps or cfg.seqlen
    from threadpoolctl import threadpool_limits

    from oracle import backbone as orc
    from synth import backbone_inputs
    bp, layers = backbone_inputs(cfg.n_layers, cfg.input_dim, 1, steps, cfg.d_model, cfg.d_inner, cfg.d_state,
                                 cfg.dt_rank, cfg.d_conv, cfg.dtype, seed=cfg.seed)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.backbone_bwd(bp, layers, bp["d_out"], cfg.d_state, cfg.dt_rank, cfg.eps)
        dt = time.perf_counter() - t0
    se = cfg.n_layers * steps * cfg.d_inner * cfg.d_state
    return {"value": se / dt, "unit": "state-elements/s", "cores": 1, "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"the first {steps} steps of 1 sequence at the workload's widths ({se} state elements, "
                      f"{dt:.1f} s, fp64 NumPy forward + backward, 1 thread)"}


def run_backbone(args, cfg):
    """mamba_backbone_bwd on the backbone workload; its activations come from mamba_backbone_fwd before the timing."""
    import torch

    import selective_state_space_bwd_amd as ssm
    from synth import backbone_inputs
    dev = torch.device("cuda:0")
    bp, layers = backbone_inputs(cfg.n_layers, cfg.input_dim, cfg.batch, cfg.seqlen, cfg.d_model, cfg.d_inner,
                                 cfg.d_state, cfg.dt_rank, cfg.d_conv, cfg.dtype, seed=cfg.seed)
    bf = ("inp", "W_ip", "d_out", "W_in", "W_x", "W_dt", "W_out")
    cv = lambda k, v: (torch.from_numpy(v).to(torch.bfloat16) if k in bf else torch.from_numpy(v)).to(dev)
    tb = {k: cv(k, v) for k, v in bp.items()}
    tl = [{k: cv(k, v) for k, v in p.items()} for p in layers]
    del bp, layers
    keep = "inputs" if args.recompute else "all"
    keep_in = keep == "all" and not args.recompute_inputs
    _, kept = ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, seg_len=args.seg_len,
                                     keep=keep, keep_scan_states=args.ckpt, keep_gemm_inputs=keep_in)
    ws = torch.empty(ssm.mamba_backbone_bwd_workspace_size(tb["inp"], tb["W_ip"], tl, seg_len=args.seg_len, keep=keep),
                     dtype=torch.uint8, device=dev)
    out = ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"], workspace=ws,
                                 seg_len=args.seg_len)

    def step(_=None):
        ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"], workspace=ws, out=out,
                               seg_len=args.seg_len)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    stats = step_stats(step, args.steps)
    M = cfg.batch * cfg.seqlen
    dm, di, R2 = cfg.d_model, cfg.d_inner, cfg.dt_rank + 2 * cfg.d_state
    layer_flops = 4 * M * (dm * di + di * cfg.dt_rank + di * R2 + 2 * di * dm)
    flops = cfg.n_layers * layer_flops + 2 * M * cfg.input_dim * dm      # input projection: dW only
    tf = flops / (ms * 1e-3) / 1e12
    kept_bytes = (sum(x.numel() * x.element_size() for x in kept["xs"])
                  + sum(v.numel() * v.element_size() for s_ in (kept["saved"] or []) for v in s_.values()))
    return {
        "metric": METRIC, "value": cfg.state_elements / (ms * 1e-3), "unit": "state-elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "n_layers": cfg.n_layers, "input_dim": cfg.input_dim, "batch": cfg.batch,
                   "seqlen": cfg.seqlen, "d_model": dm, "d_inner": di, "d_state": cfg.d_state,
                   "dt_rank": cfg.dt_rank, "d_conv": cfg.d_conv, "seg_len": args.seg_len or "auto",
                   "scan_states": "kept by the forward" if args.ckpt else "rebuilt",
                   "kept": "layer inputs only (activations recomputed)" if args.recompute else
                   "every layer's saved activations: " + (LAYER_SAVED_KEPT if keep_in else LAYER_SAVED_LEAN)},
        "timing": stats,
        "memory": {"kept_activations_bytes": kept_bytes, "workspace_bytes": ws.numel()},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "every product of the step (GEMM flops over the whole step time: a lower bound)",
                     "kernel_ms": round(ms, 4)},
    }


def copy_rate(warmup: int, steps: int):
    """A plain device-to-device copy of 1 GiB, `steps` times after `warmup`: 1 GiB read + 1 GiB
    written per launch.  Returns (ms per copy, GB/s of bytes read + written)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del a, b
    torch.cuda.empty_cache()
    return ms, 8 * n / (ms * 1e-3) / 1e9


def copy_probe(args):
    ms, gbps = copy_rate(args.warmup, args.steps)
    n = 1 << 28
    return {"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n, "ms_per_copy": round(ms, 4),
            "GBps": round(gbps, 1)}


# Default (warmup, steps) per workload.  The GPU comes to the timed region from
# seconds of idling while the host draws the inputs, and its first few tens of
# milliseconds of work run slower (clocks ramping up): on the mamba-370m-shaped
# scan 5 warm-up steps (4 ms) time 0.739 ms per step, 100 (70 ms) 0.665 ms, the
# same kernels.  So every workload warms up for at least ~70 ms and times at
# least ~130 ms.
BRIDGE_STEPS = 120  # mamba-130m steps queued before the headline's warm-up (about 35 ms of GPU work)
DEFAULT_STEPS = {"tiny": (100, 200), "mamba130m": (200, 400), "mamba370m": (100, 200), "mamba2p8b": (40, 80),
                 "layer": (30, 60), "backbone": (10, 20), "revscan": (500, 1000)}


def main():
    args = parse()
    w0, k0 = DEFAULT_STEPS.get(args.workload, (5, 20)) if not args.copy_probe else (5, 20)
    args.warmup = w0 if args.warmup is None else args.warmup
    args.steps = k0 if args.steps is None else args.steps
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding "
              "of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        print(json.dumps(copy_probe(args)), flush=True)
        return
    from synth import CONFIGS, BackboneConfig, LayerConfig, RecurrenceConfig
    cfg = CONFIGS[args.workload]
    all_configs = args.workload == "mamba370m" and not args.no_configs and not args.ckpt
    # the CPU baselines run first: their fork pools must not inherit a process that has used the GPU
    cpu = None
    cpu_configs = {}
    if not args.no_cpu_baseline and all_configs:
        cpu_configs = {k: (cpu_baseline_layer if k == "layer" else cpu_baseline_scan)(CONFIGS[k])
                       for k in ("mamba130m", "mamba2p8b", "layer")}
    if not args.no_cpu_baseline:
        if isinstance(cfg, LayerConfig):
            cpu = cpu_baseline_layer(cfg)
        elif isinstance(cfg, BackboneConfig):
            cpu = cpu_baseline_backbone(cfg)
        elif isinstance(cfg, RecurrenceConfig):
            cpu = cpu_baseline_recurrence(cfg)
        else:
            cpu = cpu_baseline_scan(cfg)
    # The default run uploads the inputs of the headline workload and of the two smaller ones, times
    # the two smaller ones, then the headline one, then the two larger ones.  After any idle gap, even
    # a few milliseconds of host-side clean-up between two workloads, the GPU's clocks take 20-30 ms of
    # work to settle (measured: the headline's steps go 0.79 -> 0.84 -> 0.69 ms over the first 25 after
    # a gap, and stay at 0.667 from the first one when queued right behind other work), while a
    # training loop keeps the GPU busy.  So the headline's warm-up steps are queued right behind
    # BRIDGE_STEPS steps of the mamba-130m workload (about 35 ms), with no host gap between them.
    head_step = None
    bridge = None
    configs = {}
    copy = None
    if all_configs:
        head_step = prepare_scan(args, cfg)
        small = {k: prepare_scan(args, CONFIGS[k]) for k in ("tiny", "mamba130m")}
        bridge = small["mamba130m"]
        configs = run_configs(args, ("tiny", "mamba130m"), small)
        for _ in range(BRIDGE_STEPS):
            bridge(None)
    if isinstance(cfg, BackboneConfig):
        line = run_backbone(args, cfg)
    elif isinstance(cfg, LayerConfig):
        line = run_layer(args, cfg)
    elif isinstance(cfg, RecurrenceConfig):
        line = run_recurrence(args, cfg)
    else:
        line = run_scan(args, cfg, step=head_step)
        del head_step
    if bridge is not None:
        line["timing"]["before_warmup"] = (f"{BRIDGE_STEPS} steps of the mamba-130m workload queued right before "
                                           "the warm-up, so the GPU does not idle into it")
        del bridge
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if all_configs:
        # the box's practical HBM rate, beside the published peak (after the headline: a bandwidth-bound
        # copy leaves the clocks low for the next few milliseconds of compute)
        copy = copy_rate(5, 10)[1]
    if copy is not None:
        line["hbm"]["measured_copy_GBps"] = round(copy, 1)
        line["hbm"]["frac_of_measured_copy"] = round(line["hbm"]["effective_GBps"] / copy, 4)
    if all_configs:
        configs.update(run_configs(args, ("mamba2p8b", "layer")))
        for k, v in cpu_configs.items():
            configs[k]["cpu_baseline"] = v
        line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the DeepSeek-V4 hyper-connection (HC) op on one MI355X.

One step = one whole HC op (RMS statistic, fn matvec, gates, Sinkhorn,
pre-mix, post update, coefficient store) over one batch of synthetic input
already resident in HBM, through the C ABI (ds4hc_fused). Default workload:
prefill, T = 4096 tokens, n_hc = 4, d = 4096, float32 state.

    python bench.py [--steps K] [--warmup W] [--workload prefill|stress]

Prints one JSON line. Three input sets are rotated so no step starts with its
inputs warm in the 256 MiB last-level cache. The CPU baseline is the fp64
oracle on the same workload (all host cores).
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

METRIC = "HC-op tokens/s and achieved HBM GB/s (% of peak) at T=4096, d=4096, n_hc=4"
HBM_PEAK_GBPS = 8000.0
KERNEL_NAME = {"default": "hc_tile_kernel", "tile": "hc_tile_kernel", "rowres": "hc_rowres_kernel",
               "splitk": "hc_partials_kernel+hc_finish_kernel"}
COUNTERS_FILE = {"prefill": "profiles/hc_tile_prefill_T4096_counters.json",
                 "stress": "profiles/hc_tile_stress_T16384_counters.json"}


def algorithmic_bytes(T, n, d, state_bytes, with_coeffs=True):
    """Bytes the op must move: read X and layer_out, write X' and layer_in,
    read W (f16) and bias once, write the coefficients."""
    m = 2 * n + n * n
    K = n * d
    b = T * K * state_bytes * 2 + T * d * state_bytes * 2 + m * K * 2 + m * 4
    if with_coeffs:
        b += T * m * 4
    return b


def load_traffic(workload, src_hash):
    path = os.path.join(ROOT, COUNTERS_FILE[workload])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != src_hash:
        return None
    return rec.get("traffic_bytes_per_launch")


def make_case(workload, seed):
    from deepseek_v4_hyper_amd import workloads as wl
    if workload == "prefill":
        return wl.make_prefill(seed)
    if workload == "stress":
        return wl.make_stress(seed)
    raise ValueError(workload)


def to_device(case):
    import torch
    from deepseek_v4_hyper_amd import workloads as wl

    def st(a):
        if case.dtype == wl.F32:
            return torch.from_numpy(a).cuda()
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    X = st(case.X)
    W = torch.from_numpy(case.W).cuda()
    b = torch.from_numpy(case.bias).cuda()
    lo = st(case.layer_out)
    return X, W, b, lo


def cpu_baseline(case, runs=3):
    """fp64 oracle on the full workload, all host cores; median of `runs`."""
    import oracle
    from deepseek_v4_hyper_amd import workloads as wl
    X = wl.state_to_f64(case.X, case.dtype)
    lo = wl.state_to_f64(case.layer_out, case.dtype)
    W = case.W.astype(np.float64)
    b = case.bias.astype(np.float64)
    oracle.fused(X[:8], W, b, lo[:8], case.eps, case.iters)  # load + warm
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.fused(X, W, b, lo, case.eps, case.iters)
        times.append(time.perf_counter() - t0)
    sec = float(np.median(times))
    return {"value": case.T / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"whole {case.name} workload (T={case.T}, n={case.n}, d={case.d}, "
                      f"{case.dtype}), median of {runs} runs, {sec:.3f} s each"}


def copy_calibration(nbytes=1 << 30):
    """One plain elementwise copy of known size (read nbytes, write nbytes) as
    the process's last kernel, for scaling rocprofv3 FETCH/WRITE counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    torch.mul(a, 1.0, out=b)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    print(json.dumps({"copy_calibration_bytes": nbytes, "copy_ms": ms,
                      "copy_gbps_read_plus_write": 2 * nbytes / ms / 1e6}), file=sys.stderr,
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "stress"])
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated across steps")
    ap.add_argument("--path", default="default", choices=["default", "rowres", "tile", "splitk"],
                    help="force one kernel path (default: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the HC op is per-token and shards over T "
              "with no exchange, so run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl

    B.load()
    cases = [make_case(args.workload, s) for s in range(args.sets)]
    c0 = cases[0]
    T, n, d = c0.T, c0.n, c0.d
    m = 2 * n + n * n
    sets = []
    for c in cases:
        X, W, b, lo = to_device(c)
        li = torch.empty((T, d), dtype=X.dtype, device="cuda")
        cf = torch.empty((T, m), dtype=torch.float32, device="cuda")
        xo = torch.empty_like(X)
        sets.append((X, W, b, lo, li, cf, xo))
    dt = B.DS4HC_F32 if c0.dtype == wl.F32 else B.DS4HC_BF16
    flags = {"default": 0, "rowres": B.DS4HC_FLAG_FORCE_ROWRES, "tile": B.DS4HC_FLAG_FORCE_TILE,
             "splitk": B.DS4HC_FLAG_FORCE_SPLITK}[args.path]
    params = B.make_params(n, d, c0.eps, c0.iters, flags)
    ws_bytes = B.ds4hc_workspace_bytes(params, T, dt)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptrs = [[ctypes.c_void_p(t.data_ptr()) for t in s] for s in sets]
    wsp = ctypes.c_void_p(ws.data_ptr())

    def step(i):
        X, W, b, lo, li, cf, xo = ptrs[i % len(ptrs)]
        st = B.ds4hc_fused_raw(params, T, dt, X, W, b, lo, li, cf, xo, wsp, ws_bytes, sp)
        if st != B.DS4HC_OK:
            raise B.Ds4hcError(st, "ds4hc_fused")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps

    if args.copy_calibration:
        copy_calibration()

    sb = 4 if c0.dtype == wl.F32 else 2
    alg = algorithmic_bytes(T, n, d, sb)
    achieved = alg / (ms * 1e-3) / 1e9
    from deepseek_v4_hyper_amd.counters import kernel_source_hash
    traffic = load_traffic(args.workload, kernel_source_hash()) if args.path in ("default", "tile") \
        else None
    rec = {
        "metric": METRIC if args.workload == "prefill" else
        f"HC-op tokens/s and achieved HBM GB/s at T={T}, d={d}, n_hc={n} ({c0.dtype} state)",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if c0.dtype == wl.F32 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: T={T}, n_hc={n}, d={d}, {c0.dtype} state, "
                               f"f16 fn weight [{m},{n * d}], {c0.iters} Sinkhorn iterations",
                   "entry_point": "ds4hc_fused", "path": args.path, "input_sets_rotated": len(sets),
                   "host_wall_s": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg,
                     "kernel": KERNEL_NAME[args.path]},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(c0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

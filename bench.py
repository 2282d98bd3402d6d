"""Benchmark of the DeepSeek-V4 hyper-connection (HC) op on one MI355X.

One step = one whole HC op (RMS statistic, fn matvec, gates, Sinkhorn,
pre-mix, post update, coefficient store) over one batch of synthetic input
already resident in HBM, through the C ABI (ds4hc_fused). Default workload:
prefill, T = 4096 tokens, n_hc = 4, d = 4096, float32 state.

    python bench.py [--steps K] [--warmup W] [--workload prefill|stress]

Prints one JSON line. Three input sets are rotated so no step starts with its
inputs warm in the 256 MiB last-level cache. Before the warm-up steps the op
runs for ~100 ms of wall time, so the timed steps see steady clocks however
few warm-up steps are asked for. Besides the headline figures the line holds:
the GPU's shader and memory clocks and package power cap as rocm-smi reports
them while the op runs (after the timed steps), the bandwidth of a plain
1 GiB device copy (libds4hc_bw.so) measured in the same process, and the op's
fraction of it, the per-call latency of the decode-sized workloads (T=1,
d=256 and T=4, d=4096) warm and with the caches flushed, and the CPU
baseline: the fp64 oracle on the same workload with all host cores, and with
one thread on a sample of it.
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
               "splitk": "hc_colchunk_partials_kernel+hc_finish_kernel"}
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


def cpu_info():
    """Host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, os.cpu_count(), usable


def gpu_clocks(step, seconds_max=8.0):
    """GPU clocks and package power cap as rocm-smi reports them while the op runs
    back to back (outside the timed region): {"sclk_mhz", "mclk_mhz", "power_cap_w"},
    or None where rocm-smi is missing or says nothing. rocm-smi runs as a child
    process; the op keeps the GPU busy until it has answered."""
    import shutil
    import subprocess
    import torch
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(exe):
        return None
    try:
        p = subprocess.Popen([exe, "--showclocks", "--showmaxpower", "--json"], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0, i = time.time(), 0
    while p.poll() is None and time.time() - t0 < seconds_max:
        for _ in range(50):
            step(i)
            i += 1
        torch.cuda.synchronize()
    try:
        out, _ = p.communicate(timeout=10)
    except subprocess.TimeoutExpired:
        p.kill()
        p.communicate()
        return None
    try:
        card = next(iter(json.loads(out).values()))
    except (ValueError, StopIteration, AttributeError):
        return None

    def num(key):
        v = card.get(key)
        if v is None:
            return None
        digits = "".join(ch for ch in str(v) if ch.isdigit() or ch == ".")
        return float(digits) if digits else None
    return {"sclk_mhz": num("sclk clock speed:"), "mclk_mhz": num("mclk clock speed:"),
            "power_cap_w": num("Max Graphics Package Power (W)"), "sampled": "rocm-smi during back-to-back steps"}


def _time_oracle(fn, min_runs, min_seconds, max_runs):
    times = []
    while len(times) < max_runs and (len(times) < min_runs or sum(times) < min_seconds):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def cpu_baseline(case, min_runs=3, min_seconds=5.0, max_runs=50, single_tokens=1024):
    """fp64 oracle on the host: all cores on the whole workload (the median of
    repeated runs, at least `min_runs` and until about `min_seconds` of oracle
    time), and one thread on the first `single_tokens` tokens (median of 3)."""
    import oracle
    from deepseek_v4_hyper_amd import workloads as wl
    X = wl.state_to_f64(case.X, case.dtype)
    lo = wl.state_to_f64(case.layer_out, case.dtype)
    W = case.W.astype(np.float64)
    b = case.bias.astype(np.float64)
    oracle.fused(X[:8], W, b, lo[:8], case.eps, case.iters)  # load + warm
    all_threads = oracle.num_threads()
    sec, runs = _time_oracle(lambda: oracle.fused(X, W, b, lo, case.eps, case.iters),
                             min_runs, min_seconds, max_runs)
    ts = min(single_tokens, case.T)
    oracle.set_threads(1)
    try:
        sec1, runs1 = _time_oracle(lambda: oracle.fused(X[:ts], W, b, lo[:ts], case.eps, case.iters),
                                   3, 0.0, 3)
    finally:
        oracle.set_threads(all_threads)
    model, ncpu, usable = cpu_info()
    return {"value": case.T / sec, "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": f"whole {case.name} workload (T={case.T}, n={case.n}, d={case.d}, "
                      f"{case.dtype}), median of {runs} runs, {sec:.3f} s each",
            "single_thread": {"value": ts / sec1, "unit": "tokens/s", "cores": 1,
                              "sample": f"first {ts} tokens of the same workload, median of "
                                        f"{runs1} runs, {sec1:.3f} s each"},
            "cpu_model": model, "nproc": ncpu, "usable_cpus": usable}


def copy_bandwidth(nbytes=1 << 30, reps=20):
    """A plain device copy at steady clocks (libds4hc_bw.so: 16-byte
    non-temporal loads and stores, 1 GiB): GB/s of read + write bytes, median
    over reps. The achievable bandwidth of a streaming kernel on this GPU."""
    import torch
    from deepseek_v4_hyper_amd import build_lib
    lib = ctypes.CDLL(build_lib.LIB_BW)
    lib.ds4hc_bw_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.ds4hc_bw_copy.restype = ctypes.c_int
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def copy():
        rc = lib.ds4hc_bw_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), nbytes, sp)
        if rc != 0:
            raise RuntimeError(f"ds4hc_bw_copy failed: {rc}")
    for _ in range(3):
        copy()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        copy()
        e.record(stream)
    torch.cuda.synchronize()
    if not torch.equal(a[:1024], b[:1024]) or not torch.equal(a[-1024:], b[-1024:]):
        raise RuntimeError("ds4hc_bw_copy: the copy is wrong")
    ms = float(np.median([s.elapsed_time(e) for s, e in ev]))
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def latency_records(reps=101, flush_bytes=512 << 20):
    """Microseconds per ds4hc_fused call for the two decode-sized workloads (the
    single token, T=1, d=256, and the speculative-verify batch, T=4, d=4096):
    warm (the same inputs call after call, W resident in the caches, as in a
    decode loop) and cold (a 512 MiB buffer written between calls, flushing
    the L2 and last-level caches). Each call is bracketed by its own HIP events
    on the launch stream; the median over `reps` calls is reported."""
    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = []
    for case in (wl.make_single(0), wl.make_verify(0)):
        X, W, b, lo = to_device(case)
        m = 2 * case.n + case.n * case.n
        li = torch.empty((case.T, case.d), device="cuda")
        cf = torch.empty((case.T, m), device="cuda")
        xo = torch.empty_like(X)
        params = B.make_params(case.n, case.d, case.eps, case.iters)
        wsb = B.ds4hc_workspace_bytes(params, case.T, B.DS4HC_F32)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        ptr = [ctypes.c_void_p(t.data_ptr()) for t in (X, W, b, lo, li, cf, xo, ws)]

        def call():
            st = B.ds4hc_fused_raw(params, case.T, B.DS4HC_F32, *ptr[:7], ptr[7], wsb, sp)
            if st != B.DS4HC_OK:
                raise B.Ds4hcError(st, "ds4hc_fused")
        rec = {"workload": case.name, "T": case.T, "n_hc": case.n, "d": case.d, "dtype": "f32"}
        for mode in ("warm", "cold"):
            for _ in range(10):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for s, e in ev:
                if mode == "cold":
                    flush.fill_(1.0)
                s.record(stream)
                call()
                e.record(stream)
            torch.cuda.synchronize()
            rec[f"{mode}_us"] = float(np.median([s.elapsed_time(e) for s, e in ev])) * 1e3
        out.append(rec)
    del flush
    return out


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


def warm_gpu(ms=60.0):
    """Keep the GPU busy for about `ms` milliseconds (a 256 MiB device copy in a
    loop) so that the measurements after it run at steady clocks."""
    import torch
    a = torch.empty(1 << 26, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            b.copy_(a)
        torch.cuda.synchronize()


def warm_with(step, ms=100.0, batch=20):
    """Run `step(i)` for about `ms` milliseconds of wall time: the GPU needs tens
    of milliseconds of this load to reach its steady clocks, however few
    warm-up steps the caller asks for."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(batch):
            step(i)
            i += 1
        torch.cuda.synchronize()
    return i


def sweep_paths(Ts=(1, 2, 3, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096), steps=200, warmup=20):
    """Per-call time of each kernel path of ds4hc_fused across T (the split-K / tile
    crossover), warm: the same inputs every call, as in a decode or verify loop."""
    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl
    paths = {"splitk": B.DS4HC_FLAG_FORCE_SPLITK, "tile": B.DS4HC_FLAG_FORCE_TILE,
             "rowres": B.DS4HC_FLAG_FORCE_ROWRES, "default": 0}
    for T in Ts:
        c = wl.make_verify(0, T=T)
        X, W, b, lo = to_device(c)
        li = torch.empty((T, c.d), dtype=X.dtype, device="cuda")
        m = 2 * c.n + c.n * c.n
        cf = torch.empty((T, m), dtype=torch.float32, device="cuda")
        xo = torch.empty_like(X)
        stream = torch.cuda.current_stream()
        sp = ctypes.c_void_p(stream.cuda_stream)
        for name, fl in paths.items():
            params = B.make_params(c.n, c.d, c.eps, c.iters, fl)
            wsb = B.ds4hc_workspace_bytes(params, T, B.DS4HC_F32)
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
            ptr = [ctypes.c_void_p(t.data_ptr()) for t in (X, W, b, lo, li, cf, xo, ws)]

            def call():
                st = B.ds4hc_fused_raw(params, T, B.DS4HC_F32, *ptr[:7], ptr[7], wsb, sp)
                if st != B.DS4HC_OK:
                    raise B.Ds4hcError(st, "ds4hc_fused")
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            print(json.dumps({"sweep": "ds4hc_fused", "T": T, "n_hc": c.n, "d": c.d, "dtype": "f32",
                              "path": name, "us_per_call": us, "tokens_per_s": T / (us * 1e-6)}),
                  flush=True)


def split_share(G, steps, warmup):
    """One GPU's share (d / G columns of every stream) of the prefill workload:
    ds4hc_partials on the share, then ds4hc_combine with all G shares' partials
    (the exchange itself is not timed: on one GPU the shares' partials are local)."""
    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl
    c = wl.make_prefill(0)
    T, n, d = c.T, c.n, c.d
    m = 2 * n + n * n
    ds = d // G
    X, W, b, lo = to_device(c)
    Xs = X[:, :, :ds].contiguous()
    Ws = W.reshape(m, n, d)[:, :, :ds].reshape(m, n * ds).contiguous()
    los = lo[:, :ds].contiguous()
    P = torch.stack([B.ds4hc_partials(Xs, Ws) for _ in range(G)])
    li = torch.empty((T, ds), device="cuda")
    cf = torch.empty((T, m), device="cuda")
    xo = torch.empty_like(Xs)
    # raw C-ABI calls on preallocated buffers: the binding's per-call checks in
    # Python would otherwise set the pace of these ~10-30 us kernels
    ps = B.make_params(n, ds)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pt = lambda t: ctypes.c_void_p(t.data_ptr())
    wsb = B.ds4hc_partials_workspace_bytes(ps, T, B.DS4HC_F32)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    a_part = (pt(Xs), pt(Ws), pt(P[0]), pt(ws))
    a_comb = (pt(P), pt(b), pt(Xs), pt(los), pt(li), pt(cf), pt(xo))

    def part():
        st = B.ds4hc_partials_raw(ps, T, B.DS4HC_F32, a_part[0], a_part[1], a_part[2], a_part[3], wsb, sp)
        if st != B.DS4HC_OK:
            raise B.Ds4hcError(st, "ds4hc_partials")

    def comb():
        st = B.ds4hc_combine_raw(ps, d, T, B.DS4HC_F32, G, *a_comb, sp)
        if st != B.DS4HC_OK:
            raise B.Ds4hcError(st, "ds4hc_combine")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("partials", part), ("combine", comb)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / steps
    # bytes one share must move: partials reads X_s and W_s, writes [T, m+1]; combine reads
    # the G partials, X_s and layer_out_s, writes X'_s, layer_in_s and the coefficients
    bp = T * n * ds * 4 + m * n * ds * 2 + T * (m + 1) * 4
    bc = G * T * (m + 1) * 4 + 2 * T * n * ds * 4 + 2 * T * ds * 4 + T * m * 4
    for name, by in (("partials", bp), ("combine", bc)):
        print(json.dumps({"split_d": G, "share_columns": ds, "T": T, "n_hc": n, "d": d, "dtype": "f32",
                          "kernel": name, "us": res[name], "algorithmic_bytes": by,
                          "GB_per_s": by / (res[name] * 1e-6) / 1e9}), flush=True)
    tot = res["partials"] + res["combine"]
    print(json.dumps({"split_d": G, "share_columns": ds, "T": T, "kernel": "share total", "us": tot,
                      "tokens_per_s_per_share": T / (tot * 1e-6),
                      "GB_per_s": (bp + bc) / (tot * 1e-6) / 1e9}), flush=True)


def decode_chain(sites=86, d=4096, n=4, reps=50):
    """Decode-token chain of `sites` HC sites (attention and FFN per layer, 43 layers),
    T = 1, each site with its own f16 weight; the layer body is the stand-in
    layer_out = 0.5 * layer_in + noise (one elementwise kernel). Variants: two
    library calls per site (ds4hc_pre ... ds4hc_post) or one (ds4hc_post_pre at
    every boundary); each run eagerly and as one captured HIP graph. Prints one
    JSON line per variant: microseconds per site and per token."""
    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl
    m = 2 * n + n * n
    rng = np.random.Generator(np.random.PCG64(0))
    X0 = torch.from_numpy(rng.standard_normal((1, n, d), dtype=np.float32)).cuda()
    Ws = [torch.from_numpy((rng.standard_normal((m, n * d), dtype=np.float32) * 0.02)
                           .astype(np.float16)).cuda() for _ in range(sites)]
    noise = torch.from_numpy(rng.standard_normal((sites, 1, d), dtype=np.float32) * 0.1).cuda()
    bias = torch.zeros(m, dtype=torch.float32, device="cuda")
    Xa, Xb = torch.empty_like(X0), torch.empty_like(X0)
    li = torch.empty((1, d), device="cuda")
    lo = torch.empty((1, d), device="cuda")
    cf = [torch.empty((1, m), device="cuda") for _ in range(2)]
    p = B.make_params(n, d)
    wsb = max(B.ds4hc_workspace_bytes(p, 1, B.DS4HC_F32), B.ds4hc_post_pre_workspace_bytes(p, 1, B.DS4HC_F32))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p
    pt = lambda t: P(t.data_ptr())

    def chk(st, what):
        if st != B.DS4HC_OK:
            raise B.Ds4hcError(st, what)

    def run(one_pass):
        sp = P(torch.cuda.current_stream().cuda_stream)
        Xa.copy_(X0)
        cur, nxt = Xa, Xb
        chk(B.ds4hc_pre_raw(p, 1, 0, pt(cur), pt(Ws[0]), pt(bias), pt(li), pt(cf[0]), None, pt(ws),
                            wsb, sp), "pre")
        for s_ in range(sites):
            torch.add(noise[s_], li, alpha=0.5, out=lo)
            c_now, c_next = cf[s_ % 2], cf[(s_ + 1) % 2]
            if s_ + 1 < sites and one_pass:
                chk(B.ds4hc_post_pre_raw(p, 1, 0, pt(cur), pt(c_now), pt(lo), pt(Ws[s_ + 1]), pt(bias),
                                         pt(nxt), pt(li), pt(c_next), None, pt(ws), wsb, sp), "post_pre")
            else:
                chk(B.ds4hc_post_raw(p, 1, 0, pt(cur), pt(c_now), pt(lo), pt(nxt), sp), "post")
                if s_ + 1 < sites:
                    chk(B.ds4hc_pre_raw(p, 1, 0, pt(nxt), pt(Ws[s_ + 1]), pt(bias), pt(li), pt(c_next),
                                        None, pt(ws), wsb, sp), "pre")
            cur, nxt = nxt, cur
        return cur

    results = {}
    for one_pass in (False, True):
        for _ in range(3):
            out = run(one_pass)
        torch.cuda.synchronize()
        ref = out.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run(one_pass)
        e1.record()
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / reps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gout = run(one_pass)
        # replays, each checked against the eager result with eager work in between
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(gout, ref):
                raise RuntimeError("graph replay differs from the eager chain")
            run(one_pass)
            torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / reps
        name = "post_pre" if one_pass else "pre+post"
        results[name] = (eager_us, graph_us)
        for mode, us in (("eager", eager_us), ("graph", graph_us)):
            print(json.dumps({"chain": "decode", "sites": sites, "T": 1, "n_hc": n, "d": d, "dtype": "f32",
                              "calls_per_site": 1 if one_pass else 2, "variant": name, "mode": mode,
                              "us_per_token": us, "us_per_site": us / sites}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU reaches its steady clocks only after ~30 ms of this load: with 10
    # warm-up steps the timed average of the prefill step read 167.8 us, with
    # 200 it reads 157.0 us (the same kernel). 200 + 300 steps take ~0.1 s.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "stress"])
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated across steps")
    ap.add_argument("--path", default="default", choices=["default", "rowres", "tile", "splitk"],
                    help="force one kernel path (default: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the copy-bandwidth and decode-latency measurements")
    ap.add_argument("--warm-ms", type=float, default=100.0,
                    help="milliseconds of untimed steps before the warm-up steps (steady clocks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for counter scaling)")
    ap.add_argument("--chain", action="store_true",
                    help="instead of the benchmark line: the 86-site decode chain (T=1, n=4, d=4096, "
                         "fp32), eager and HIP-graph replay, two calls per site vs one-pass post+pre")
    ap.add_argument("--split-d", type=int, default=0, metavar="G",
                    help="instead of the benchmark line: one GPU's share of a split over d into G "
                         "column shares at the prefill shape: ds4hc_partials and ds4hc_combine timed")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line: time every kernel path of ds4hc_fused over "
                         "T = 1..4096 (verify recipe, n=4, d=4096, fp32), one JSON line per (T, path)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the HC op is per-token and shards over T "
              "with no exchange, so run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from deepseek_v4_hyper_amd import binding as B
    from deepseek_v4_hyper_amd import workloads as wl

    B.load()
    if args.sweep:
        warm_gpu()
        sweep_paths()
        return
    if args.chain:
        warm_gpu()
        decode_chain()
        return
    if args.split_d:
        warm_gpu()
        split_share(args.split_d, args.steps, args.warmup)
        return
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

    # time-based warm-up first (steady clocks), then the requested warm-up steps
    warm_with(step, args.warm_ms)
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

    extras = {}
    if not args.no_extras:
        extras["clocks"] = gpu_clocks(step)
        extras["copy_gbps"] = copy_bandwidth()
        extras["latency"] = latency_records()
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
    if "copy_gbps" in extras:
        rec["roofline"]["copy_gbps"] = extras["copy_gbps"]
        rec["roofline"]["frac_of_copy"] = achieved / extras["copy_gbps"]
        rec["latency_us"] = extras["latency"]
        rec["gpu_clocks"] = extras["clocks"]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(c0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

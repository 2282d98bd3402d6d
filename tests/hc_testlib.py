"""Shared helpers for the GPU tests: moving seeded cases to the device,
reading results back as float64, and the per-row normwise error metric.

Error metric (one number per token row t):
    e_t = max|Y_gpu[t] - Y_ref[t]| / max|Y_ref[t]|,
with an all-zero reference row required to be exactly zero. Elementwise
relative error is meaningless here: outputs near zero come from
cancellation. Tolerances: 2e-5 for float32 state, 1e-2 for bfloat16 state
(bf16's unit roundoff is 2^-8 = 3.9e-3 and the GPU rounds once);
coefficients (values in [0, 1]) within 2e-5 absolute.
"""
from __future__ import annotations

import sys

import numpy as np

from deepseek_v4_hyper_amd import workloads as wl

TOL = {wl.F32: 2e-5, wl.BF16: 1e-2}
COEFF_TOL = 2e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def state_to_torch(a, dtype, device="cuda"):
    import torch
    if dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    bits = np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16)


def torch_to_f64(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return wl.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def case_to_device(case, device="cuda"):
    import torch
    X = state_to_torch(case.X, case.dtype, device)
    W = torch.from_numpy(np.ascontiguousarray(case.W, dtype=np.float16)).to(device)
    b = torch.from_numpy(np.ascontiguousarray(case.bias, dtype=np.float32)).to(device)
    lo = None if case.layer_out is None else state_to_torch(case.layer_out, case.dtype, device)
    return X, W, b, lo


def rowwise_err(got, ref):
    """Max over rows of the normwise error; rows are the leading axis."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    assert got.shape == ref.shape
    scale = np.abs(ref).max(axis=1)
    diff = np.abs(got - ref).max(axis=1)
    zero = scale == 0
    if np.any(zero & (diff != 0)):
        return float("inf")
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.where(zero, 0.0, diff / np.where(zero, 1.0, scale))
    if np.any(np.isnan(e)):
        return float("inf")
    return float(e.max()) if len(e) else 0.0


def assert_close_rows(got, ref, tol, what):
    e = rowwise_err(got, ref)
    assert e <= tol, f"{what}: max row normwise error {e:.3e} > {tol:.1e}"
    return e


def assert_coeffs(got, ref, what="coeffs"):
    d = float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max()) \
        if np.size(ref) else 0.0
    assert d <= COEFF_TOL, f"{what}: max abs error {d:.3e} > {COEFF_TOL:.0e}"
    return d

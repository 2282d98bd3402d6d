"""fp64 CPU oracle of the DeepSeek-V4 hyper-connection (HC) op.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this; the HIP library and its Python
binding never do. The arithmetic lives in ``ds4hc_oracle.c`` (plain C, IEEE
double, ascending-index sums); this module only widens inputs to float64 and
calls it through ctypes.

Parity pins (what checks the oracle against something other than itself) are
in ``tests/test_oracle_pins.py``. The op's readings, and the passages of the
lucebox pages they rest on, are listed at the top of ``ds4hc_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ds4hc_oracle.c")
_SO = os.path.join(_HERE, "libds4hc_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE, OpenMP over tokens)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
                               "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, ci, cd = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.ds4hc_oracle_pre.argtypes = [i64, ci, ci, _D, _D, _D, cd, ci, _D, _D, _D]
        lib.ds4hc_oracle_sinkhorn.argtypes = [i64, ci, ci, _D, _D]
        lib.ds4hc_oracle_post.argtypes = [i64, ci, ci, _D, _D, _D, _D]
        lib.ds4hc_oracle_fused.argtypes = [i64, ci, ci, _D, _D, _D, _D, cd, ci, _D, _D, _D]
        lib.ds4hc_oracle_partials.argtypes = [i64, ci, ci, _D, _D, _D]
        for f in ("pre", "sinkhorn", "post", "fused", "partials"):
            getattr(lib, "ds4hc_oracle_" + f).restype = ci
        lib.ds4hc_oracle_num_threads.restype = ci
        lib.ds4hc_oracle_set_threads.argtypes = [ci]
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(_D) if a is not None else None


def num_threads() -> int:
    return _load().ds4hc_oracle_num_threads()


def set_threads(n: int) -> None:
    _load().ds4hc_oracle_set_threads(int(n))


def n_logits(n: int) -> int:
    return 2 * n + n * n


def pre(X, W, b, eps=1e-6, iters=20):
    """HC-pre (RMS norm, fn matvec, gates, Sinkhorn, pre-mix).

    X [T, n, d], W [2n+n*n, n*d], b [2n+n*n]; any real dtype (widened exactly).
    Returns (layer_in [T, d], coeffs [T, m] = pre|post|H row-major, logits [T, m]).
    """
    X, W, b = _f64(X), _f64(W), _f64(b)
    T, n, d = X.shape
    m = n_logits(n)
    assert W.shape == (m, n * d) and b.shape == (m,)
    layer_in = np.empty((T, d))
    coeffs = np.empty((T, m))
    logits = np.empty((T, m))
    rc = _load().ds4hc_oracle_pre(T, n, d, _p(X), _p(W), _p(b), float(eps), int(iters),
                                  _p(layer_in), _p(coeffs), _p(logits))
    if rc:
        raise ValueError("ds4hc_oracle_pre rejected its arguments")
    return layer_in, coeffs, logits


def sinkhorn(logits_res, iters=20):
    """Max-subtracted exp then `iters` x (row, column) normalisation. [T, n, n] -> [T, n, n]."""
    Z = _f64(logits_res)
    T, n, n2 = Z.shape
    assert n == n2
    H = np.empty_like(Z)
    if _load().ds4hc_oracle_sinkhorn(T, n, int(iters), _p(Z), _p(H)):
        raise ValueError("ds4hc_oracle_sinkhorn rejected its arguments")
    return H


def post(X, coeffs, layer_out):
    """hc_post: X'[i] = sum_j H[i][j] X[j] + post_i * layer_out. Returns [T, n, d]."""
    X, coeffs, layer_out = _f64(X), _f64(coeffs), _f64(layer_out)
    T, n, d = X.shape
    assert coeffs.shape == (T, n_logits(n)) and layer_out.shape == (T, d)
    out = np.empty_like(X)
    if _load().ds4hc_oracle_post(T, n, d, _p(X), _p(coeffs), _p(layer_out), _p(out)):
        raise ValueError("ds4hc_oracle_post rejected its arguments")
    return out


def fused(X, W, b, layer_out, eps=1e-6, iters=20):
    """Whole op. Returns (layer_in [T, d], coeffs [T, m], X_out [T, n, d])."""
    X, W, b, layer_out = _f64(X), _f64(W), _f64(b), _f64(layer_out)
    T, n, d = X.shape
    m = n_logits(n)
    layer_in = np.empty((T, d))
    coeffs = np.empty((T, m))
    out = np.empty_like(X)
    rc = _load().ds4hc_oracle_fused(T, n, d, _p(X), _p(W), _p(b), _p(layer_out), float(eps),
                                    int(iters), _p(layer_in), _p(coeffs), _p(out))
    if rc:
        raise ValueError("ds4hc_oracle_fused rejected its arguments")
    return layer_in, coeffs, out


def partials(X_share, W_share):
    """Split-over-d partial sums of one column share: X_share [T, n, ds],
    W_share [m, n*ds]. Returns [T, m+1]: the unnormalised fn dots, then the sum of squares."""
    X, W = _f64(X_share), _f64(W_share)
    T, n, ds = X.shape
    m = n_logits(n)
    assert W.shape == (m, n * ds)
    out = np.empty((T, m + 1))
    if _load().ds4hc_oracle_partials(T, n, ds, _p(X), _p(W), _p(out)):
        raise ValueError("ds4hc_oracle_partials rejected its arguments")
    return out


def chain(X0, Ws, b, noise, eps=1e-6, iters=20, layer_scale=0.5):
    """Decode chain: per layer, HC-pre, a stand-in layer body
    layer_out = layer_scale * layer_in + noise[l], then hc_post.

    Returns the list of states [X_0, X_1, ..., X_L] (float64)."""
    X = _f64(X0)
    states = [X]
    for l, W in enumerate(Ws):
        layer_in, coeffs, _ = pre(X, W, b, eps, iters)
        layer_out = layer_scale * layer_in + _f64(noise[l])[None, :]
        X = post(X, coeffs, layer_out)
        states.append(X)
    return states

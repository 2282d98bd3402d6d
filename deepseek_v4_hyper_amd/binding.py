"""ctypes binding of libds4hc.so (include/ds4hc.h).

Argument marshalling only: each Python function checks tensor shapes/dtypes,
passes device pointers and the current HIP stream to the C function of the
same name, and turns a non-OK status into an exception. Every step of the op
runs in the library's HIP kernels; PyTorch only provides device memory and
the stream. There is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libds4hc.so")

DS4HC_OK = 0
DS4HC_ERR_INVALID_ARG = 1
DS4HC_ERR_UNSUPPORTED = 2
DS4HC_ERR_HIP = 3
DS4HC_F32 = 0
DS4HC_BF16 = 1
DS4HC_FLAG_DETERMINISTIC = 1
DS4HC_FLAG_FORCE_ROWRES = 2
DS4HC_FLAG_FORCE_SPLITK = 4
DS4HC_FLAG_FORCE_TILE = 8

EXPORTED = ("ds4hc_pre", "ds4hc_sinkhorn", "ds4hc_post", "ds4hc_fused", "ds4hc_workspace_bytes",
            "ds4hc_post_pre", "ds4hc_post_pre_workspace_bytes", "ds4hc_post_pre_noalloc",
            "ds4hc_partials", "ds4hc_partials_workspace_bytes", "ds4hc_combine",
            "ds4hc_status_string", "ds4hc_last_hip_error", "ds4hc_abi_version")


class Ds4hcError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where} failed: {status_string(status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


class Params(ctypes.Structure):
    _fields_ = [("n_hc", ctypes.c_int32), ("d", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("sinkhorn_iters", ctypes.c_int32), ("flags", ctypes.c_uint32)]


def make_params(n_hc: int, d: int, rms_eps: float = 1e-6, sinkhorn_iters: int = 20,
                flags: int = 0) -> Params:
    return Params(int(n_hc), int(d), float(rms_eps), int(sinkhorn_iters), int(flags))


_lib = None


def load(path: str = LIB_PATH):
    """Load libds4hc.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libds4hc.so not found at {path}; build it with "
                           "`python -m deepseek_v4_hyper_amd.build_lib`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Params)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.ds4hc_pre.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ds4hc_sinkhorn.argtypes = [i64, i32, i32, vp, vp, vp]
    lib.ds4hc_post.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.ds4hc_fused.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ds4hc_post_pre.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ds4hc_post_pre_noalloc.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ds4hc_partials.argtypes = [P, i64, ctypes.c_int, vp, vp, vp, vp, sz, vp]
    lib.ds4hc_combine.argtypes = [P, i32, i64, ctypes.c_int, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    for f in ("ds4hc_pre", "ds4hc_sinkhorn", "ds4hc_post", "ds4hc_fused", "ds4hc_post_pre",
              "ds4hc_post_pre_noalloc", "ds4hc_partials", "ds4hc_combine"):
        getattr(lib, f).restype = ctypes.c_int
    for f in ("ds4hc_workspace_bytes", "ds4hc_post_pre_workspace_bytes",
              "ds4hc_partials_workspace_bytes"):
        getattr(lib, f).argtypes = [P, i64, ctypes.c_int]
        getattr(lib, f).restype = sz
    lib.ds4hc_status_string.argtypes = [ctypes.c_int]
    lib.ds4hc_status_string.restype = ctypes.c_char_p
    lib.ds4hc_last_hip_error.restype = ctypes.c_char_p
    lib.ds4hc_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().ds4hc_status_string(int(status)).decode()
    except Exception:
        return f"status {status}"


def abi_version() -> int:
    return load().ds4hc_abi_version()


def _check(status: int, where: str):
    if status != DS4HC_OK:
        detail = load().ds4hc_last_hip_error().decode() if status == DS4HC_ERR_HIP else ""
        raise Ds4hcError(status, where, detail)


# ------------------------------------------------------------------ raw pointer calls

def ds4hc_workspace_bytes(params: Params, T: int, dtype: int) -> int:
    return int(load().ds4hc_workspace_bytes(ctypes.byref(params), int(T), int(dtype)))


def ds4hc_post_pre_workspace_bytes(params: Params, T: int, dtype: int) -> int:
    return int(load().ds4hc_post_pre_workspace_bytes(ctypes.byref(params), int(T), int(dtype)))


def ds4hc_post_pre_raw(params, T, dtype, X, coeffs_prev, layer_out, W_next, bias_next, X_out,
                       layer_in, coeffs, logits, ws, ws_bytes, stream):
    return load().ds4hc_post_pre(ctypes.byref(params), int(T), int(dtype), X, coeffs_prev,
                                 layer_out, W_next, bias_next, X_out, layer_in, coeffs, logits, ws,
                                 int(ws_bytes), stream)


NOALLOC_SCRATCH_BYTES = 2 << 20   # DS4HC_NOALLOC_SCRATCH_BYTES


def ds4hc_post_pre_noalloc_raw(params, T, dtype, X, coeffs_prev, layer_out, W_next, bias_next,
                               X_out, layer_in, coeffs, logits, stream):
    return load().ds4hc_post_pre_noalloc(ctypes.byref(params), int(T), int(dtype), X, coeffs_prev,
                                         layer_out, W_next, bias_next, X_out, layer_in, coeffs,
                                         logits, stream)


def ds4hc_pre_raw(params, T, dtype, X, W, bias, layer_in, coeffs, logits, ws, ws_bytes, stream):
    return load().ds4hc_pre(ctypes.byref(params), int(T), int(dtype), X, W, bias, layer_in,
                            coeffs, logits, ws, int(ws_bytes), stream)


def ds4hc_fused_raw(params, T, dtype, X, W, bias, layer_out, layer_in, coeffs, X_out, ws,
                    ws_bytes, stream):
    return load().ds4hc_fused(ctypes.byref(params), int(T), int(dtype), X, W, bias, layer_out,
                              layer_in, coeffs, X_out, ws, int(ws_bytes), stream)


def ds4hc_post_raw(params, T, dtype, X, coeffs, layer_out, X_out, stream):
    return load().ds4hc_post(ctypes.byref(params), int(T), int(dtype), X, coeffs, layer_out,
                             X_out, stream)


def ds4hc_sinkhorn_raw(T, n_hc, iters, logits_res, H, stream):
    return load().ds4hc_sinkhorn(int(T), int(n_hc), int(iters), logits_res, H, stream)


def ds4hc_partials_workspace_bytes(params: Params, T: int, dtype: int) -> int:
    return int(load().ds4hc_partials_workspace_bytes(ctypes.byref(params), int(T), int(dtype)))


def ds4hc_partials_raw(params, T, dtype, X_share, W_share, partials, ws, ws_bytes, stream):
    return load().ds4hc_partials(ctypes.byref(params), int(T), int(dtype), X_share, W_share,
                                 partials, ws, int(ws_bytes), stream)


def ds4hc_combine_raw(params, d_total, T, dtype, G, partials, bias, X_share, layer_out_share,
                      layer_in_share, coeffs, X_out_share, stream):
    return load().ds4hc_combine(ctypes.byref(params), int(d_total), int(T), int(dtype), int(G),
                                partials, bias, X_share, layer_out_share, layer_in_share, coeffs,
                                X_out_share, stream)


# ------------------------------------------------------------------ torch-tensor calls

def _torch():
    import torch
    return torch


def _state_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DS4HC_F32
    if t.dtype == torch.bfloat16:
        return DS4HC_BF16
    raise TypeError(f"state dtype must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the binding allocates what it passes to a call on `stream`.

    The caching allocator ties a block to the stream that was current when it
    was allocated, and hands it out again once it is freed with no regard for
    work still queued on other streams. Buffers the binding creates (workspace,
    default outputs) are therefore allocated with the kernels' own stream
    current: a workspace dropped on return is then reused only by work ordered
    after the kernels that read it."""
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _empty(shape, dtype, device):
    return _torch().empty(shape, dtype=dtype, device=device)


def _scratch(need, workspace, device):
    """The caller's workspace, or a fresh one of `need` bytes (none if 0)."""
    if workspace is None and need:
        workspace = _empty(need, _torch().uint8, device)
    return workspace, (workspace.numel() * workspace.element_size() if workspace is not None else 0)


def ds4hc_pre(X, W, bias, *, rms_eps=1e-6, sinkhorn_iters=20, flags=0, layer_in=None,
              coeffs=None, logits=None, workspace=None, stream=None, want_logits=False):
    """HC-pre. X [T, n, d] (float32|bfloat16), W [m, n*d] float16, bias [m] float32.
    Returns (layer_in [T, d], coeffs [T, m], logits [T, m] or None)."""
    torch = _torch()
    T, n, d = X.shape
    m = 2 * n + n * n
    dt = _state_code(X)
    p = make_params(n, d, rms_eps, sinkhorn_iters, flags)
    _need(X, (T, n, d), X.dtype, "X")
    _need(W, (m, n * d), torch.float16, "W")
    _need(bias, (m,), torch.float32, "bias")
    with _on(stream):
        if layer_in is None:
            layer_in = _empty((T, d), X.dtype, X.device)
        if coeffs is None:
            coeffs = _empty((T, m), torch.float32, X.device)
        if logits is None and want_logits:
            logits = _empty((T, m), torch.float32, X.device)
        workspace, ws_bytes = _scratch(ds4hc_workspace_bytes(p, T, dt), workspace, X.device)
    _check(ds4hc_pre_raw(p, T, dt, _ptr(X), _ptr(W), _ptr(bias), _ptr(layer_in), _ptr(coeffs),
                         _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)), "ds4hc_pre")
    return layer_in, coeffs, logits


def ds4hc_fused(X, W, bias, layer_out, *, rms_eps=1e-6, sinkhorn_iters=20, flags=0,
                layer_in=None, coeffs=None, X_out=None, workspace=None, stream=None,
                want_coeffs=True):
    """Whole HC op. Returns (layer_in [T, d], coeffs [T, m] or None, X_out [T, n, d])."""
    torch = _torch()
    T, n, d = X.shape
    m = 2 * n + n * n
    dt = _state_code(X)
    p = make_params(n, d, rms_eps, sinkhorn_iters, flags)
    _need(X, (T, n, d), X.dtype, "X")
    _need(W, (m, n * d), torch.float16, "W")
    _need(bias, (m,), torch.float32, "bias")
    _need(layer_out, (T, d), X.dtype, "layer_out")
    with _on(stream):
        if layer_in is None:
            layer_in = _empty((T, d), X.dtype, X.device)
        if coeffs is None and want_coeffs:
            coeffs = _empty((T, m), torch.float32, X.device)
        if X_out is None:
            X_out = _empty(X.shape, X.dtype, X.device)
        workspace, ws_bytes = _scratch(ds4hc_workspace_bytes(p, T, dt), workspace, X.device)
    _check(ds4hc_fused_raw(p, T, dt, _ptr(X), _ptr(W), _ptr(bias), _ptr(layer_out),
                           _ptr(layer_in), _ptr(coeffs), _ptr(X_out), _ptr(workspace), ws_bytes,
                           _stream(stream)), "ds4hc_fused")
    return layer_in, coeffs, X_out


def ds4hc_post(X, coeffs, layer_out, *, X_out=None, stream=None, rms_eps=1e-6,
               sinkhorn_iters=20):
    """hc_post: X' = H.X + post (x) layer_out. X_out may be X itself (in place)."""
    torch = _torch()
    T, n, d = X.shape
    m = 2 * n + n * n
    dt = _state_code(X)
    p = make_params(n, d, rms_eps, sinkhorn_iters, 0)
    _need(X, (T, n, d), X.dtype, "X")
    _need(coeffs, (T, m), torch.float32, "coeffs")
    _need(layer_out, (T, d), X.dtype, "layer_out")
    with _on(stream):
        if X_out is None:
            X_out = _empty(X.shape, X.dtype, X.device)
    _check(ds4hc_post_raw(p, T, dt, _ptr(X), _ptr(coeffs), _ptr(layer_out), _ptr(X_out),
                          _stream(stream)), "ds4hc_post")
    return X_out


def ds4hc_post_pre(X, coeffs_prev, layer_out, W_next, bias_next, *, rms_eps=1e-6,
                   sinkhorn_iters=20, flags=0, X_out=None, layer_in=None, coeffs=None,
                   logits=None, workspace=None, stream=None, want_logits=False):
    """post(l) then pre(l+1): X' = H_l.X + post_l (x) layer_out_l, then HC-pre of
    site l+1 on X'. Returns (X_out [T,n,d], layer_in [T,d], coeffs [T,m], logits or None).
    X_out may be X itself (in place)."""
    torch = _torch()
    T, n, d = X.shape
    m = 2 * n + n * n
    dt = _state_code(X)
    p = make_params(n, d, rms_eps, sinkhorn_iters, flags)
    _need(X, (T, n, d), X.dtype, "X")
    _need(coeffs_prev, (T, m), torch.float32, "coeffs_prev")
    _need(layer_out, (T, d), X.dtype, "layer_out")
    _need(W_next, (m, n * d), torch.float16, "W_next")
    _need(bias_next, (m,), torch.float32, "bias_next")
    with _on(stream):
        if X_out is None:
            X_out = _empty(X.shape, X.dtype, X.device)
        if layer_in is None:
            layer_in = _empty((T, d), X.dtype, X.device)
        if coeffs is None:
            coeffs = _empty((T, m), torch.float32, X.device)
        if logits is None and want_logits:
            logits = _empty((T, m), torch.float32, X.device)
        workspace, ws_bytes = _scratch(ds4hc_post_pre_workspace_bytes(p, T, dt), workspace,
                                       X.device)
    _check(ds4hc_post_pre_raw(p, T, dt, _ptr(X), _ptr(coeffs_prev), _ptr(layer_out), _ptr(W_next),
                              _ptr(bias_next), _ptr(X_out), _ptr(layer_in), _ptr(coeffs),
                              _ptr(logits), _ptr(workspace), ws_bytes, _stream(stream)),
           "ds4hc_post_pre")
    return X_out, layer_in, coeffs, logits


def ds4hc_partials(X_share, W_share, *, flags=0, partials=None, workspace=None, stream=None):
    """One column share: X_share [T, n, d_s], W_share [m, n*d_s] -> partials [T, m+1]
    (unnormalised fn dots, then the sum of squares)."""
    torch = _torch()
    T, n, ds = X_share.shape
    m = 2 * n + n * n
    dt = _state_code(X_share)
    p = make_params(n, ds, 1e-6, 20, flags)
    _need(X_share, (T, n, ds), X_share.dtype, "X_share")
    _need(W_share, (m, n * ds), torch.float16, "W_share")
    with _on(stream):
        if partials is None:
            partials = _empty((T, m + 1), torch.float32, X_share.device)
        workspace, ws_bytes = _scratch(ds4hc_partials_workspace_bytes(p, T, dt), workspace,
                                       X_share.device)
    _check(ds4hc_partials_raw(p, T, dt, _ptr(X_share), _ptr(W_share), _ptr(partials),
                              _ptr(workspace), ws_bytes, _stream(stream)), "ds4hc_partials")
    return partials


def ds4hc_combine(partials, bias, X_share, layer_out_share, d_total, *, rms_eps=1e-6,
                  sinkhorn_iters=20, coeffs=None, want_coeffs=True, layer_in_share=None,
                  X_out_share=None, stream=None):
    """partials [G, T, m+1] of all shares -> (layer_in_share, coeffs or None, X_out_share)."""
    torch = _torch()
    T, n, ds = X_share.shape
    m = 2 * n + n * n
    G = partials.shape[0]
    dt = _state_code(X_share)
    p = make_params(n, ds, rms_eps, sinkhorn_iters, 0)
    _need(partials, (G, T, m + 1), torch.float32, "partials")
    _need(bias, (m,), torch.float32, "bias")
    _need(X_share, (T, n, ds), X_share.dtype, "X_share")
    _need(layer_out_share, (T, ds), X_share.dtype, "layer_out_share")
    with _on(stream):
        if layer_in_share is None:
            layer_in_share = _empty((T, ds), X_share.dtype, X_share.device)
        if coeffs is None and want_coeffs:
            coeffs = _empty((T, m), torch.float32, X_share.device)
        if X_out_share is None:
            X_out_share = _empty(X_share.shape, X_share.dtype, X_share.device)
    _check(ds4hc_combine_raw(p, d_total, T, dt, G, _ptr(partials), _ptr(bias), _ptr(X_share),
                             _ptr(layer_out_share), _ptr(layer_in_share), _ptr(coeffs),
                             _ptr(X_out_share), _stream(stream)), "ds4hc_combine")
    return layer_in_share, coeffs, X_out_share


def ds4hc_sinkhorn(logits_res, *, iters=20, H=None, stream=None):
    """Sinkhorn of residual logits [T, n, n] float32 -> H [T, n, n]."""
    torch = _torch()
    T, n, n2 = logits_res.shape
    _need(logits_res, (T, n, n), torch.float32, "logits_res")
    with _on(stream):
        if H is None:
            H = _empty(logits_res.shape, torch.float32, logits_res.device)
    _check(ds4hc_sinkhorn_raw(T, n, iters, _ptr(logits_res), _ptr(H), _stream(stream)),
           "ds4hc_sinkhorn")
    return H


def ds4hc_post_pre_noalloc(X, coeffs_prev, layer_out, W_next, bias_next, X_out, layer_in, coeffs,
                           *, logits=None, rms_eps=1e-6, sinkhorn_iters=20, flags=0, stream=None):
    """ds4hc_post_pre with the library's device-resident scratch instead of a
    workspace. Every output is the caller's (this function allocates nothing)."""
    torch = _torch()
    T, n, d = X.shape
    m = 2 * n + n * n
    dt = _state_code(X)
    p = make_params(n, d, rms_eps, sinkhorn_iters, flags)
    _need(X, (T, n, d), X.dtype, "X")
    _need(coeffs_prev, (T, m), torch.float32, "coeffs_prev")
    _need(layer_out, (T, d), X.dtype, "layer_out")
    _need(W_next, (m, n * d), torch.float16, "W_next")
    _need(bias_next, (m,), torch.float32, "bias_next")
    _need(X_out, (T, n, d), X.dtype, "X_out")
    _need(layer_in, (T, d), X.dtype, "layer_in")
    _need(coeffs, (T, m), torch.float32, "coeffs")
    if logits is not None:
        _need(logits, (T, m), torch.float32, "logits")
    _check(ds4hc_post_pre_noalloc_raw(p, T, dt, _ptr(X), _ptr(coeffs_prev), _ptr(layer_out),
                                      _ptr(W_next), _ptr(bias_next), _ptr(X_out), _ptr(layer_in),
                                      _ptr(coeffs), _ptr(logits), _stream(stream)),
           "ds4hc_post_pre_noalloc")
    return X_out, layer_in, coeffs, logits

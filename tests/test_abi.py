"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, and rejects bad arguments on the host before any
HIP call (a rejected call enqueues nothing).

The argument-validation tests pass fake (never dereferenced) device
addresses, so they only run where no GPU is visible: there, even a
validation bug could not launch a kernel on them.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from deepseek_v4_hyper_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation runs without a GPU")


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(ds4hc_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("ds4hc_pre", "ds4hc_sinkhorn", "ds4hc_post", "ds4hc_fused"):
        assert want in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_status_strings():
    assert B.abi_version() == 1
    assert B.status_string(0) == "DS4HC_OK"
    assert B.status_string(1) == "DS4HC_ERR_INVALID_ARG"
    assert B.status_string(2) == "DS4HC_ERR_UNSUPPORTED"
    assert B.status_string(3) == "DS4HC_ERR_HIP"
    assert B.load().ds4hc_last_hip_error() == b""


def test_workspace_bytes_is_pure_and_path_dependent():
    p = B.make_params(4, 4096)
    # T up to 160 takes the split-K path: column chunks of 16 lanes x V columns of
    # every stream (32 lanes where 16 would give more than 64 chunks), chunks * T *
    # (m + 1) floats
    P = 4096 // 64
    assert B.ds4hc_workspace_bytes(p, 1, B.DS4HC_F32) == P * 1 * 25 * 4
    assert B.ds4hc_workspace_bytes(p, 4, B.DS4HC_F32) == P * 4 * 25 * 4
    Pb = 4096 // 128
    assert B.ds4hc_workspace_bytes(p, 4, B.DS4HC_BF16) == Pb * 4 * 25 * 4
    assert B.ds4hc_workspace_bytes(B.make_params(4, 7168), 2, B.DS4HC_F32) == (7168 // 128) * 2 * 25 * 4
    ps = B.make_params(2, 264, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    assert B.ds4hc_workspace_bytes(ps, 3, B.DS4HC_F32) == 5 * 3 * 9 * 4  # ragged, m = 8
    assert B.ds4hc_workspace_bytes(p, 4096, B.DS4HC_F32) == 0
    # from T = 32 split-K takes the streamed 16-token partials over column chunks
    # (multiples of 256 columns of the flattened row, about 512 workgroups, at
    # most 64 chunks): 64 chunks of 256 at T = 32, 16 of 1024 at T = 448, 2 of
    # 8192 at T = 4096
    pf = B.make_params(4, 4096, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    assert B.ds4hc_workspace_bytes(pf, 31, B.DS4HC_F32) == P * 31 * 25 * 4
    assert B.ds4hc_workspace_bytes(pf, 32, B.DS4HC_F32) == 64 * 32 * 25 * 4
    assert B.ds4hc_workspace_bytes(pf, 448, B.DS4HC_F32) == 16 * 448 * 25 * 4
    assert B.ds4hc_workspace_bytes(pf, 4096, B.DS4HC_F32) == 2 * 4096 * 25 * 4
    assert B.ds4hc_workspace_bytes(ps, 64, B.DS4HC_F32) == 3 * 64 * 9 * 4  # K = 528: 256, 256, 16
    pr = B.make_params(4, 4096, flags=B.DS4HC_FLAG_FORCE_ROWRES)
    assert B.ds4hc_workspace_bytes(pr, 1, B.DS4HC_F32) == 0
    # invalid arguments give 0
    assert B.ds4hc_workspace_bytes(B.make_params(4, 4095), 1, B.DS4HC_F32) == 0
    assert B.ds4hc_workspace_bytes(B.make_params(3, 4096), 1, B.DS4HC_F32) == 0


# ------------------------------------------------------------------ validation

A = 1 << 40  # fake, 16-byte-aligned device addresses, far apart


def fake(i, off=0):
    return ctypes.c_void_p(A * (i + 1) + off)


def fused(p, T=8, dt=B.DS4HC_F32, **over):
    args = dict(X=fake(0), W=fake(1), bias=fake(2), layer_out=fake(3), layer_in=fake(4),
                coeffs=fake(5), X_out=fake(6), ws=fake(7), ws_bytes=1 << 30)
    args.update(over)
    return B.ds4hc_fused_raw(p, T, dt, args["X"], args["W"], args["bias"], args["layer_out"],
                             args["layer_in"], args["coeffs"], args["X_out"], args["ws"],
                             args["ws_bytes"], None)


@no_gpu_only
@pytest.mark.parametrize("n,d,iters,eps,flags,dt,T,want", [
    (4, 4096, 20, 1e-6, 0, 5, 8, B.DS4HC_ERR_INVALID_ARG),          # unknown dtype
    (4, 4096, 20, 1e-6, 0, 0, -1, B.DS4HC_ERR_INVALID_ARG),         # T < 0
    (0, 4096, 20, 1e-6, 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),          # n < 1
    (4, 0, 20, 1e-6, 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),             # d <= 0
    (4, 4100, 20, 1e-6, 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),          # d % 8 != 0
    (4, 4096, -1, 1e-6, 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),          # iters < 0
    (4, 4096, 20, -1.0, 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),          # eps < 0
    (4, 4096, 20, float("nan"), 0, 0, 8, B.DS4HC_ERR_INVALID_ARG),  # eps NaN
    (4, 4096, 20, 1e-6, 16, 0, 8, B.DS4HC_ERR_INVALID_ARG),         # unknown flag
    (4, 4096, 20, 1e-6, 6, 0, 8, B.DS4HC_ERR_INVALID_ARG),          # two force flags
    (4, 4096, 20, 1e-6, 10, 0, 8, B.DS4HC_ERR_INVALID_ARG),         # two force flags
    (4, 8192, 20, 1e-6, 8, 0, 64, B.DS4HC_ERR_UNSUPPORTED),         # f32 row too long for tile
    (3, 4096, 20, 1e-6, 0, 0, 8, B.DS4HC_ERR_UNSUPPORTED),          # n = 3
    (8, 4096, 20, 1e-6, 0, 0, 8, B.DS4HC_ERR_UNSUPPORTED),          # n = 8
    (4, 4096, 1001, 1e-6, 0, 0, 8, B.DS4HC_ERR_UNSUPPORTED),        # iters too many
    (4, 4096, 20, 1e-6, 0, 0, (1 << 24) + 1, B.DS4HC_ERR_UNSUPPORTED),  # T too large
    (4, 65536, 20, 1e-6, 2, 0, 64, B.DS4HC_ERR_UNSUPPORTED),        # row too long to force rowres
    (4, 4096, 20, 1e-6, 0, 0, 0, B.DS4HC_OK),                       # T = 0: nothing to do
])
def test_fused_rejects_bad_params(n, d, iters, eps, flags, dt, T, want):
    p = B.make_params(n, d, eps, iters, flags)
    assert fused(p, T, dt) == want


@no_gpu_only
@pytest.mark.parametrize("field", ["X", "W", "bias", "layer_out", "layer_in", "X_out"])
def test_fused_rejects_null_pointers(field):
    p = B.make_params(4, 4096)
    assert fused(p, **{field: None}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
@pytest.mark.parametrize("field,off", [("X", 4), ("W", 8), ("layer_in", 2), ("layer_out", 12),
                                       ("X_out", 4), ("bias", 2), ("coeffs", 1), ("ws", 2)])
def test_fused_rejects_misaligned(field, off):
    p = B.make_params(4, 4096)
    idx = {"X": 0, "W": 1, "bias": 2, "layer_out": 3, "layer_in": 4, "coeffs": 5, "X_out": 6,
           "ws": 7}[field]
    assert fused(p, **{field: fake(idx, off)}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
def test_fused_rejects_small_workspace():
    p = B.make_params(4, 4096)
    need = B.ds4hc_workspace_bytes(p, 4, B.DS4HC_F32)
    assert need > 0
    assert fused(p, 4, ws_bytes=need - 4) == B.DS4HC_ERR_INVALID_ARG
    assert fused(p, 4, ws=None) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
def test_fused_rejects_overlaps_but_allows_in_place():
    p = B.make_params(4, 4096)
    T = 4096  # tile path: no workspace
    # layer_in inside X
    assert fused(p, T, layer_in=fake(0, 4096)) == B.DS4HC_ERR_INVALID_ARG
    # X_out overlapping X by a shifted window
    assert fused(p, T, X_out=fake(0, 16)) == B.DS4HC_ERR_INVALID_ARG
    # coeffs inside W
    assert fused(p, T, coeffs=fake(1, 64)) == B.DS4HC_ERR_INVALID_ARG
    # X_out exactly X is allowed: validation passes, so without a GPU the launch fails (ERR_HIP)
    assert fused(p, T, X_out=fake(0)) == B.DS4HC_ERR_HIP
    assert B.load().ds4hc_last_hip_error() != b""


@no_gpu_only
def test_pre_post_sinkhorn_validation():
    p = B.make_params(4, 4096)
    vp = fake
    # pre requires coeffs
    assert B.ds4hc_pre_raw(p, 8, 0, vp(0), vp(1), vp(2), vp(3), None, None, vp(7), 1 << 30,
                           None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_pre_raw(p, 0, 0, vp(0), vp(1), vp(2), vp(3), vp(4), None, None, 0,
                           None) == B.DS4HC_OK
    # post: X_out may be X; partial overlap rejected; null rejected
    assert B.ds4hc_post_raw(p, 8, 0, vp(0), vp(1), vp(2), vp(0, 16), None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_post_raw(p, 8, 0, vp(0), None, vp(2), vp(3), None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_post_raw(p, 0, 0, vp(0), vp(1), vp(2), vp(0), None) == B.DS4HC_OK
    # sinkhorn
    assert B.ds4hc_sinkhorn_raw(8, 3, 20, vp(0), vp(1), None) == B.DS4HC_ERR_UNSUPPORTED
    assert B.ds4hc_sinkhorn_raw(8, 0, 20, vp(0), vp(1), None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_sinkhorn_raw(8, 4, -1, vp(0), vp(1), None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_sinkhorn_raw(8, 4, 20, vp(0), vp(0, 4), None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_sinkhorn_raw(0, 4, 20, vp(0), vp(1), None) == B.DS4HC_OK
    # zero tokens: pointers are not looked at
    assert B.ds4hc_sinkhorn_raw(0, 4, 20, None, None, None) == B.DS4HC_OK
    assert B.ds4hc_post_raw(p, 0, 0, None, None, None, None, None) == B.DS4HC_OK
    assert B.ds4hc_pre_raw(p, 0, 0, None, None, None, None, None, None, None, 0,
                           None) == B.DS4HC_OK
    assert fused(p, 0, X=None, W=None, layer_in=None, ws=None) == B.DS4HC_OK


def post_pre(p, T=8, dt=B.DS4HC_F32, **over):
    args = dict(X=fake(0), cp=fake(1), lo=fake(2), W=fake(3), b=fake(4), X_out=fake(5),
                li=fake(6), c=fake(7), z=None, ws=fake(8), ws_bytes=1 << 30)
    args.update(over)
    return B.ds4hc_post_pre_raw(p, T, dt, args["X"], args["cp"], args["lo"], args["W"], args["b"],
                                args["X_out"], args["li"], args["c"], args["z"], args["ws"],
                                args["ws_bytes"], None)


def test_default_path_follows_the_measured_crossover():
    """HC-pre / fused pick split-K (the only path with a workspace), the row-resident
    or the tile kernel by the cost model fitted to the path sweeps: split-K through
    T = 519 at f32 d = 4096 (tile from 520) and through T = 591 at bf16 d = 7168
    (split-K streams its partials from T = 32); short rows: the tile kernel at
    d = 256, split-K at d = 1024 and 2048 for small T."""
    def splitk(n, d, T, dt):
        return B.ds4hc_workspace_bytes(B.make_params(n, d), T, dt) > 0
    assert all(splitk(4, 4096, T, B.DS4HC_F32) for T in (1, 4, 160, 192, 256, 384, 448, 512))
    assert not any(splitk(4, 4096, T, B.DS4HC_F32) for T in (520, 768, 1024, 4096))
    assert all(splitk(4, 7168, T, B.DS4HC_BF16) for T in (1, 4, 128, 200, 256, 320, 448, 512))
    assert not any(splitk(4, 7168, T, B.DS4HC_BF16) for T in (600, 768, 16384))
    assert not any(splitk(4, 256, T, B.DS4HC_F32) for T in (1, 4, 64, 256, 4096))
    assert all(splitk(4, 1024, T, B.DS4HC_F32) for T in (1, 4, 64))
    assert all(splitk(4, 2048, T, B.DS4HC_F32) for T in (1, 4, 64))


def test_post_pre_workspace_bytes():
    p = B.make_params(4, 4096)
    # one pass for T <= 160: column chunks of L lanes x V columns (L = 16 while that
    # gives at most 64 chunks, else 32), (m + 1) floats per token
    assert B.ds4hc_post_pre_workspace_bytes(p, 1, B.DS4HC_F32) == (4096 // 64) * 1 * 25 * 4
    assert B.ds4hc_post_pre_workspace_bytes(p, 32, B.DS4HC_BF16) == (4096 // 128) * 32 * 25 * 4
    assert B.ds4hc_post_pre_workspace_bytes(p, 160, B.DS4HC_F32) == 64 * 160 * 25 * 4
    p7 = B.make_params(4, 7168)
    assert B.ds4hc_post_pre_workspace_bytes(p7, 2, B.DS4HC_BF16) == (7168 // 128) * 2 * 25 * 4
    assert B.ds4hc_post_pre_workspace_bytes(p7, 2, B.DS4HC_F32) == (7168 // 128) * 2 * 25 * 4  # 32 lanes
    assert B.ds4hc_post_pre_workspace_bytes(B.make_params(4, 256), 1, B.DS4HC_F32) == 4 * 25 * 4
    # larger T: post, then HC-pre on its default path (split-K through T = 519 at
    # d = 4096 f32, with its workspace; the tile kernel above: none)
    assert B.ds4hc_post_pre_workspace_bytes(p, 161, B.DS4HC_F32) == 32 * 161 * 25 * 4  # streamed, 512 columns
    assert B.ds4hc_post_pre_workspace_bytes(p, 4096, B.DS4HC_F32) == 0
    pf = B.make_params(4, 4096, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    assert B.ds4hc_post_pre_workspace_bytes(pf, 4096, B.DS4HC_F32) == 64 * 4096 * 25 * 4
    assert B.ds4hc_post_pre_workspace_bytes(B.make_params(3, 4096), 1, B.DS4HC_F32) == 0


@no_gpu_only
@pytest.mark.parametrize("field", ["X", "cp", "lo", "W", "b", "X_out", "li", "c"])
def test_post_pre_rejects_null_pointers(field):
    assert post_pre(B.make_params(4, 4096), **{field: None}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
@pytest.mark.parametrize("field,idx,off", [("X", 0, 4), ("lo", 2, 8), ("W", 3, 2), ("X_out", 5, 4),
                                           ("li", 6, 12), ("cp", 1, 2), ("c", 7, 1)])
def test_post_pre_rejects_misaligned(field, idx, off):
    assert post_pre(B.make_params(4, 4096), **{field: fake(idx, off)}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
def test_post_pre_overlaps_workspace_and_in_place():
    p = B.make_params(4, 4096)
    # new coefficients over the previous ones
    assert post_pre(p, c=fake(1)) == B.DS4HC_ERR_INVALID_ARG
    # X_out overlapping X by a shifted window; layer_in inside layer_out
    assert post_pre(p, X_out=fake(0, 16)) == B.DS4HC_ERR_INVALID_ARG
    assert post_pre(p, li=fake(2, 64)) == B.DS4HC_ERR_INVALID_ARG
    # workspace too small or missing for the one-pass path
    need = B.ds4hc_post_pre_workspace_bytes(p, 8, B.DS4HC_F32)
    assert post_pre(p, ws_bytes=need - 4) == B.DS4HC_ERR_INVALID_ARG
    assert post_pre(p, ws=None) == B.DS4HC_ERR_INVALID_ARG
    # bad params; zero tokens ignore the pointers
    assert post_pre(B.make_params(3, 4096)) == B.DS4HC_ERR_UNSUPPORTED
    assert post_pre(p, 0, X=None, cp=None, lo=None, W=None, b=None, X_out=None, li=None, c=None,
                    ws=None) == B.DS4HC_OK
    # in place is allowed: validation passes, so without a GPU the launch fails (ERR_HIP)
    assert post_pre(p, X_out=fake(0)) == B.DS4HC_ERR_HIP


def test_partials_workspace_bytes():
    p = B.make_params(4, 1024)   # a quarter share of d = 4096
    P = (4 * 1024) // 256
    assert B.ds4hc_partials_workspace_bytes(p, 1, B.DS4HC_F32) == P * 1 * 25 * 4
    assert B.ds4hc_partials_workspace_bytes(p, 4096, B.DS4HC_F32) == 0   # streamed 16-token kernel
    pt = B.make_params(4, 1024, flags=B.DS4HC_FLAG_FORCE_TILE)
    assert B.ds4hc_partials_workspace_bytes(pt, 4096, B.DS4HC_F32) == 0  # tile kernel, partials mode
    pr = B.make_params(4, 1024, flags=B.DS4HC_FLAG_FORCE_ROWRES)
    assert B.ds4hc_partials_workspace_bytes(pr, 8, B.DS4HC_F32) == 0      # unsupported -> 0
    # share rows past 2^24 columns (n * d_s) leave the streamed kernel (32-bit offsets) for split-K
    assert B.ds4hc_partials_workspace_bytes(B.make_params(4, 1 << 22), 200, B.DS4HC_F32) == 0
    big = B.make_params(4, (1 << 22) + 8)   # split-K: 32-lane chunks of 32 x V columns of every stream
    assert B.ds4hc_partials_workspace_bytes(big, 200, B.DS4HC_BF16) == ((1 << 22) + 8 + 255) // 256 * 200 * 25 * 4
    assert B.ds4hc_partials_workspace_bytes(big, 200, B.DS4HC_F32) == ((1 << 22) + 8 + 127) // 128 * 200 * 25 * 4


@no_gpu_only
def test_partials_and_combine_validation():
    p = B.make_params(4, 1024)
    f = fake
    # partials: null pointers, small workspace, overlap of the output with X
    assert B.ds4hc_partials_raw(p, 8, 0, None, f(1), f(2), f(3), 1 << 30, None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_partials_raw(p, 8, 0, f(0), f(1), None, f(3), 1 << 30, None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_partials_raw(p, 8, 0, f(0), f(1), f(2), f(3), 16, None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_partials_raw(p, 8, 0, f(0), f(1), f(0, 64), f(3), 1 << 30, None) == B.DS4HC_ERR_INVALID_ARG
    assert B.ds4hc_partials_raw(B.make_params(4, 1024, flags=B.DS4HC_FLAG_FORCE_ROWRES), 8, 0, f(0),
                                f(1), f(2), f(3), 1 << 30, None) == B.DS4HC_ERR_UNSUPPORTED
    assert B.ds4hc_partials_raw(p, 0, 0, None, None, None, None, 0, None) == B.DS4HC_OK

    def comb(d_total=4096, G=4, **over):
        a = dict(P=f(0), b=f(1), X=f(2), lo=f(3), li=f(4), c=f(5), Xo=f(6))
        a.update(over)
        return B.ds4hc_combine_raw(p, d_total, 8, 0, G, a["P"], a["b"], a["X"], a["lo"], a["li"],
                                   a["c"], a["Xo"], None)
    assert comb(d_total=1000) == B.DS4HC_ERR_INVALID_ARG      # d_total < share width
    assert comb(d_total=4100) == B.DS4HC_ERR_INVALID_ARG      # d_total % 8
    assert comb(G=0) == B.DS4HC_ERR_INVALID_ARG
    assert comb(b=None) == B.DS4HC_ERR_INVALID_ARG
    assert comb(li=f(2, 16)) == B.DS4HC_ERR_INVALID_ARG       # layer_in inside X_share
    assert comb(Xo=f(2, 16)) == B.DS4HC_ERR_INVALID_ARG       # shifted in-place
    assert comb(Xo=f(2)) == B.DS4HC_ERR_HIP                   # exact in place passes validation


# ------------------------------------------------------------------ stated alignments

@no_gpu_only
@pytest.mark.parametrize("field,idx", [("bias", 2), ("coeffs", 5), ("ws", 7)])
def test_fused_float_arrays_need_4_byte_alignment_only(field, idx):
    """The float32 arrays and the workspace need 4-byte alignment: at a 4-byte
    offset validation passes (so without a GPU the launch fails, ERR_HIP); at a
    2-byte offset the call is rejected."""
    p = B.make_params(4, 4096)
    assert fused(p, 4, **{field: fake(idx, 4)}) == B.DS4HC_ERR_HIP
    assert fused(p, 4, **{field: fake(idx, 2)}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
@pytest.mark.parametrize("field,idx", [("X", 0), ("W", 1), ("layer_out", 3), ("layer_in", 4),
                                       ("X_out", 6)])
def test_fused_state_arrays_and_weight_need_16_byte_alignment(field, idx):
    p = B.make_params(4, 4096)
    assert fused(p, 4, **{field: fake(idx, 8)}) == B.DS4HC_ERR_INVALID_ARG
    assert fused(p, 4, **{field: fake(idx, 4)}) == B.DS4HC_ERR_INVALID_ARG


@no_gpu_only
def test_other_entry_points_float_arrays_need_4_byte_alignment_only():
    p = B.make_params(4, 4096)
    f = fake
    # post_pre: coeffs_prev, bias_next, coeffs, logits, workspace at 4-byte offsets pass
    assert post_pre(p, cp=f(1, 4), b=f(4, 4), c=f(7, 4), z=f(9, 4), ws=f(8, 4)) == B.DS4HC_ERR_HIP
    assert post_pre(p, z=f(9, 2)) == B.DS4HC_ERR_INVALID_ARG
    # pre: logits at a 4-byte offset passes
    assert B.ds4hc_pre_raw(p, 4, 0, f(0), f(1), f(2, 4), f(3), f(4, 4), f(5, 4), f(7, 4), 1 << 30,
                           None) == B.DS4HC_ERR_HIP
    # post: coeffs at a 4-byte offset passes, X at 8 does not
    assert B.ds4hc_post_raw(p, 4, 0, f(0), f(1, 4), f(2), f(3), None) == B.DS4HC_ERR_HIP
    assert B.ds4hc_post_raw(p, 4, 0, f(0, 8), f(1), f(2), f(3), None) == B.DS4HC_ERR_INVALID_ARG
    # sinkhorn: both arrays are float32
    assert B.ds4hc_sinkhorn_raw(4, 4, 20, f(0, 4), f(1, 4), None) == B.DS4HC_ERR_HIP
    assert B.ds4hc_sinkhorn_raw(4, 4, 20, f(0, 2), f(1), None) == B.DS4HC_ERR_INVALID_ARG
    # partials: partials and workspace at 4-byte offsets pass, X_share at 8 does not
    ps = B.make_params(4, 1024)
    assert B.ds4hc_partials_raw(ps, 8, 0, f(0), f(1), f(2, 4), f(3, 4), 1 << 30, None) == B.DS4HC_ERR_HIP
    assert B.ds4hc_partials_raw(ps, 8, 0, f(0, 8), f(1), f(2), f(3), 1 << 30, None) == B.DS4HC_ERR_INVALID_ARG
    # combine: partials, bias, coeffs at 4-byte offsets pass, layer_in_share at 8 does not
    assert B.ds4hc_combine_raw(ps, 4096, 8, 0, 4, f(0, 4), f(1, 4), f(2), f(3), f(4), f(5, 4), f(6),
                               None) == B.DS4HC_ERR_HIP
    assert B.ds4hc_combine_raw(ps, 4096, 8, 0, 4, f(0), f(1), f(2), f(3), f(4, 8), f(5), f(6),
                               None) == B.DS4HC_ERR_INVALID_ARG


# ------------------------------------------------------------------ the entry point that allocates nothing

@no_gpu_only
def test_post_pre_noalloc_validation():
    """Rejections happen on the host before any HIP call: bad arguments, and a
    workspace need beyond the fixed scratch array (DS4HC_ERR_UNSUPPORTED)."""
    f = fake

    def call(p, T=8, **over):
        a = dict(X=f(0), cp=f(1), lo=f(2), W=f(3), b=f(4), X_out=f(5), li=f(6), c=f(7), z=None)
        a.update(over)
        return B.ds4hc_post_pre_noalloc_raw(p, T, 0, a["X"], a["cp"], a["lo"], a["W"], a["b"],
                                            a["X_out"], a["li"], a["c"], a["z"], None)
    p = B.make_params(4, 4096)
    assert call(p, X=None) == B.DS4HC_ERR_INVALID_ARG
    assert call(p, X_out=f(0, 16)) == B.DS4HC_ERR_INVALID_ARG
    assert call(p, c=f(1)) == B.DS4HC_ERR_INVALID_ARG
    assert call(p, 0, X=None, cp=None, lo=None, W=None, b=None, X_out=None, li=None, c=None) == B.DS4HC_OK
    pf = B.make_params(4, 4096, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    assert B.ds4hc_post_pre_workspace_bytes(pf, 4096, B.DS4HC_F32) > B.NOALLOC_SCRATCH_BYTES
    assert call(pf, 4096) == B.DS4HC_ERR_UNSUPPORTED
    # within the scratch: validation passes, so without a GPU the device lookup fails (ERR_HIP)
    assert B.ds4hc_post_pre_workspace_bytes(p, 160, B.DS4HC_F32) <= B.NOALLOC_SCRATCH_BYTES
    assert call(p, 160) == B.DS4HC_ERR_HIP


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "ds4hc.h")).read()
    m = re.search(r"#define DS4HC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES

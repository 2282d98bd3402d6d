"""ds4hc_post_pre_noalloc (the decode-chain step for callers that cannot
allocate) against ds4hc_post_pre, through the C ABI: bitwise equal on two calls
in a row, the second with a smaller input, on the one-pass path (which uses
the scratch) and on the post-then-pre path (which needs none); sizes beyond
the scratch array refused with nothing written; and a captured HIP graph of the
call replayed with eager work between replays."""
import ctypes

import numpy as np
import pytest

from deepseek_v4_hyper_amd import binding as B
from deepseek_v4_hyper_amd import workloads as wl
from hc_testlib import case_to_device, say

pytestmark = pytest.mark.gpu


def _inputs(torch, seed, T, n, d, dtype):
    case = wl.make_random(seed, T, n, d, dtype)
    nxt = wl.make_random(seed + 1000, 1, n, d, dtype)
    X, W, b, lo = case_to_device(case)
    _, c_prev, _ = B.ds4hc_pre(X, W, b)
    Wn = torch.from_numpy(np.ascontiguousarray(nxt.W)).cuda()
    bn = torch.from_numpy(np.ascontiguousarray(nxt.bias)).cuda()
    torch.cuda.synchronize()
    return X, c_prev, lo, Wn, bn


def _bits(t):
    import torch
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _noalloc(torch, X, c_prev, lo, Wn, bn, flags=0):
    T, n, d = X.shape
    m = 2 * n + n * n
    Xo = torch.full_like(X, float("nan"))
    li = torch.full((T, d), float("nan"), dtype=X.dtype, device="cuda")
    c = torch.full((T, m), float("nan"), device="cuda")
    z = torch.full((T, m), float("nan"), device="cuda")
    p = B.make_params(n, d, flags=flags)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = B.ds4hc_post_pre_noalloc_raw(p, T, B.DS4HC_F32 if X.dtype == torch.float32 else B.DS4HC_BF16,
                                      P(X), P(c_prev), P(lo), P(Wn), P(bn), P(Xo), P(li), P(c), P(z), sp)
    return st, (Xo, li, c, z)


@pytest.mark.parametrize("dtype,d,T1,T2", [(wl.F32, 4096, 37, 3), (wl.BF16, 7168, 160, 1),
                                           (wl.F32, 4096, 300, 200)])
def test_noalloc_equals_post_pre_two_calls(dtype, d, T1, T2):
    import torch
    for T in (T1, T2):
        X, c_prev, lo, Wn, bn = _inputs(torch, 50 + T, T, 4, d, dtype)
        say(f"[gpu] ds4hc_post_pre_noalloc T={T} d={d} {dtype}")
        p = B.make_params(4, d)
        dt = B.DS4HC_F32 if dtype == wl.F32 else B.DS4HC_BF16
        need = B.ds4hc_post_pre_workspace_bytes(p, T, dt)
        assert need <= B.NOALLOC_SCRATCH_BYTES
        ref = B.ds4hc_post_pre(X, c_prev, lo, Wn, bn, want_logits=True)
        st, got = _noalloc(torch, X, c_prev, lo, Wn, bn)
        assert st == B.DS4HC_OK
        torch.cuda.synchronize()
        for a, e in zip(got, ref):
            assert torch.equal(_bits(a), _bits(e))
        say(f"    bitwise equal to ds4hc_post_pre (workspace {need} bytes)")


def test_noalloc_refuses_more_than_its_scratch():
    import torch
    T, d = 4096, 4096
    X, c_prev, lo, Wn, bn = _inputs(torch, 77, T, 4, d, wl.F32)
    p = B.make_params(4, d, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    assert B.ds4hc_post_pre_workspace_bytes(p, T, B.DS4HC_F32) > B.NOALLOC_SCRATCH_BYTES
    say("[gpu] ds4hc_post_pre_noalloc beyond the scratch: refused")
    st, got = _noalloc(torch, X, c_prev, lo, Wn, bn, flags=B.DS4HC_FLAG_FORCE_SPLITK)
    torch.cuda.synchronize()
    assert st == B.DS4HC_ERR_UNSUPPORTED
    for t in got:
        assert torch.isnan(t.float()).all()   # nothing was written


def test_noalloc_in_a_captured_graph():
    import torch
    X, c_prev, lo, Wn, bn = _inputs(torch, 91, 1, 4, 4096, wl.F32)
    ref = B.ds4hc_post_pre(X, c_prev, lo, Wn, bn)
    T, n, d = X.shape
    Xo = torch.empty_like(X)
    li = torch.empty((T, d), device="cuda")
    c = torch.empty((T, 24), device="cuda")
    say("[gpu] ds4hc_post_pre_noalloc captured in a HIP graph, 3 replays")
    B.ds4hc_post_pre_noalloc(X, c_prev, lo, Wn, bn, Xo, li, c)   # eager first call on the device
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.ds4hc_post_pre_noalloc(X, c_prev, lo, Wn, bn, Xo, li, c)
    other = _inputs(torch, 92, 5, 4, 4096, wl.F32)
    for rep in range(3):
        for t in (Xo, li, c):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip((Xo, li, c), ref[:3]):
            assert torch.equal(_bits(a), _bits(e)), f"replay {rep}"
        _noalloc(torch, *other)   # eager use of the same scratch between replays
        torch.cuda.synchronize()

"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs, for every workload and both kernel paths.

Small and reduced-T cases are compared on every output element; the
full-size prefill and stress workloads, in the launch configuration the
benchmark times, are compared on sampled token rows the oracle computes one
by one (rows are independent).
"""
import numpy as np
import pytest

import oracle
from deepseek_v4_hyper_amd import binding as B
from deepseek_v4_hyper_amd import workloads as wl
from hc_testlib import (TOL, assert_close_rows, assert_coeffs, case_to_device, say,
                        state_to_torch, torch_to_f64)

pytestmark = pytest.mark.gpu

FLAGS = {"default": 0, "rowres": B.DS4HC_FLAG_FORCE_ROWRES, "tile": B.DS4HC_FLAG_FORCE_TILE,
         "splitk": B.DS4HC_FLAG_FORCE_SPLITK}
PATHS = ["default", "rowres", "tile", "splitk"]


def torch_mod():
    import torch
    return torch


def run_fused(case, flags=0, X=None):
    torch = torch_mod()
    Xd, W, b, lo = case_to_device(case)
    if X is not None:
        Xd = X
    say(f"[gpu] ds4hc_fused {case.name} T={case.T} n={case.n} d={case.d} {case.dtype} flags={flags}")
    li, c, xo = B.ds4hc_fused(Xd, W, b, lo, rms_eps=case.eps, sinkhorn_iters=case.iters,
                              flags=flags)
    torch.cuda.synchronize()
    return torch_to_f64(li), c.cpu().numpy().astype(np.float64), torch_to_f64(xo)


def oracle_fused(case, rows=None):
    X = wl.state_to_f64(case.X if rows is None else case.X[rows], case.dtype)
    lo = wl.state_to_f64(case.layer_out if rows is None else case.layer_out[rows], case.dtype)
    return oracle.fused(X, case.W, case.bias, lo, case.eps, case.iters)


def check_full(case, got, what):
    li, c, xo = got
    rli, rc, rxo = oracle_fused(case)
    tol = TOL[case.dtype]
    e1 = assert_close_rows(li, rli, tol, f"{what} layer_in")
    e2 = assert_close_rows(xo, rxo, tol, f"{what} X_out")
    e3 = assert_coeffs(c, rc, f"{what} coeffs")
    say(f"    errors: layer_in {e1:.2e}  X_out {e2:.2e}  coeffs {e3:.2e}")


# ------------------------------------------------------------------ workloads, every element

@pytest.mark.parametrize("path", PATHS)
def test_single_token(path):
    case = wl.make_single(0)
    check_full(case, run_fused(case, FLAGS[path]), f"single/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_verify_batch(path):
    case = wl.make_verify(0)
    check_full(case, run_fused(case, FLAGS[path]), f"verify/{path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("q", [2, 3])
def test_verify_widths(path, q):
    """Speculative-verify batches of width q = 2 and 3 (adaptive draft widths):
    a partly filled split-K token group and a partly filled tile."""
    case = wl.make_verify(10 + q, T=q)
    check_full(case, run_fused(case, FLAGS[path]), f"verify q={q}/{path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [37, 67])
def test_prefill_reduced_T(path, T):
    """Prefill shape and value recipe (per-token log-uniform scales) at a T the
    oracle finishes in seconds; 37 / 67 leave ragged tails on both paths."""
    case = wl.make_prefill(1, T=T)
    check_full(case, run_fused(case, FLAGS[path]), f"prefill T={T}/{path}")


@pytest.mark.parametrize("path", PATHS)
def test_stress_reduced_T(path):
    """Stress recipe (bf16, residual logit std ~20, 5 % zero rows) at T = 41, d = 7168:
    d is not a multiple of the row-resident chunk, so the last chunk is ragged."""
    case = wl.make_stress(2, T=41)
    assert len(case.zero_rows) == 2
    got = run_fused(case, FLAGS[path])
    check_full(case, got, f"stress T=41/{path}")
    li = got[0]
    assert np.all(li[case.zero_rows] == 0.0)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("n,d", [(1, 8), (1, 1032), (2, 264), (2, 4096), (4, 8), (4, 2056),
                                 (4, 16384)])
@pytest.mark.parametrize("path", ["rowres", "tile", "splitk"])
def test_shapes(dtype, n, d, path):
    V = 4 if dtype == wl.F32 else 8
    cap = (7 if dtype == wl.F32 else 5) if n == 4 else 8
    if path == "rowres" and d > cap * 256 * V:
        pytest.skip("row too long for the row-resident kernel")
    if path == "tile" and d > 8 * 4 * 32 * V:
        pytest.skip("row too long for the tile kernel")
    case = wl.make_random(3 + n + d, 5, n, d, dtype)
    check_full(case, run_fused(case, FLAGS[path]), f"n={n} d={d} {dtype}/{path}")


# ------------------------------------------------------------------ persistent tile grid

def _cu_count():
    return torch_mod().cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("n,d,dtype", [(4, 512, wl.F32), (4, 1024, wl.BF16), (2, 264, wl.F32),
                                       (1, 1032, wl.BF16)])
def test_tile_several_tiles_per_workgroup(n, d, dtype):
    """T = 8 * CUs + 3: the persistent grid has one workgroup per CU, so each
    takes two tiles of four tokens and the first takes a third, ragged one of
    three; the weight ring and the row prefetch carry over between tiles.
    Every element is compared."""
    T = 8 * _cu_count() + 3
    case = wl.make_random(11 + n + d, T, n, d, dtype)
    check_full(case, run_fused(case, FLAGS["tile"]), f"tile x3 n={n} d={d} {dtype}")


@pytest.mark.parametrize("path", ["tile", "rowres", "splitk"])
def test_bf16_wide_dynamic_range(path):
    """bfloat16 rows whose elements span 2^-60 .. 2^0 (each scaled by its own
    random power of two): the tile kernel's projection uses only the f16 hi part
    of a bfloat16 element, which is exact down to 2^30 below the lane's largest
    value, so even rows like these match the oracle within the bfloat16
    tolerance, with the coefficients within 2e-5."""
    import dataclasses
    rng = np.random.Generator(np.random.PCG64(77))
    T, n, d = 2 * _cu_count() + 5, 4, 2048
    base = wl.make_random(77, T, n, d, wl.BF16)
    x = wl.bf16_bits_to_f32(base.X).astype(np.float64)
    x = x * np.exp2(-rng.integers(0, 61, size=x.shape))
    case = dataclasses.replace(base, name="bf16_wide_range",
                               X=wl.f32_to_bf16_bits(x.astype(np.float32)))
    check_full(case, run_fused(case, FLAGS[path]), f"bf16 wide range/{path}")


def test_tile_prefill_recipe_several_tiles_in_place_and_pre():
    """Prefill recipe at T = 8 * CUs + 3 on the tile path: fused against the
    oracle on every element, in place (X_out = X) bitwise equal to out of
    place, and HC-pre alone bitwise equal to the fused layer_in / coeffs."""
    torch = torch_mod()
    T = 8 * _cu_count() + 3
    case = wl.make_prefill(12, T=T)
    X, W, b, lo = case_to_device(case)
    fl = FLAGS["tile"]
    say(f"[gpu] tile path, prefill recipe T={T}: fused, in place, pre")
    li, c, xo = B.ds4hc_fused(X, W, b, lo, flags=fl)
    Xi = X.clone()
    li2, c2, xo2 = B.ds4hc_fused(Xi, W, b, lo, flags=fl, X_out=Xi)
    li3, c3, _ = B.ds4hc_pre(X, W, b, flags=fl)
    torch.cuda.synchronize()
    assert torch.equal(Xi, xo) and torch.equal(li2, li) and torch.equal(c2, c)
    assert torch.equal(li3, li) and torch.equal(c3, c)
    got = (torch_to_f64(li), c.cpu().numpy().astype(np.float64), torch_to_f64(xo))
    check_full(case, got, f"prefill T={T}/tile")


# ------------------------------------------------------------------ full-size workloads, sampled rows

def _sampled_check(case, flags, nsample, extra_rows=()):
    torch = torch_mod()
    got_li, got_c, got_xo = run_fused(case, flags)
    rng = np.random.Generator(np.random.PCG64(123))
    rows = np.unique(np.concatenate([[0, case.T - 1], rng.choice(case.T, nsample, replace=False),
                                     np.asarray(extra_rows, dtype=np.int64)])).astype(np.int64)
    rli, rc, rxo = oracle_fused(case, rows)
    tol = TOL[case.dtype]
    e1 = assert_close_rows(got_li[rows], rli, tol, f"{case.name} layer_in")
    e2 = assert_close_rows(got_xo[rows], rxo, tol, f"{case.name} X_out")
    e3 = assert_coeffs(got_c[rows], rc, f"{case.name} coeffs")
    say(f"    {len(rows)} sampled rows: layer_in {e1:.2e}  X_out {e2:.2e}  coeffs {e3:.2e}")
    # properties that hold for every row at any size
    assert np.all(np.isfinite(got_xo)) and np.all(np.isfinite(got_li))
    H = got_c[:, 2 * case.n:].reshape(case.T, case.n, case.n)
    assert np.abs(H.sum(axis=1) - 1.0).max() < 1e-5      # columns normalised last
    assert np.all((got_c >= 0) & (got_c <= 1))
    del torch
    return got_li, got_c, got_xo


def test_prefill_full_size_sampled():
    case = wl.make_prefill(0)
    _sampled_check(case, 0, 96)


def test_stress_full_size_sampled():
    case = wl.make_stress(0)
    li, c, xo = _sampled_check(case, 0, 64, extra_rows=case.zero_rows[:16])
    # every all-zero row: layer_in = 0, pre = post = 1/2, H = 1/n, X' = layer_out / 2 (bf16-exact)
    zr = case.zero_rows
    assert np.all(li[zr] == 0.0)
    assert np.all(c[zr, :8] == 0.5) and np.all(c[zr, 8:] == 0.25)
    lo = wl.state_to_f64(case.layer_out[zr], case.dtype)
    np.testing.assert_array_equal(xo[zr], np.repeat(0.5 * lo[:, None, :], case.n, axis=1))


# ------------------------------------------------------------------ decode chain

def test_decode_chain_43_layers():
    """43 x (HC-pre -> stand-in layer body -> hc_post), stream-ordered, one sync.
    Checked per layer under teacher forcing (oracle fed the GPU's X_l) and end to end."""
    torch = torch_mod()
    case = wl.make_chain(0)
    n, d = case.n, case.d
    X = state_to_torch(case.X, case.dtype)
    b = torch.zeros(case.m, dtype=torch.float32, device="cuda")
    Ws = [torch.from_numpy(w).cuda() for w in case.chain_W]
    noise = torch.from_numpy(case.chain_noise).cuda()
    states = [X.clone()]
    ins, coeffs = [], []
    say("[gpu] decode chain: 43 layers, T=1, d=4096")
    for l in range(len(Ws)):
        li, c, _ = B.ds4hc_pre(X, Ws[l], b)
        lo = li * 0.5 + noise[l][None, :]
        X = B.ds4hc_post(X, c, lo)
        states.append(X)
        ins.append(li)
        coeffs.append(c)
    torch.cuda.synchronize()
    worst = 0.0
    for l in range(len(Ws)):
        Xl = torch_to_f64(states[l])
        rli, rc, _ = oracle.pre(Xl, case.chain_W[l], case.bias)
        lo = torch_to_f64(ins[l]) * 0.5 + case.chain_noise[l].astype(np.float64)[None, :]
        rx = oracle.post(Xl, rc, lo)
        worst = max(worst, assert_close_rows(torch_to_f64(ins[l]), rli, TOL[wl.F32], f"layer {l} layer_in"),
                    assert_close_rows(torch_to_f64(states[l + 1]), rx, TOL[wl.F32], f"layer {l} X'"))
        assert_coeffs(coeffs[l].cpu().numpy(), rc, f"layer {l} coeffs")
    ref = oracle.chain(wl.state_to_f64(case.X, case.dtype), case.chain_W, case.bias, case.chain_noise)
    e2e = assert_close_rows(torch_to_f64(states[-1]), ref[-1], 1e-4, "chain end to end")
    say(f"    teacher-forced worst {worst:.2e}; end-to-end {e2e:.2e}")


# ------------------------------------------------------------------ Sinkhorn alone

@pytest.mark.parametrize("n", [1, 2, 4])
@pytest.mark.parametrize("iters", [0, 1, 7, 20, 200])
def test_sinkhorn_random(n, iters):
    torch = torch_mod()
    rng = np.random.Generator(np.random.PCG64(n * 1000 + iters))
    Z = (rng.standard_normal((1000, n, n)) * 3).astype(np.float32)
    say(f"[gpu] ds4hc_sinkhorn n={n} iters={iters}")
    H = B.ds4hc_sinkhorn(torch.from_numpy(Z).cuda(), iters=iters).cpu().numpy()
    assert_coeffs(H, oracle.sinkhorn(Z, iters), "sinkhorn")


def test_sinkhorn_entries_within_unit_interval():
    # logits at the stress workload's scale (std 20): every entry of H lies in
    # [0, 1] (an entry equal to its row or column sum must not round above 1),
    # and a NaN logit turns its own matrix into NaN and no other
    torch = torch_mod()
    rng = np.random.Generator(np.random.PCG64(7))
    Z = (rng.standard_normal((20000, 4, 4)) * 20).astype(np.float32)
    Z[5, 1, 2] = np.nan
    for iters in (1, 2, 20):
        say(f"[gpu] ds4hc_sinkhorn n=4 iters={iters} logit std 20, one NaN matrix")
        H = B.ds4hc_sinkhorn(torch.from_numpy(Z).cuda(), iters=iters).cpu().numpy()
        assert np.isnan(H[5]).all()
        rest = np.delete(H, 5, axis=0)
        assert np.all((rest >= 0) & (rest <= 1))
        assert_coeffs(rest, oracle.sinkhorn(np.delete(Z, 5, axis=0), iters), "sinkhorn")


def test_sinkhorn_closed_forms():
    torch = torch_mod()
    P = np.zeros((4, 4))
    P[np.arange(4), [1, 2, 3, 0]] = 1
    Zs = np.stack([np.zeros((4, 4)), 5 * P, 90 * P, 200 * P]).astype(np.float32)
    say("[gpu] ds4hc_sinkhorn closed forms")
    H = B.ds4hc_sinkhorn(torch.from_numpy(Zs).cuda(), iters=20).cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(H[0], 0.25)
    for k, c in ((1, 5.0), (2, 90.0)):
        # closed form ((e^c - 1) P + J) / (e^c + n - 1); at c = 90 the off-diagonal
        # 1/(e^90 + 3) = 8.2e-40 is a float32 subnormal, and exp(90) itself would
        # overflow float32 without the max subtraction
        want = (np.expm1(c) * P + 1) / (np.exp(c) + 3)
        np.testing.assert_allclose(H[k], want, rtol=1e-5, atol=1e-44)
    np.testing.assert_array_equal(H[3], P)   # e^-200 underflows to 0 in float32


# ------------------------------------------------------------------ API behaviour on the GPU

def test_pre_then_post_equals_fused_bitwise():
    torch = torch_mod()
    case = wl.make_prefill(4, T=64)
    X, W, b, lo = case_to_device(case)
    say("[gpu] pre+post vs fused, T=64")
    li1, c1, xo1 = B.ds4hc_fused(X, W, b, lo)
    li2, c2, _ = B.ds4hc_pre(X, W, b)
    xo2 = B.ds4hc_post(X, c2, lo)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(li1, li2) and torch.equal(xo1, xo2)


def test_in_place_update():
    torch = torch_mod()
    for T in (3, 50):
        case = wl.make_prefill(5, T=T)
        X, W, b, lo = case_to_device(case)
        say(f"[gpu] in-place fused T={T}")
        li_ref, c_ref, xo_ref = B.ds4hc_fused(X, W, b, lo)
        Xi = X.clone()
        li, c, xo = B.ds4hc_fused(Xi, W, b, lo, X_out=Xi)
        torch.cuda.synchronize()
        assert xo.data_ptr() == Xi.data_ptr()
        assert torch.equal(Xi, xo_ref) and torch.equal(li, li_ref) and torch.equal(c, c_ref)


def test_deterministic_repeats():
    import hashlib
    torch = torch_mod()
    case = wl.make_prefill(6, T=512)
    X, W, b, lo = case_to_device(case)
    say("[gpu] 20 repeats, T=512 fused + T=4 fused")
    small = wl.make_verify(6)
    Xs, Ws, bs, los = case_to_device(small)
    digests = set()
    for _ in range(20):
        outs = B.ds4hc_fused(X, W, b, lo) + B.ds4hc_fused(Xs, Ws, bs, los)
        torch.cuda.synchronize()
        h = hashlib.sha256()
        for o in outs:
            h.update(o.view(torch.uint8).cpu().numpy().tobytes())
        digests.add(h.hexdigest())
    assert len(digests) == 1


@pytest.mark.parametrize("workload", ["prefill", "stress"])
def test_deterministic_repeats_full_size(workload):
    """The benchmark's own launch configuration (prefill: 4 tiles per tile-kernel
    workgroup; stress: 16), run 3 times: every output identical bit for bit."""
    import hashlib
    torch = torch_mod()
    case = wl.make_prefill(5) if workload == "prefill" else wl.make_stress(5)
    X, W, b, lo = case_to_device(case)
    say(f"[gpu] 3 repeats of ds4hc_fused, {workload} T={case.T} d={case.d} {case.dtype}")
    digests = set()
    for _ in range(3):
        outs = B.ds4hc_fused(X, W, b, lo)
        torch.cuda.synchronize()
        h = hashlib.sha256()
        for o in outs:
            h.update(o.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        digests.add(h.hexdigest())
        del outs
    assert len(digests) == 1


def test_nan_row_stays_in_its_token():
    torch = torch_mod()
    case = wl.make_prefill(7, T=40)
    X = case.X.copy()
    X[11, 2, 100] = np.nan
    say("[gpu] NaN propagation")
    li, c, xo = run_fused(case, 0, X=state_to_torch(X, case.dtype))
    assert np.all(np.isnan(li[11])) and np.all(np.isnan(xo[11])) and np.all(np.isnan(c[11]))
    good = np.setdiff1d(np.arange(40), [11])
    case.X = X
    rli, rc, rxo = oracle_fused(case, good)
    assert_close_rows(xo[good], rxo, TOL[wl.F32], "non-NaN rows")


def test_zero_tokens_is_a_no_op():
    torch = torch_mod()
    X = torch.empty((0, 4, 256), device="cuda")
    W = torch.zeros((24, 1024), dtype=torch.float16, device="cuda")
    b = torch.zeros(24, device="cuda")
    lo = torch.empty((0, 256), device="cuda")
    li, c, xo = B.ds4hc_fused(X, W, b, lo)
    torch.cuda.synchronize()
    assert li.shape == (0, 256) and xo.shape == (0, 4, 256)


@pytest.mark.parametrize("iters", [0, 1, 3])
def test_iteration_counts(iters):
    case = wl.make_prefill(8, T=40)
    case.iters = iters
    check_full(case, run_fused(case, 0), f"iters={iters}")


def test_logits_output_matches_oracle():
    torch = torch_mod()
    case = wl.make_verify(9)
    X, W, b, _ = case_to_device(case)
    say("[gpu] ds4hc_pre logits")
    for flags in (0, B.DS4HC_FLAG_FORCE_ROWRES, B.DS4HC_FLAG_FORCE_TILE):
        li, c, z = B.ds4hc_pre(X, W, b, flags=flags, want_logits=True)
        torch.cuda.synchronize()
        _, _, rz = oracle.pre(wl.state_to_f64(case.X, case.dtype), case.W, case.bias)
        assert_close_rows(z.cpu().numpy(), rz, 2e-5, "logits")


# ------------------------------------------------------------------ one-pass chain step post(l) + pre(l+1)

def _post_pre_case(seed, T, n, d, dtype):
    """X, site l's coefficients (from ds4hc_pre with W_l), layer_out_l, and site l+1's weight."""
    torch = torch_mod()
    case = wl.make_random(seed, T, n, d, dtype)
    nxt = wl.make_random(seed + 1000, 1, n, d, dtype)
    X, W, b, lo = case_to_device(case)
    _, c_prev, _ = B.ds4hc_pre(X, W, b)
    Wn = torch.from_numpy(np.ascontiguousarray(nxt.W)).cuda()
    bn = torch.from_numpy(np.ascontiguousarray(nxt.bias)).cuda()
    return case, nxt, X, c_prev, lo, Wn, bn


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("n,d", [(4, 4096), (2, 264), (1, 1032), (4, 2056)])
@pytest.mark.parametrize("T", [1, 3, 37, 200])
def test_post_pre_equals_post_then_pre(dtype, n, d, T):
    """ds4hc_post_pre against ds4hc_post followed by ds4hc_pre (T = 1, 3, 37: the
    one-pass split-K kernels, one or several token groups; T = 200: post, then the
    row-resident pre on X'). X' must be bitwise what
    ds4hc_post writes; layer_in and coeffs are checked against the oracle's HC-pre
    of that X' and against the two-call path."""
    torch = torch_mod()
    case, nxt, X, c_prev, lo, Wn, bn = _post_pre_case(20 + T + n, T, n, d, dtype)
    say(f"[gpu] ds4hc_post_pre T={T} n={n} d={d} {dtype}")
    Xo, li, c, _ = B.ds4hc_post_pre(X, c_prev, lo, Wn, bn)
    Xp = B.ds4hc_post(X, c_prev, lo)
    li2, c2, _ = B.ds4hc_pre(Xp, Wn, bn)
    torch.cuda.synchronize()
    assert torch.equal(Xo, Xp)
    tol = TOL[dtype]
    rli, rc, _ = oracle.pre(torch_to_f64(Xo), nxt.W, nxt.bias)
    assert_close_rows(torch_to_f64(li), rli, tol, "post_pre layer_in")
    assert_coeffs(c.cpu().numpy().astype(np.float64), rc, "post_pre coeffs")
    assert_close_rows(torch_to_f64(li), torch_to_f64(li2), tol, "post_pre vs two calls")
    rxp = oracle.post(torch_to_f64(X), c_prev.cpu().numpy().astype(np.float64),
                      torch_to_f64(lo))
    assert_close_rows(torch_to_f64(Xo), rxp, tol, "post_pre X'")


@pytest.mark.parametrize("T", [2, 40, 200])
def test_post_pre_in_place(T):
    torch = torch_mod()
    case, nxt, X, c_prev, lo, Wn, bn = _post_pre_case(31, T, 4, 4096, wl.F32)
    say(f"[gpu] ds4hc_post_pre in place T={T}")
    Xo, li, c, _ = B.ds4hc_post_pre(X, c_prev, lo, Wn, bn)
    Xi = X.clone()
    Xo2, li2, c2, _ = B.ds4hc_post_pre(Xi, c_prev, lo, Wn, bn, X_out=Xi)
    torch.cuda.synchronize()
    assert Xo2.data_ptr() == Xi.data_ptr()
    assert torch.equal(Xi, Xo) and torch.equal(li2, li) and torch.equal(c2, c)


def test_decode_chain_43_layers_post_pre():
    """The 43-layer chain with one ds4hc_post_pre per layer boundary (ds4hc_pre for
    the first site, ds4hc_post after the last): same end state as the oracle's chain."""
    torch = torch_mod()
    case = wl.make_chain(0)
    X = state_to_torch(case.X, case.dtype)
    b = torch.zeros(case.m, dtype=torch.float32, device="cuda")
    Ws = [torch.from_numpy(w).cuda() for w in case.chain_W]
    noise = torch.from_numpy(case.chain_noise).cuda()
    say("[gpu] decode chain with ds4hc_post_pre: 43 layers, T=1, d=4096")
    li, c, _ = B.ds4hc_pre(X, Ws[0], b)
    for l in range(len(Ws)):
        lo = li * 0.5 + noise[l][None, :]
        if l + 1 < len(Ws):
            X, li, c, _ = B.ds4hc_post_pre(X, c, lo, Ws[l + 1], b)
        else:
            X = B.ds4hc_post(X, c, lo)
    torch.cuda.synchronize()
    ref = oracle.chain(wl.state_to_f64(case.X, case.dtype), case.chain_W, case.bias, case.chain_noise)
    e2e = assert_close_rows(torch_to_f64(X), ref[-1], 1e-4, "post_pre chain end to end")
    say(f"    end-to-end {e2e:.2e}")


# ------------------------------------------------------------------ split over d (one GPU's share)

def _shares(case, G):
    torch = torch_mod()
    X, W, b, lo = case_to_device(case)
    n, d, m = case.n, case.d, case.m
    ds = d // G
    Wr = W.reshape(m, n, d)
    sh = []
    for g in range(G):
        cols = slice(g * ds, (g + 1) * ds)
        sh.append((X[:, :, cols].contiguous(), Wr[:, :, cols].reshape(m, n * ds).contiguous(),
                   lo[:, cols].contiguous()))
    return X, W, b, lo, sh


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("G,n,d", [(2, 4, 4096), (4, 4, 4096), (2, 2, 528)])
@pytest.mark.parametrize("T", [1, 5, 700])
def test_split_over_d(dtype, G, n, d, T):
    """G column shares: partials per share, the [G, T, m+1] exchange, then each share
    combines and finishes its own columns. The assembled result is the whole op
    (checked against the oracle); every share computes bitwise the same coefficients."""
    torch = torch_mod()
    case = wl.make_random(40 + G + T, T, n, d, dtype)
    X, W, b, lo, sh = _shares(case, G)
    say(f"[gpu] split over d: G={G} T={T} n={n} d={d} {dtype}")
    P = torch.stack([B.ds4hc_partials(xs, ws) for xs, ws, _ in sh])
    outs = [B.ds4hc_combine(P, b, xs, los, d) for xs, _, los in sh]
    torch.cuda.synchronize()
    for li_g, c_g, _ in outs[1:]:
        assert torch.equal(c_g, outs[0][1])
    li = torch.cat([o[0] for o in outs], dim=1)
    xo = torch.cat([o[2] for o in outs], dim=2)
    got = (torch_to_f64(li), outs[0][1].cpu().numpy().astype(np.float64), torch_to_f64(xo))
    check_full(case, got, f"split d G={G} T={T}")

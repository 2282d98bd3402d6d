"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs, for every workload and both kernel paths.

Every case is compared on every output element, the full-size prefill and
stress workloads (in the launch configuration the benchmark times) included:
there the oracle runs over token chunks, since rows are independent.
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


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("n,d", [(1, 8), (1, 1032), (2, 264), (4, 8), (4, 2056), (4, 16384)])
@pytest.mark.parametrize("T", [37, 300])
def test_shapes_streamed_splitk(dtype, n, d, T):
    """Split-K from T = 32 takes the streamed 16-token partials over column chunks
    (multiples of 256 columns of the flattened row, the last one ragged where K is
    not a multiple): a ragged last token group (T = 37) and a few dozen chunks
    (T = 300), against the oracle."""
    case = wl.make_random(70 + n + d + T, T, n, d, dtype)
    got = run_fused(case, FLAGS["splitk"])
    check_full(case, got, f"streamed split-K T={T} n={n} d={d} {dtype}")
    again = run_fused(case, FLAGS["splitk"])
    for a, b in zip(got, again):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "repeat differs"


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


# ------------------------------------------------------------------ full-size workloads, every element

def _full_size_check(case, flags, chunk=1024):
    """The workload at its full size, in the launch configuration the benchmark
    times, compared with the oracle on every element of layer_in, X_out and the
    coefficients. Rows are independent, so the oracle runs over token chunks and
    its float64 outputs never hold more than `chunk` rows at a time."""
    torch = torch_mod()
    Xd, W, b, lo = case_to_device(case)
    say(f"[gpu] ds4hc_fused full size {case.name} T={case.T} n={case.n} d={case.d} {case.dtype} "
        f"flags={flags}: every element")
    li, c, xo = B.ds4hc_fused(Xd, W, b, lo, rms_eps=case.eps, sinkhorn_iters=case.iters, flags=flags)
    torch.cuda.synchronize()
    del Xd, lo
    tol = TOL[case.dtype]
    got_c = c.cpu().numpy().astype(np.float64)
    e = [0.0, 0.0, 0.0]
    for a in range(0, case.T, chunk):
        rows = slice(a, min(case.T, a + chunk))
        rli, rc, rxo = oracle_fused(case, rows)
        e[0] = max(e[0], assert_close_rows(torch_to_f64(li[rows]), rli, tol, f"{case.name} layer_in"))
        e[1] = max(e[1], assert_close_rows(torch_to_f64(xo[rows]), rxo, tol, f"{case.name} X_out"))
        e[2] = max(e[2], assert_coeffs(got_c[rows], rc, f"{case.name} coeffs"))
    say(f"    all {case.T} rows: layer_in {e[0]:.2e}  X_out {e[1]:.2e}  coeffs {e[2]:.2e}")
    assert np.all(np.isfinite(got_c)) and np.all((got_c >= 0) & (got_c <= 1))
    return li, got_c, xo


def test_prefill_full_size_every_element():
    _full_size_check(wl.make_prefill(0), 0)


@pytest.mark.parametrize("path", ["default", "splitk"])
def test_stress_full_size_every_element(path):
    case = wl.make_stress(0)
    li, c, xo = _full_size_check(case, FLAGS[path])
    # every all-zero row: layer_in = 0, pre = post = 1/2, H = 1/n, X' = layer_out / 2 (bf16-exact)
    torch = torch_mod()
    zr = case.zero_rows
    zi = torch.from_numpy(zr).to(li.device)
    assert np.all(torch_to_f64(li.index_select(0, zi)) == 0.0)
    assert np.all(c[zr, :8] == 0.5) and np.all(c[zr, 8:] == 0.25)
    lo = wl.state_to_f64(case.layer_out[zr], case.dtype)
    np.testing.assert_array_equal(torch_to_f64(xo.index_select(0, zi)),
                                  np.repeat(0.5 * lo[:, None, :], case.n, axis=1))


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
    e2e = assert_close_rows(torch_to_f64(states[-1]), ref[-1], TOL[wl.F32], "chain end to end")
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
@pytest.mark.parametrize("n,d", [(4, 4096), (2, 264), (1, 1032), (4, 2056), (4, 7168), (1, 8200)])
@pytest.mark.parametrize("T", [1, 3, 37, 200])
def test_post_pre_equals_post_then_pre(dtype, n, d, T):
    """ds4hc_post_pre against ds4hc_post followed by ds4hc_pre (T = 1, 3, 37: the
    one-pass split-K kernels, one or several token groups; T = 200: post, then
    HC-pre on X' on its default path). The one-pass step takes column chunks of 16 lanes
    where that gives at most 64 chunks, else 32: d = 7168 fp32 and d = 8200
    (either type, with a ragged last chunk) take 32. X' must be bitwise what
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
    e2e = assert_close_rows(torch_to_f64(X), ref[-1], TOL[wl.F32], "post_pre chain end to end")
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


def _check_partials(got, ref, Xs, Ws, what):
    """Dots within 2e-6 of sum_k |W_jk x_k| (float32 accumulation over K terms),
    the sum of squares within 2e-6 relative."""
    m = Ws.shape[0]
    T = Xs.shape[0]
    x = Xs.reshape(T, -1)
    scale = np.abs(x) @ np.abs(Ws).T
    err = np.abs(got[:, :m] - ref[:, :m])
    assert np.all(err <= 2e-6 * scale + 1e-30), f"{what}: dots max err/scale {np.max(err / (scale + 1e-300)):.3g}"
    rel = np.abs(got[:, m] - ref[:, m]) / np.maximum(ref[:, m], 1e-300)
    assert np.all((rel <= 2e-6) | (ref[:, m] == 0)), f"{what}: sum of squares max rel {np.max(rel):.3g}"
    say(f"    {what}: dots max err/scale {np.max(err / (scale + 1e-300)):.2e}, sum of squares max rel {np.max(rel):.2e}")


@pytest.mark.parametrize("path,dtype,n,ds,T", [
    ("default", wl.F32, 4, 1024, 4096),    # the prefill share the benchmark times (streamed kernel)
    ("default", wl.BF16, 4, 1792, 4096),   # a quarter of the stress width
    ("default", wl.F32, 2, 264, 700),      # K = 528: a partial last k-step, a partial token group
    ("default", wl.BF16, 1, 520, 161),     # n = 1 (one 16-row block), K = 520
    ("default", wl.F32, 4, 1024, 37),      # split-K chunks at small T
    ("tile", wl.F32, 4, 1024, 700),
    ("tile", wl.BF16, 2, 264, 161),
    ("splitk", wl.BF16, 4, 1024, 700),
])
def test_partials_against_oracle(path, dtype, n, ds, T):
    """ds4hc_partials of one column share against the oracle's partial sums, on
    every path that can produce them."""
    torch = torch_mod()
    case = wl.make_random(60 + T + n, T, n, ds, dtype)
    X, W, _, _ = case_to_device(case)
    flags = {"default": 0, "tile": B.DS4HC_FLAG_FORCE_TILE, "splitk": B.DS4HC_FLAG_FORCE_SPLITK}[path]
    say(f"[gpu] ds4hc_partials path={path} T={T} n={n} d_s={ds} {dtype}")
    got = B.ds4hc_partials(X, W, flags=flags)
    torch.cuda.synchronize()
    Xs = wl.state_to_f64(case.X, dtype)
    Ws = np.asarray(case.W, dtype=np.float64)
    ref = oracle.partials(Xs, Ws)
    _check_partials(got.cpu().numpy().astype(np.float64), ref, Xs, Ws, f"partials {path}")


# ------------------------------------------------------------------ 86-site decode chain, eager and graph

def _chain_86(torch, case, b, Ws, noise, states, ins, coeffs, ws, wsb):
    """One decode token through the 86 HC sites (attention and FFN per layer of
    43): HC-pre of site 0, then at every boundary the stand-in layer body
    layer_out = 0.5 * layer_in + noise_s and one ds4hc_post_pre, and hc_post
    after the last site. Every site's input state, layer_in and coefficients
    land in buffers of their own (states[s], ins[s], coeffs[s]); raw calls on the
    current stream with preallocated buffers, so the same code can be captured."""
    import ctypes
    P = ctypes.c_void_p
    pt = lambda t: P(t.data_ptr())
    sp = P(torch.cuda.current_stream().cuda_stream)
    p = B.make_params(case.n, case.d)
    sites = len(Ws)
    st = B.ds4hc_pre_raw(p, 1, B.DS4HC_F32, pt(states[0]), pt(Ws[0]), pt(b), pt(ins[0]), pt(coeffs[0]),
                         None, pt(ws), wsb, sp)
    assert st == B.DS4HC_OK
    lo = torch.empty((1, case.d), device="cuda")
    for s_ in range(sites):
        torch.add(noise[s_][None, :], ins[s_], alpha=0.5, out=lo)
        if s_ + 1 < sites:
            st = B.ds4hc_post_pre_raw(p, 1, B.DS4HC_F32, pt(states[s_]), pt(coeffs[s_]), pt(lo),
                                      pt(Ws[s_ + 1]), pt(b), pt(states[s_ + 1]), pt(ins[s_ + 1]),
                                      pt(coeffs[s_ + 1]), None, pt(ws), wsb, sp)
        else:
            st = B.ds4hc_post_raw(p, 1, B.DS4HC_F32, pt(states[s_]), pt(coeffs[s_]), pt(lo),
                                  pt(states[s_ + 1]), sp)
        assert st == B.DS4HC_OK


def _check_chain_86(case, states, ins, coeffs, ref, what):
    """Every site teacher forced (the oracle's HC-pre and hc_post fed the GPU's own
    input state and layer_out) within 2e-5, and the end state against the
    oracle's whole chain within 2e-5."""
    worst = 0.0
    for s_ in range(len(case.chain_W)):
        Xs = torch_to_f64(states[s_])
        rli, rc, _ = oracle.pre(Xs, case.chain_W[s_], case.bias)
        worst = max(worst, assert_close_rows(torch_to_f64(ins[s_]), rli, TOL[wl.F32], f"{what} site {s_} layer_in"))
        assert_coeffs(coeffs[s_].cpu().numpy(), rc, f"{what} site {s_} coeffs")
        lo = torch_to_f64(ins[s_]) * 0.5 + case.chain_noise[s_].astype(np.float64)[None, :]
        rx = oracle.post(Xs, rc, lo)
        worst = max(worst, assert_close_rows(torch_to_f64(states[s_ + 1]), rx, TOL[wl.F32], f"{what} site {s_} X'"))
    e2e = assert_close_rows(torch_to_f64(states[-1]), ref[-1], TOL[wl.F32], f"{what} end to end")
    say(f"    {what}: teacher-forced worst {worst:.2e}; end-to-end {e2e:.2e} "
        f"(state max |x| {np.abs(ref[-1]).max():.2e})")


def test_decode_chain_86_sites_eager_and_graph():
    """The decode token's 86 HC sites (the pages count 86 HC launches per decoded
    token), T = 1, n = 4, d = 4096, float32, each site with its own f16 fn weight.
    Run eagerly, then captured once as a HIP graph and replayed three times with
    other eager work (the eager chain on other buffers) between the replays. The
    eager run and every replay are checked against the oracle (per site and end
    to end, 2e-5), and every replay is bitwise equal to the eager run."""
    torch = torch_mod()
    case = wl.make_chain(0, layers=86)
    sites = len(case.chain_W)
    b = torch.zeros(case.m, dtype=torch.float32, device="cuda")
    Ws = [torch.from_numpy(w).cuda() for w in case.chain_W]
    noise = torch.from_numpy(case.chain_noise).cuda()
    p = B.make_params(case.n, case.d)
    wsb = max(B.ds4hc_workspace_bytes(p, 1, B.DS4HC_F32), B.ds4hc_post_pre_workspace_bytes(p, 1, B.DS4HC_F32))

    def buffers():
        X0 = state_to_torch(case.X, case.dtype)
        states = [X0] + [torch.empty_like(X0) for _ in range(sites)]
        ins = [torch.empty((1, case.d), device="cuda") for _ in range(sites)]
        coeffs = [torch.empty((1, case.m), device="cuda") for _ in range(sites)]
        return states, ins, coeffs, torch.empty(wsb, dtype=torch.uint8, device="cuda")

    ref = oracle.chain(wl.state_to_f64(case.X, case.dtype), case.chain_W, case.bias, case.chain_noise)
    say("[gpu] decode chain, 86 sites, eager")
    eager = buffers()
    _chain_86(torch, case, b, Ws, noise, *eager, wsb)
    torch.cuda.synchronize()
    _check_chain_86(case, *eager[:3], ref, "eager")

    say("[gpu] decode chain, 86 sites, captured as one HIP graph")
    gbuf = buffers()
    other = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream's allocations once
        _chain_86(torch, case, b, Ws, noise, *gbuf, wsb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _chain_86(torch, case, b, Ws, noise, *gbuf, wsb)
    for rep in range(3):
        for t in gbuf[0][1:] + gbuf[1] + gbuf[2]:
            t.fill_(float("nan"))      # a replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip(gbuf[0] + gbuf[1] + gbuf[2], eager[0] + eager[1] + eager[2]):
            assert torch.equal(a.view(torch.int32), e.view(torch.int32)), f"replay {rep} differs from eager"
        _check_chain_86(case, *gbuf[:3], ref, f"graph replay {rep}")
        _chain_86(torch, case, b, Ws, noise, *other, wsb)   # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ determinism: 20 repeats per workload

def _bits(t):
    import torch
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _sha(ts):
    import hashlib
    h = hashlib.sha256()
    for t in ts:
        h.update(_bits(t).cpu().numpy().tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("workload", ["single", "verify", "prefill", "stress"])
def test_deterministic_20_repeats(workload):
    """The deterministic mode is bit-stable run to run: 20 runs of ds4hc_fused on
    the same inputs, each followed by a call on other inputs of another size (so
    the GPU's caches and workgroup placement differ between repeats), all
    bitwise identical (compared on the GPU as integers, so NaN bits count too),
    with the SHA-256 of the first and the last run's outputs equal."""
    torch = torch_mod()
    case = {"single": wl.make_single, "verify": wl.make_verify, "prefill": wl.make_prefill,
            "stress": wl.make_stress}[workload](5)
    X, W, b, lo = case_to_device(case)
    noise_case = wl.make_random(99, 37, case.n, case.d, case.dtype)
    Xn, Wn, bn, lon = case_to_device(noise_case)
    say(f"[gpu] 20 repeats of ds4hc_fused, {workload} T={case.T} d={case.d} {case.dtype}, "
        f"flags=DETERMINISTIC")
    fl = B.DS4HC_FLAG_DETERMINISTIC
    first = B.ds4hc_fused(X, W, b, lo, flags=fl)
    torch.cuda.synchronize()
    h0 = _sha(first)
    for r in range(1, 20):
        B.ds4hc_fused(Xn, Wn, bn, lon, flags=fl)
        outs = B.ds4hc_fused(X, W, b, lo, flags=fl)
        torch.cuda.synchronize()
        for a, e in zip(outs, first):
            assert torch.equal(_bits(a), _bits(e)), f"repeat {r} differs"
        if r == 19:
            assert _sha(outs) == h0
        del outs
    say(f"    sha256 {h0[:16]}... stable over 20 runs")


@pytest.mark.parametrize("T", [4096, 37])
def test_deterministic_20_repeats_split_over_d(T):
    """The split over d is bit-stable run to run: 20 runs of ds4hc_partials on one
    1024-column share of the prefill state (T = 4096: the streamed kernel; T = 37:
    split-K), each after a call on other inputs, and the combine of the four shares'
    partials, all bitwise identical."""
    torch = torch_mod()
    case = wl.make_prefill(5, T=T)
    X, W, b, lo, sh = _shares(case, 4)
    noise = wl.make_random(98, 53, case.n, 1024, case.dtype)
    Xn, Wn, _, _ = case_to_device(noise)
    say(f"[gpu] 20 repeats of ds4hc_partials + ds4hc_combine, prefill share T={T}")
    fl = B.DS4HC_FLAG_DETERMINISTIC

    def run():
        P = torch.stack([B.ds4hc_partials(xs, ws, flags=fl) for xs, ws, _ in sh])
        out = B.ds4hc_combine(P, b, sh[0][0], sh[0][2], case.d)
        return (P,) + tuple(out)

    first = run()
    torch.cuda.synchronize()
    h0 = _sha(first)
    for r in range(1, 20):
        B.ds4hc_partials(Xn, Wn, flags=fl)
        outs = run()
        torch.cuda.synchronize()
        for a, e in zip(outs, first):
            assert torch.equal(_bits(a), _bits(e)), f"repeat {r} differs"
        if r == 19:
            assert _sha(outs) == h0
        del outs
    say(f"    sha256 {h0[:16]}... stable over 20 runs")


def test_deterministic_20_repeats_chain():
    """The 43-layer decode chain (ds4hc_pre, then one ds4hc_post_pre per layer
    boundary, then ds4hc_post), 20 runs: every layer's layer_in and coefficients
    and the end state bitwise identical run to run."""
    torch = torch_mod()
    case = wl.make_chain(5)
    b = torch.zeros(case.m, dtype=torch.float32, device="cuda")
    Ws = [torch.from_numpy(w).cuda() for w in case.chain_W]
    noise = torch.from_numpy(case.chain_noise).cuda()
    say("[gpu] 20 repeats of the 43-layer decode chain")

    def run():
        X = state_to_torch(case.X, case.dtype)
        li, c, _ = B.ds4hc_pre(X, Ws[0], b)
        outs = []
        for l in range(len(Ws)):
            outs += [li, c]
            lo = li * 0.5 + noise[l][None, :]
            if l + 1 < len(Ws):
                X, li, c, _ = B.ds4hc_post_pre(X, c, lo, Ws[l + 1], b)
            else:
                X = B.ds4hc_post(X, c, lo)
        torch.cuda.synchronize()
        return outs + [X]

    first = run()
    h0 = _sha(first)
    for r in range(1, 20):
        outs = run()
        for a, e in zip(outs, first):
            assert torch.equal(_bits(a), _bits(e)), f"repeat {r} differs"
    assert _sha(outs) == h0
    say(f"    sha256 {h0[:16]}... stable over 20 runs")


# ------------------------------------------------------------------ calls on a side stream

def test_side_stream_matches_default_stream():
    """The binding's stream= argument: ds4hc_fused (split-K, whose workspace the
    binding allocates and drops) and ds4hc_post_pre at T = 1 enqueued on a side
    stream, with the default stream kept busy meanwhile, give bitwise what the
    same calls give on the default stream."""
    torch = torch_mod()
    case = wl.make_verify(21, T=1)
    X, W, b, lo = case_to_device(case)
    nxt = wl.make_random(1021, 1, case.n, case.d, case.dtype)
    Wn = torch.from_numpy(nxt.W).cuda()
    bn = torch.from_numpy(nxt.bias).cuda()
    say("[gpu] ds4hc_fused / ds4hc_post_pre on a side stream, T=1")
    ref_f = B.ds4hc_fused(X, W, b, lo)
    ref_pp = B.ds4hc_post_pre(X, ref_f[1], lo, Wn, bn)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    big = torch.empty(1 << 26, device="cuda")
    for rep in range(20):
        got_f = B.ds4hc_fused(X, W, b, lo, stream=s)
        got_pp = B.ds4hc_post_pre(X, got_f[1], lo, Wn, bn, stream=s)
        big.fill_(float(rep))      # default-stream work that allocates meanwhile
        junk = torch.empty(1 << 20, device="cuda").fill_(1.0)
        torch.cuda.synchronize()
        for a, e in zip(got_f + got_pp[:3], ref_f + ref_pp[:3]):
            assert torch.equal(_bits(a), _bits(e)), f"side-stream repeat {rep} differs"
        del junk

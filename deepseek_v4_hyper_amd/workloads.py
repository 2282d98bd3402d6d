"""Seeded synthetic inputs for the DeepSeek-V4 hyper-connection (HC) op.

This module only draws random numbers and casts them to storage types. It
holds none of the op's arithmetic, so both the fp64 oracle and the HIP path
can be fed from it without sharing any computation.

Workloads (the op is per-token, so T is the only size that changes between a
decode step and a prefill):

* ``single``  T=1, n_hc=4, d=256, fp32 state.
* ``chain``   T=1, n_hc=4, d=4096, 43 layers, each with its own fn weight,
              plus per-layer noise that stands in for the layer body.
              (The model has 43 layers: lucebox PR #507 "correct layer-split
              HC handoff and per-device state", Validation, split [0,22)/[22,43).)
* ``verify``  T=4 (a q=4 speculative verify batch; lucebox PR #496 "DSpark
              speculative runtime", adaptive q=2/3/4 verification), d=4096, fp32.
* ``prefill`` T=4096, d=4096, fp32 state with a per-token scale drawn
              log-uniform in [0.1, 10].
* ``stress``  T=16384, d=7168, bf16 state, residual logits of std ~20, 5 % of
              token rows all zero.

Draw order per workload, from one ``numpy.random.Generator(PCG64(seed))``:
X, then (prefill) the per-token scales, then W (one per layer for the chain),
then layer_out (not for the chain), then (stress) the zero-row indices, then
(chain) the per-layer noise. Large arrays are drawn directly in float32.
``N(mu, s)`` means standard deviation ``s``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"
DEFAULT_EPS = 1e-6
DEFAULT_ITERS = 20


def n_logits(n_hc: int) -> int:
    """Number of fn-projection outputs: n pre gates, n post gates, n*n residual."""
    return 2 * n_hc + n_hc * n_hc


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    quiet = ((u >> 16) | 0x0040).astype(np.uint16)
    return np.where(nan, quiet, rounded)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def state_to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 view of a state array stored as float32 or bf16 bits."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


@dataclass
class HCCase:
    """One synthetic HC-op input set in storage types.

    X         [T, n, d]  float32, or uint16 bf16 bits when dtype == "bf16"
    W         [m, n*d]   float16 (m = 2n + n*n), row-major
    bias      [m]        float32
    layer_out [T, d]     same storage as X (None for the chain)
    chain_W   list of per-layer W (chain only), chain_noise [L, d] float32
    """

    name: str
    T: int
    n: int
    d: int
    dtype: str
    X: np.ndarray
    W: np.ndarray
    bias: np.ndarray
    layer_out: np.ndarray | None
    eps: float = DEFAULT_EPS
    iters: int = DEFAULT_ITERS
    chain_W: list = field(default_factory=list)
    chain_noise: np.ndarray | None = None
    zero_rows: np.ndarray | None = None

    @property
    def m(self) -> int:
        return n_logits(self.n)

    @property
    def K(self) -> int:
        return self.n * self.d


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _weight(rng, n, d, std=0.02, residual_std=None):
    m, K = n_logits(n), n * d
    w = _normal(rng, (m, K), std)
    if residual_std is not None:
        w[2 * n:] *= np.float32(residual_std / std)
    return w.astype(np.float16)


def _cast_state(x32: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x32) if dtype == F32 else f32_to_bf16_bits(x32)


def make_single(seed: int = 0, T: int = 1, n: int = 4, d: int = 256) -> HCCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    W = _weight(rng, n, d)
    lo = _normal(rng, (T, d))
    return HCCase("single", T, n, d, F32, X, W, np.zeros(n_logits(n), np.float32), lo)


def make_verify(seed: int = 0, T: int = 4, n: int = 4, d: int = 4096) -> HCCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    W = _weight(rng, n, d)
    lo = _normal(rng, (T, d))
    return HCCase("verify", T, n, d, F32, X, W, np.zeros(n_logits(n), np.float32), lo)


def make_prefill(seed: int = 0, T: int = 4096, n: int = 4, d: int = 4096) -> HCCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    scale = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=T)).astype(np.float32)
    X *= scale[:, None, None]
    W = _weight(rng, n, d)
    lo = _normal(rng, (T, d))
    return HCCase("prefill", T, n, d, F32, X, W, np.zeros(n_logits(n), np.float32), lo)


def make_stress(seed: int = 0, T: int = 16384, n: int = 4, d: int = 7168,
                zero_frac: float = 0.05) -> HCCase:
    """bf16 state; residual fn rows scaled so the residual logits have std ~20."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    K = n * d
    W = _weight(rng, n, d, residual_std=20.0 / np.sqrt(K))
    lo = _normal(rng, (T, d))
    nz = int(round(zero_frac * T))
    zero_rows = np.sort(rng.choice(T, nz, replace=False)) if nz else np.zeros(0, np.int64)
    X[zero_rows] = 0.0
    return HCCase("stress", T, n, d, BF16, f32_to_bf16_bits(X), W,
                  np.zeros(n_logits(n), np.float32), f32_to_bf16_bits(lo),
                  zero_rows=zero_rows)


def make_chain(seed: int = 0, layers: int = 43, T: int = 1, n: int = 4, d: int = 4096) -> HCCase:
    """Decode chain: X_0, then one fn weight per layer, then per-layer noise N(0, 0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    Ws = [_weight(rng, n, d) for _ in range(layers)]
    noise = _normal(rng, (layers, d), 0.1)
    return HCCase("chain", T, n, d, F32, X, Ws[0], np.zeros(n_logits(n), np.float32), None,
                  chain_W=Ws, chain_noise=noise)


def make_random(seed: int, T: int, n: int, d: int, dtype: str = F32,
                w_std: float = 0.02, lo_std: float = 1.0) -> HCCase:
    """Generic case for shape sweeps and edge cases (same draw order as above)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _normal(rng, (T, n, d))
    W = _weight(rng, n, d, std=w_std)
    lo = _normal(rng, (T, d), lo_std)
    return HCCase(f"random_n{n}_d{d}_T{T}", T, n, d, dtype, _cast_state(X, dtype), W,
                  np.zeros(n_logits(n), np.float32), _cast_state(lo, dtype))


WORKLOADS = {
    "single": make_single,
    "chain": make_chain,
    "verify": make_verify,
    "prefill": make_prefill,
    "stress": make_stress,
}

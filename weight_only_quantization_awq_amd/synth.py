"""Seeded synthetic layer inputs for the AWQ per-layer path.

This module only draws random numbers and stores them in the input formats
the library accepts (fp32, or fp32 values that are exactly representable in
bfloat16).  It holds none of the method's arithmetic: no statistics, scales,
quantisation, losses or packing.  Both the CPU oracle's tests and the GPU
path are fed from here, so the two sides see identical bytes.

Shapes and value distributions stand in for the LLaMA/OPT projection layers
that the AWQ pages calibrate on Pile samples (those models and data are not
available): X is [N x D_in] with a few large "salient" input channels or a
heavy-tailed per-channel spread, W is [D_in x D_out] Gaussian.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerCase",
    "alpha_grid",
    "to_bf16_values",
    "bf16_bits",
    "make_layer",
    "config_case",
    "decode_x",
    "CONFIG_NAMES",
]


def alpha_grid(n: int = 21) -> np.ndarray:
    """The caller-supplied alpha grid {0, 1/(n-1), ..., 1} as float32."""
    if n == 1:
        return np.zeros(1, np.float32)
    return (np.arange(n, dtype=np.float64) / (n - 1)).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-half-to-even.

    Used only to store generated inputs in bf16; NaN is not expected here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array of values exactly representable in bf16 (RNE storage)."""
    b = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).reshape(np.shape(x))


@dataclass
class LayerCase:
    """One synthetic linear layer: X [N x D_in], W [D_in x D_out].

    ``X`` and ``W`` are float32 arrays; when ``dtype == "bf16"`` every value is
    exactly representable in bfloat16 and the GPU receives the bf16 bits.
    """

    name: str
    X: np.ndarray
    W: np.ndarray
    dtype: str  # "f32" or "bf16"
    bits: int
    group: int
    alphas: np.ndarray = field(default_factory=alpha_grid)
    salient: np.ndarray | None = None

    @property
    def N(self) -> int:
        return self.X.shape[0]

    @property
    def D_in(self) -> int:
        return self.X.shape[1]

    @property
    def D_out(self) -> int:
        return self.W.shape[1]


def make_layer(
    N: int,
    D_in: int,
    D_out: int,
    *,
    seed: int,
    dtype: str = "bf16",
    bits: int = 4,
    group: int = 128,
    x_kind: str = "salient",
    n_salient: int = 0,
    salient_lo: float = 20.0,
    salient_hi: float | None = None,
    w_std: float = 0.02,
    t_nu: float = 4.0,
    lognorm_sigma: float = 1.0,
    n_alpha: int = 21,
    name: str = "custom",
) -> LayerCase:
    """Draw one layer.  Draw order: X, salient indices, salient factors, W.

    x_kind:
      "salient"   X ~ N(0,1); ``n_salient`` seed-chosen channels multiplied by
                  a factor (fixed ``salient_lo`` if ``salient_hi`` is None,
                  else log-uniform in [salient_lo, salient_hi]).
      "heavy"     X = Student-t(nu) per element times a per-channel magnitude
                  drawn LogNormal(0, sigma).
    """
    rng = np.random.default_rng(seed)
    sal = None
    if x_kind == "salient":
        X = rng.standard_normal((N, D_in), dtype=np.float32)
        if n_salient:
            sal = np.sort(rng.choice(D_in, n_salient, replace=False))
            if salient_hi is None:
                f = np.full(n_salient, salient_lo, np.float32)
            else:
                f = np.exp(rng.uniform(np.log(salient_lo), np.log(salient_hi), n_salient)).astype(np.float32)
            X[:, sal] *= f[None, :]
    elif x_kind == "heavy":
        X = rng.standard_t(t_nu, size=(N, D_in)).astype(np.float32)
        mag = rng.lognormal(0.0, lognorm_sigma, D_in).astype(np.float32)
        X *= mag[None, :]
    else:
        raise ValueError(f"unknown x_kind {x_kind!r}")
    W = rng.standard_normal((D_in, D_out), dtype=np.float32) * np.float32(w_std)
    if dtype == "bf16":
        X = to_bf16_values(X)
        W = to_bf16_values(W)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return LayerCase(name, np.ascontiguousarray(X), np.ascontiguousarray(W), dtype, bits, group,
                     alpha_grid(n_alpha), sal)


CONFIG_NAMES = {
    1: "single layer 256x256, N=128, fp32, INT4 g128",
    2: "attention projection 4096x4096, N=2048, bf16, INT4 g128",
    3: "MLP up-projection 4096x11008, N=4096, bf16, INT4 g128",
    4: "MLP down-projection 11008x4096, N=4096, bf16, INT3 g128",
    5: "large layer 8192x28672, N=4096, bf16, INT4 g128",
}


def config_case(cfg: int, *, seed: int | None = None, n_tokens: int | None = None) -> LayerCase:
    """The five benchmark layers (seed defaults to 1000 + cfg).

    ``n_tokens`` overrides N (used to draw bounded samples of a workload).
    """
    seed = 1000 + cfg if seed is None else seed
    if cfg == 1:
        return make_layer(n_tokens or 128, 256, 256, seed=seed, dtype="f32", n_salient=3,
                          salient_lo=20.0, w_std=0.02, name="cfg1")
    if cfg == 2:
        return make_layer(n_tokens or 2048, 4096, 4096, seed=seed, dtype="bf16", n_salient=41,
                          salient_lo=10.0, salient_hi=100.0, w_std=0.02, name="cfg2")
    if cfg == 3:
        return make_layer(n_tokens or 4096, 4096, 11008, seed=seed, dtype="bf16", x_kind="heavy",
                          w_std=0.02, name="cfg3")
    if cfg == 4:
        return make_layer(n_tokens or 4096, 11008, 4096, seed=seed, dtype="bf16", x_kind="heavy",
                          w_std=0.015, bits=3, name="cfg4")
    if cfg == 5:
        return make_layer(n_tokens or 4096, 8192, 28672, seed=seed, dtype="bf16", n_salient=82,
                          salient_lo=50.0, w_std=0.01, name="cfg5a")
    raise ValueError(f"unknown config {cfg}")


def decode_x(M: int, D_in: int = 8192, *, seed: int | None = None) -> np.ndarray:
    """Decode-time activations X ~ N(0,1), bf16 values, [M x D_in]."""
    rng = np.random.default_rng(1050 + M if seed is None else seed)
    return to_bf16_values(rng.standard_normal((M, D_in), dtype=np.float32))

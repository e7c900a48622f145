"""Seeded synthetic inputs for the rotated W2A4 linear and the KV4 quantizer.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark. It draws random numbers and shapes only: it contains none of the
method's arithmetic (no rotation, no scale rule, no rounding to codes, no
packing). Everything the pages fix about the inputs is the source model of the
Qift abstract (page "Qift: Shift-Friendly No-Zero W2 Post-Training
Quantization for Rotated W2A4/KV4 LLM Inference", abstract): rotated weights
behave like zero-centred Gaussians. The sizes below are LLaMA-2-7B and
LLaMA-3.1-8B linear shapes (the abstract counts 224 linear modules per model,
i.e. 32 layers x 7 linears).

Distributions used:

* weights: i.i.d. N(0, sigma^2), sigma = 0.02 (LLaMA-7B-shaped) or 0.015
  (LLaMA-3.1-8B-shaped);
* activations: i.i.d. N(0, 1) with a fixed set of outlier channels scaled by
  20 (4 channels for the 16x256 case, round(0.01*K) channels otherwise);
* KV: i.i.d. N(0, 1) in bf16, [T, H, D];
* calibration activations (error-compensated weight quantization): N(0, 1)
  plus a shared rank-8 part, outlier channels x20.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------

#: one LLaMA-2-7B decoder layer: (name, K_in, N_out, hadamard block along K)
LLAMA7B_LAYER = (
    ("q_proj", 4096, 4096, 4096),
    ("k_proj", 4096, 4096, 4096),
    ("v_proj", 4096, 4096, 4096),
    ("o_proj", 4096, 4096, 4096),
    ("gate_proj", 4096, 11008, 4096),
    ("up_proj", 4096, 11008, 4096),
    ("down_proj", 11008, 4096, 256),
)

#: one LLaMA-3.1-8B decoder layer (grouped-query k/v)
LLAMA31_8B_LAYER = (
    ("q_proj", 4096, 4096, 4096),
    ("k_proj", 4096, 1024, 4096),
    ("v_proj", 4096, 1024, 4096),
    ("o_proj", 4096, 4096, 4096),
    ("gate_proj", 4096, 14336, 4096),
    ("up_proj", 4096, 14336, 4096),
    ("down_proj", 14336, 4096, 1024),
)

N_LAYERS = 32


def n_outlier_channels(K: int) -> int:
    """round(0.01 * K): 41, 110 and 143 for K = 4096, 11008 and 14336."""
    return int(round(0.01 * K))


# --------------------------------------------------------------------------
# numpy generators (CPU; used by the oracle side and copied to the GPU side)
# --------------------------------------------------------------------------

def small_linear_case():
    """The CPU-sized single linear: W [256, 256] ~ N(0, 0.02^2), X [16, 256]
    ~ N(0, 1) with 4 seeded outlier channels x20. Drawn in this order from
    ``numpy.random.default_rng(0)``: W, X, then the outlier channels.
    Returns float32 arrays (W, X, channels)."""
    rng = np.random.default_rng(0)
    W = rng.normal(0.0, 0.02, size=(256, 256))
    X = rng.standard_normal((16, 256))
    ch = rng.choice(256, 4, replace=False)
    X[:, ch] *= 20.0
    return W.astype(np.float32), X.astype(np.float32), np.sort(ch)


def activations(M: int, K: int, seed: int, n_outliers: int | None = None,
                outlier_gain: float = 20.0) -> np.ndarray:
    """float32 [M, K] ~ N(0, 1) with ``n_outliers`` (default round(0.01 K))
    seeded channels multiplied by ``outlier_gain``, the same channels for
    every token."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    n = n_outlier_channels(K) if n_outliers is None else n_outliers
    if n > 0:
        ch = rng.choice(K, n, replace=False)
        X[:, ch] *= outlier_gain
    return X.astype(np.float32)


def calibration_activations(S: int, K: int, seed: int, rank: int = 8,
                            n_outliers: int | None = None,
                            outlier_gain: float = 20.0) -> np.ndarray:
    """float32 [S, K] calibration tokens: i.i.d. N(0, 1) plus a shared
    low-rank part G V (G [S, rank], V [rank, K], both N(0, 1)), so that the
    features are correlated, with ``n_outliers`` (default round(0.01 K))
    seeded channels multiplied by ``outlier_gain``."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((S, K))
    if rank > 0:
        X += rng.standard_normal((S, rank)) @ rng.standard_normal((rank, K))
    n = n_outlier_channels(K) if n_outliers is None else n_outliers
    if n > 0:
        ch = rng.choice(K, n, replace=False)
        X[:, ch] *= outlier_gain
    return X.astype(np.float32)


def weights(N: int, K: int, seed: int, sigma: float = 0.02) -> np.ndarray:
    """float32 [N, K] ~ N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, sigma, size=(N, K)).astype(np.float32)


def heavy_tailed_weights(N: int, K: int, seed: int, dof: float = 3.0,
                         sigma: float = 0.02) -> np.ndarray:
    """float32 [N, K] Student-t rows (excess kurtosis >> 0), scaled to sigma.
    Used to show that the rotation makes a heavy-tailed row close to Gaussian."""
    rng = np.random.default_rng(seed)
    return (sigma * rng.standard_t(dof, size=(N, K))).astype(np.float32)


def kv(T: int, H: int, D: int, seed: int) -> np.ndarray:
    """float32 [T, H, D] ~ N(0, 1) (callers round to bf16 for the KV4 path)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, D)).astype(np.float32)


def uniform_codes(shape, n_values: int, seed: int) -> np.ndarray:
    """int64 array of uniformly drawn integers in [0, n_values)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_values, size=shape, dtype=np.int64)


def uniform_int4(shape, seed: int, lo: int = -7, hi: int = 7) -> np.ndarray:
    """int64 array of uniformly drawn integers in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64)


def subnormal_rows(R: int, K: int, seed: int) -> np.ndarray:
    """float32 [R, K] rows at the bottom of the float32 range: row r holds
    integer multiples of 2^-149 (the smallest subnormal) drawn uniformly in
    [-m, m], m = 1 + (r mod 64), with +-m placed at one seeded position, so
    the rows' absmax values run over m * 2^-149 for m = 1..64."""
    rng = np.random.default_rng(seed)
    tiny = np.float32(2.0 ** -149)
    X = np.zeros((R, K), np.float32)
    for r in range(R):
        m = 1 + r % 64
        k = rng.integers(-m, m + 1, K)
        k[rng.integers(0, K)] = m if rng.integers(0, 2) else -m
        X[r] = k.astype(np.float32) * tiny
    return X


def positive_scales(n: int, seed: int, lo: float = 0.01, hi: float = 2.0) -> np.ndarray:
    """float32 [n] drawn uniformly in [lo, hi)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=n).astype(np.float32)


# --------------------------------------------------------------------------
# torch helpers (dtype conversion and device-side draws for the large sizes)
# --------------------------------------------------------------------------

def to_bf16(x: np.ndarray):
    """torch.bfloat16 CPU tensor holding ``x`` rounded to bf16."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_values(t) -> np.ndarray:
    """float64 numpy copy of a bf16 (or any float) torch tensor, exactly."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def device_weights(N: int, K: int, seed: int, sigma: float, device):
    """float32 [N, K] ~ N(0, sigma^2) drawn on ``device`` with a seeded
    torch.Generator (used where the host draw would be too slow)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32).mul_(sigma)


def device_activations(M: int, K: int, seed: int, device, n_outliers: int | None = None,
                       outlier_gain: float = 20.0):
    """bf16 [M, K] ~ N(0, 1) on ``device`` with seeded outlier channels x20."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    n = n_outlier_channels(K) if n_outliers is None else n_outliers
    if n > 0:
        gc = torch.Generator(device="cpu")
        gc.manual_seed(int(seed) + 7919)
        ch = torch.randperm(K, generator=gc)[:n].to(device)
        x[:, ch] *= outlier_gain
    return x.to(torch.bfloat16)


def device_kv(T: int, H: int, D: int, seed: int, device):
    """bf16 [T, H, D] ~ N(0, 1) on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((T, H, D), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

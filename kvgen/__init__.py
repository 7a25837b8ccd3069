"""Seeded synthetic K/V/q generators shared by the tests and the bench.

This module draws inputs only; it holds none of the codec's arithmetic
(no rotation, codebook, quantisation or attention).  Every generator takes
an explicit integer seed and a torch device, so the same call reproduces the
same tensor on that device.  Shapes and value distributions follow the
workloads the pages describe:

* iid N(0, 1) rows (the Foundry spec's "Synthetic (Gaussian)" quality rows);
* unit-norm random directions scaled by lognormal norms (the Engine spec's
  accuracy contract is stated on unit vectors of random direction);
* channel-correlated rows with a few large outlier channels (the Foundry
  spec's "Realistic (correlated)" column; real K/V are not available here);
* heavy-tailed Student-t rows.
"""
from __future__ import annotations

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """iid N(0, 1) values, rounded to ``dtype`` (bf16 rounding is RNE)."""
    x = torch.randn(*shape, generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    return x.to(dtype)


def unit_dirs_lognormal(shape, seed: int, device="cpu", sigma: float = 0.5,
                        dtype=torch.float32) -> torch.Tensor:
    """Rows z/||z|| * exp(sigma * eps): a uniformly random direction with a
    lognormal(0, sigma) length.  ``shape[-1]`` is the row length."""
    g = _gen(seed, device)
    z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    eps = torch.randn(*shape[:-1], 1, generator=g, device=device, dtype=torch.float32)
    z = z / torch.linalg.vector_norm(z, dim=-1, keepdim=True)
    return (z * torch.exp(sigma * eps)).to(dtype)


def ar1_outliers(shape, seed: int, device="cpu", rho: float = 0.6,
                 n_outliers: int = 4, outlier_scale: float = 8.0,
                 dtype=torch.bfloat16) -> torch.Tensor:
    """Rows with AR(1) correlation along the channel axis,
    x_0 = e_0, x_i = rho x_{i-1} + sqrt(1 - rho^2) e_i, and ``n_outliers``
    channels per head scaled by ``outlier_scale``.

    ``shape`` = (layers, heads, tokens, d); the outlier channels are drawn per
    (layer, head) by a seeded random permutation."""
    L, H, T, d = shape
    g = _gen(seed, device)
    e = torch.randn(L, H, T, d, generator=g, device=device, dtype=torch.float32)
    # x = e @ A^T with A[i, j] = c_j rho^(i-j) for j <= i (c_0 = 1, else sqrt(1-rho^2))
    i = torch.arange(d, device=device, dtype=torch.float32)
    expo = (i[:, None] - i[None, :])
    A = torch.where(expo >= 0, rho ** expo.clamp(min=0), torch.zeros_like(expo))
    c = torch.full((d,), (1.0 - rho * rho) ** 0.5, device=device)
    c[0] = 1.0
    A = A * c[None, :]
    x = torch.matmul(e.reshape(-1, d), A.t().contiguous()).reshape(L, H, T, d)
    del e
    keys = torch.rand(L, H, d, generator=g, device=device)
    chans = keys.argsort(dim=-1)[..., :n_outliers]          # [L, H, n_outliers]
    scale = torch.ones(L, H, d, device=device)
    scale.scatter_(-1, chans, outlier_scale)
    x.mul_(scale[:, :, None, :])
    return x.to(dtype)


def student_t(shape, seed: int, nu: int = 3, device="cpu",
              dtype=torch.bfloat16) -> torch.Tensor:
    """iid Student-t(nu) values e / sqrt(chi2_nu / nu), chi2 as a sum of nu
    squared normals (integer nu)."""
    g = _gen(seed, device)
    e = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros_like(e)
    for _ in range(nu):
        z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        chi2.addcmul_(z, z)
    return (e / torch.sqrt(chi2 / nu)).to(dtype)

"""Seeded smooth-field + noise Q/K/V for a latent video grid.

Recipe (all draws from one seeded torch generator, in this fixed order):
  1. 16 spatio-temporal frequencies f_j in cycles per (frame, row, column),
     f_j ~ N(0, diag(1/8^2, 1/32^2, 1/32^2)), and phases b_j ~ U[0, 2*pi);
     they are shared by Q, K, V and all heads (the "content").
  2. Fourier features phi_j(t, y, x) = cos(2*pi*f_j . (t, y, x) + b_j) over the
     real tokens in raster order (t, y, x).
  3. Per head, for X in (Q, K, V) in that order: a map W_X ~ N(0,1)^{16 x d}
     and noise eps ~ N(0, 0.5^2)^{T*H*W x d}.
  4. X = (amplitude * phi @ W_X + eps) / sqrt(d), formed in float64, rounded
     to float32, then (for bf16 workloads) to bfloat16 round-to-nearest-even.
The output is raster order [batch, heads, T*H*W, d].
"""
from __future__ import annotations

import math

import numpy as np

import torch


def round_to_bf16(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bfloat16 with round-to-nearest-even (torch's conversion)."""
    return x.to(torch.float32).to(torch.bfloat16)


def fourier_video_qkv(T: int, H: int, W: int, heads: int, d: int, amplitude: float = 1.0,
                      seed: int = 0, dtype: str = "f32", batch: int = 1,
                      device: str | torch.device = "cpu"):
    """Return (q, k, v) raster tensors [batch, heads, T*H*W, d] of ``dtype``.

    dtype: "f32" or "bf16". Generation happens on ``device`` (the GPU for large
    workloads); the same seed gives the same tensors on the same device type.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    f64 = torch.float64
    std = torch.tensor([1 / 8, 1 / 32, 1 / 32], dtype=f64, device=dev)
    freqs = torch.randn(16, 3, generator=gen, dtype=f64, device=dev) * std
    phases = torch.rand(16, generator=gen, dtype=f64, device=dev) * (2 * math.pi)
    t, y, x = torch.meshgrid(torch.arange(T, dtype=f64, device=dev),
                             torch.arange(H, dtype=f64, device=dev),
                             torch.arange(W, dtype=f64, device=dev), indexing="ij")
    coords = torch.stack([t.reshape(-1), y.reshape(-1), x.reshape(-1)], dim=1)   # [THW, 3]
    phi = torch.cos(2 * math.pi * coords @ freqs.T + phases)                   # [THW, 16]
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = T * H * W
    outs = [torch.empty(batch, heads, n, d, dtype=out_dtype, device=dev) for _ in range(3)]
    inv = 1.0 / math.sqrt(d)
    for b in range(batch):
        for h in range(heads):
            for X in range(3):
                w = torch.randn(16, d, generator=gen, dtype=f64, device=dev)
                eps = torch.randn(n, d, generator=gen, dtype=f64, device=dev) * 0.5
                val = ((amplitude * (phi @ w) + eps) * inv).to(torch.float32)
                outs[X][b, h] = val.to(out_dtype)
    return tuple(outs)


def gaussian_video_qkv(T: int, H: int, W: int, heads: int, d: int, seed: int = 0,
                       v_std: float = 0.5, dtype: str = "bf16", batch: int = 1,
                       device: str | torch.device = "cpu"):
    """Token-independent inputs on a latent video grid: Q and K ~ N(0, 1) and
    V ~ N(0, v_std^2) per element, raster order [batch, heads, T*H*W, d].

    Unlike ``fourier_video_qkv`` neighbouring tokens share nothing, so with a
    softmax scale of a few units over sqrt(d) each query's weights concentrate
    on a handful of keys (logits spread over tens of units in base 2). Draws
    from one seeded torch generator: per batch and head, Q, K, V in that order.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = T * H * W
    outs = [torch.empty(batch, heads, n, d, dtype=out_dtype, device=dev) for _ in range(3)]
    for b in range(batch):
        for h in range(heads):
            for X, std in enumerate((1.0, 1.0, v_std)):
                val = torch.randn(n, d, generator=gen, dtype=torch.float32, device=dev) * std
                outs[X][b, h] = val.to(out_dtype)
    return tuple(outs)


def gaussian_mixture_qk(n: int, heads: int, d: int, components: int = 64, spread: float = 0.15,
                        amplitude: float = 1.0, seed: int = 0, dtype: str = "bf16",
                        device: str | torch.device = "cpu"):
    """Q and K drawn from a seeded Gaussian mixture in R^d (recoverable clusters).

    Per head: ``components`` centres c_m of norm ``amplitude`` (random
    directions); every token picks a centre uniformly and adds N(0, (amplitude
    * spread)^2 / d) per coordinate. Q and K share the centres of their head
    but draw memberships and noise independently. Returns (q, k) [1, heads, n, d].
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    f64 = torch.float64
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.empty(1, heads, n, d, dtype=out_dtype, device=dev)
    k = torch.empty(1, heads, n, d, dtype=out_dtype, device=dev)
    for h in range(heads):
        c = torch.randn(components, d, generator=gen, dtype=f64, device=dev)
        c = amplitude * c / c.norm(dim=1, keepdim=True)
        for dst in (q, k):
            member = torch.randint(0, components, (n,), generator=gen, device=dev)
            noise = torch.randn(n, d, generator=gen, dtype=f64, device=dev) * (
                amplitude * spread / math.sqrt(d))
            dst[0, h] = (c[member] + noise).to(torch.float32).to(out_dtype)
    return q, k


def kmeans_init_indices(n: int, clusters: int, heads: int, seed: int = 0) -> np.ndarray:
    """Seeded k-means initialisation draw: ``clusters`` distinct token indices
    per head, int32 [heads, clusters] (numpy PCG64)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(n, clusters, replace=False) for _ in range(heads)]).astype(np.int32)

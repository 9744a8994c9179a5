"""Seeded synthetic workloads generated directly on the GPU (torch Philox).

For the large workloads (hundreds of millions of vectors) host generation and
upload would dominate; these generators draw the same laws as the host
generators in ``synth`` on the device. Deterministic in (seed, stream) for a
given torch version. The CPU baseline copies the rows it samples back to the
host, so the oracle always sees exactly the values the GPU saw.
"""
from __future__ import annotations

import torch


def generator(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cuda")
    g.manual_seed((int(seed) * 1000003 + int(stream) * 7919) & 0x7FFFFFFFFFFFFFFF)
    return g


def lognormal_norm_vectors(n: int, d: int, seed: int, sigma: float = 0.5, chunk: int = 1 << 21,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [n, d]: x = l g / |g|, g ~ N(0, I_d), l ~ LogNormal(0, sigma)."""
    gen = generator(seed, 0)
    if out is None:
        out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        g = torch.randn((hi - lo, d), generator=gen, device="cuda", dtype=torch.float32)
        ell = torch.exp(sigma * torch.randn((hi - lo, 1), generator=gen, device="cuda", dtype=torch.float32))
        out[lo:hi] = (g * (ell / g.norm(dim=1, keepdim=True))).to(torch.bfloat16)
    return out


def kv_with_outliers(B: int, H: int, T: int, d: int, n_out: int, scale: float, seed: int, stream: int,
                     chunk_tokens: int = 1 << 16) -> torch.Tensor:
    """bf16 [B, H, T, d]: N(0, 1) entries, n_out seeded channels per KV head scaled by `scale`."""
    gen = generator(seed, stream)
    out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    ch = torch.stack([torch.randperm(d, generator=gen, device="cuda")[:n_out] for _ in range(H)])
    mult = torch.ones((H, d), device="cuda")
    mult.scatter_(1, ch, scale)
    for b in range(B):
        for lo in range(0, T, chunk_tokens):
            hi = min(T, lo + chunk_tokens)
            x = torch.randn((H, hi - lo, d), generator=gen, device="cuda", dtype=torch.float32)
            out[b, :, lo:hi] = (x * mult[:, None, :]).to(torch.bfloat16)
    return out


def gaussian_mixture(n: int, d: int, n_comp: int, seed: int, stream: int, means: torch.Tensor | None = None,
                     chunk: int = 1 << 18, out: torch.Tensor | None = None):
    """fp32 [n, d] unit-normalised draws from a uniform mixture of N(mu_k, I), mu_k ~ N(0, I)."""
    if means is None:
        means = torch.randn((n_comp, d), generator=generator(seed, 99), device="cuda", dtype=torch.float32)
    gen = generator(seed, stream)
    if out is None:
        out = torch.empty((n, d), dtype=torch.float32, device="cuda")
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        comp = torch.randint(0, n_comp, (hi - lo,), generator=gen, device="cuda")
        x = means[comp] + torch.randn((hi - lo, d), generator=gen, device="cuda", dtype=torch.float32)
        out[lo:hi] = x / x.norm(dim=1, keepdim=True)
    return out, means

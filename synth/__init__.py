"""Seeded synthetic inputs for the HiMuon step.

Shared by the tests, the smoke check and the benchmark; holds none of the
method's arithmetic (no normalisation, no Newton-Schulz, no update).

Momentum-gradient matrices follow one recipe: G = U diag(sigma) V^T + 0.01 N(0, 1)
with U (H x r) and V (W x r) Haar-distributed orthonormal columns (QR of a
Gaussian matrix, signs fixed by diag(R), Mezzadri 2007), sigma_i = 1 / i for
i = 1..r and r = min(H, W).  Everything is drawn from torch generators seeded
explicitly, on the device the tensor is made on.
"""
from __future__ import annotations

import torch

# layer stacks: list of (H, W) row-major shapes
STACKS = {
    "single-256x512": [(256, 512)],
    "gpt2-small-12L": [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12,
    "decoder-1b-16L": ([(2048, 2048)] * 4 + [(2048, 8192)] * 2 + [(8192, 2048)]) * 16,
    "llama3-8b-32L": ([(4096, 4096)] * 2 + [(4096, 1024)] * 2 + [(4096, 14336)] * 2
                      + [(14336, 4096)]) * 32,
}


def ragged_shapes(n: int = 24, lo: int = 100, hi: int = 6000, seed: int = 4000):
    """n shapes with H, W uniform in [lo, hi]; multiples of 32 are drawn again so that
    tiles of 64, 128 and 256 all leave ragged edges."""
    g = torch.Generator().manual_seed(seed)
    out = []
    while len(out) < n:
        h, w = (int(v) for v in torch.randint(lo, hi + 1, (2,), generator=g))
        if h % 32 == 0 or w % 32 == 0:
            continue
        out.append((h, w))
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def haar_columns(n: int, k: int, gen: torch.Generator, device, dtype) -> torch.Tensor:
    """n x k matrix with Haar-distributed orthonormal columns (k <= n)."""
    Z = torch.randn(n, k, generator=gen, device=device, dtype=dtype)
    Q, R = torch.linalg.qr(Z)
    d = torch.sign(torch.diagonal(R))
    d[d == 0] = 1
    return Q * d


def power_law_factors(H: int, W: int, seed: int, device="cpu", dtype=torch.float64):
    """(U, sigma, V) of the low-rank part: Haar U, V and sigma_i = 1/i."""
    r = min(H, W)
    g = _gen(seed, device)
    U = haar_columns(H, r, g, device, dtype)
    V = haar_columns(W, r, g, device, dtype)
    sigma = 1.0 / torch.arange(1, r + 1, device=device, dtype=dtype)
    return U, sigma, V


def power_law_matrix(H: int, W: int, seed: int, device="cpu", dtype=torch.float64,
                     noise: float = 0.01, factors=None, noise_seed: int | None = None):
    """G = U diag(1/i) V^T + noise * N(0, 1), shape H x W, in `dtype` on `device`.

    `factors` may pass (U, sigma, V) drawn earlier for this shape (shared between
    matrices of one shape in large stacks); the noise is then drawn from
    `noise_seed` (default: seed).
    """
    work = torch.float64 if torch.device(device).type == "cpu" else torch.float32
    if factors is None:
        U, sigma, V = power_law_factors(H, W, seed, device, work)
        g = _gen(seed + 7919, device) if noise_seed is None else _gen(noise_seed, device)
    else:
        U, sigma, V = factors
        g = _gen(seed if noise_seed is None else noise_seed, device)
    G = (U * sigma) @ V.T
    G += noise * torch.randn(H, W, generator=g, device=device, dtype=work)
    return G.to(dtype)


def weights(H: int, W: int, seed: int, device="cpu", scale: float = 0.02):
    """fp32 master weights W0 = scale * N(0, 1)."""
    g = _gen(seed + 104729, device)
    return scale * torch.randn(H, W, generator=g, device=device, dtype=torch.float32)


def stack_inputs(shapes, seed0: int, device="cpu", state_dtype=torch.bfloat16,
                 share_factors: bool = False):
    """Per-matrix (W, M, G) tensors: W fp32 master weights, M zeros (first step), G
    from the power-law recipe with seed seed0 + index.  With share_factors, the
    Haar factors are drawn once per distinct shape (a transposed shape reuses
    them swapped) and only the noise is drawn per matrix."""
    cache = {}
    out = []
    for i, (H, W) in enumerate(shapes):
        fac = None
        if share_factors:
            key = (H, W)
            if key not in cache and (W, H) in cache:
                U, s, V = cache[(W, H)]
                cache[key] = (V, s, U)
            if key not in cache:
                work = torch.float64 if torch.device(device).type == "cpu" else torch.float32
                cache[key] = power_law_factors(H, W, seed0 + 100000 + len(cache), device, work)
            fac = cache[key]
        G = power_law_matrix(H, W, seed0 + i, device, state_dtype, factors=fac)
        M = torch.zeros(H, W, device=device, dtype=state_dtype)
        Wt = weights(H, W, seed0 + i, device)
        out.append((Wt, M, G))
    return out

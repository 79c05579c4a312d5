"""Matrix-function diagnostics of HiMuon on the GPU.

"Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon Optimization"
(Abstract) pairs its training runs with "controlled matrix-function diagnostics" and
frames tiling as a local matrix function rather than an approximation of the
full-matrix map; it does not define the diagnostics.  Measured here, for a momentum
matrix M and the tiled output O_T of the HIP path (O_FULL at T = FULL):

* deviation(T) = ||O_T - O_FULL||_F / ||O_FULL||_F,
* the singular values of O_T (how close to orthogonal the output is),
* alignment(T) = <M, O_T> / ||M||_*  (1 for the exact polar factor of M).

Every tile is normalised on its own, so O_T carries about sqrt(H / T) times the norm of
O_FULL; two scale-free companions come with them: cosine(T) = <O_T, O_FULL> /
(||O_T||_F ||O_FULL||_F), and dual alignment(T) = <M, O_T> / (||M||_* ||O_T||_2), which
is 1 exactly for positive multiples of the polar factor.

O_T comes from the library's kernels (one step with zero prior momentum, G = M, so the
stored momentum is M itself, and the NS output written through
HIMUON_FLAG_WRITE_UPDATE); the reductions and singular values of the report are torch
float64 routines on the device.
"""
from __future__ import annotations

import time

from . import HiMuon, QUINTIC


def ns_output(M, tile: int, steps: int = 5, coeffs=QUINTIC, precision=None, eps: float = 1e-7):
    """O_T of the 2-D CUDA tensor M (float32 or bfloat16) through the HIP path.
    Returns (O as float32, milliseconds of the step on the device)."""
    import torch
    if M.dim() != 2 or not M.is_cuda:
        raise ValueError("M must be a 2-D CUDA tensor")
    G = M.contiguous()
    Mo = torch.zeros_like(G)
    W = torch.zeros(G.shape, dtype=torch.float32, device=G.device)
    U = torch.empty(G.shape, dtype=torch.float32, device=G.device)
    opt = HiMuon([(W, Mo, G, U)], tile, steps, coeffs, beta=0.0, eps=eps, precision=precision)
    stream = torch.cuda.current_stream(G.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    opt.step(0.0, stream)
    e1.record(stream)
    torch.cuda.synchronize(G.device)
    opt.close()
    return U, e0.elapsed_time(e1)


def report(M, tiles, steps: int = 5, coeffs=QUINTIC, precision=None, eps: float = 1e-7,
           spectrum: bool = True) -> dict:
    """Diagnostics of M at each T in `tiles` (0 = FULL); FULL is always computed as the
    reference.  Per T: deviation, alignment, sv_min / sv_max / sv_mean (and the spectrum
    when `spectrum`), and the device time of the NS step in ms."""
    import torch
    t0 = time.time()
    O_full, ms_full = ns_output(M, 0, steps, coeffs, precision, eps)
    Mf = M.double()
    nuc = torch.linalg.svdvals(Mf).sum()
    Of = O_full.double()
    nf = torch.linalg.norm(Of)
    out = {}
    for T in tiles:
        if T == 0:
            O, ms = O_full, ms_full
        else:
            O, ms = ns_output(M, T, steps, coeffs, precision, eps)
        Od = O.double()
        inner = (Mf * Od).sum()
        r = {"deviation": float(torch.linalg.norm(Od - Of) / nf),
             "alignment": float(inner / nuc),
             "cosine": float((Od * Of).sum() / (torch.linalg.norm(Od) * nf)), "ms": ms}
        sv = torch.linalg.svdvals(Od)
        r.update(dual_alignment=float(inner / (nuc * sv.max())), sv_min=float(sv.min()),
                 sv_max=float(sv.max()), sv_mean=float(sv.mean()))
        if spectrum:
            r["spectrum"] = sv.cpu().numpy()
        out[T] = r
    out["seconds"] = time.time() - t0
    return out

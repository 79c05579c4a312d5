"""Pins of the oracle's matrix-function diagnostics (CPU).

The Newton-Schulz map acts on singular values: with M = U diag(s) V^T and
X = M / (||M||_F + eps), K steps give U diag(phi^K(s / (||s|| + eps))) V^T.  That fixes
the FULL-matrix spectrum and alignment in closed form; a block-diagonal matrix whose
blocks sit on the tile grid, iterated to convergence, pins deviation(T) = 0."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import diagnostics as dg

Q, C = oracle.COEFFS_QUINTIC, oracle.COEFFS_CUBIC


def exact_low_rank(H, W, seed):
    U, s, V = synth.power_law_factors(H, W, seed)
    U, s, V = U.numpy(), s.numpy(), V.numpy()
    return (U * s) @ V.T, s


@pytest.mark.parametrize("H,W", [(96, 160), (160, 96), (128, 128)])
@pytest.mark.parametrize("coeffs,K", [(Q, 5), (C, 5), (Q, 8)])
def test_full_spectrum_and_alignment_closed_form(H, W, coeffs, K):
    M, s = exact_low_rank(H, W, 3)
    rep = dg.report(M, [0], K, coeffs)[0]
    mapped = np.abs(oracle.phi_iterate(s / (np.linalg.norm(s) + 1e-7), K, coeffs))
    want_sv = np.sort(mapped)[::-1]
    assert np.allclose(rep["spectrum"], want_sv, rtol=0, atol=1e-10)
    want_align = float(np.sum(s * oracle.phi_iterate(s / (np.linalg.norm(s) + 1e-7), K, coeffs)) / s.sum())
    assert abs(rep["alignment"] - want_align) < 1e-10
    assert rep["deviation"] == 0.0 and abs(rep["cosine"] - 1.0) < 1e-12
    want_dual = want_align / want_sv[0]
    assert abs(rep["dual_alignment"] - want_dual) < 1e-10


def test_polar_factor_scores_one():
    M, s = exact_low_rank(64, 96, 5)
    U, _, Vt = np.linalg.svd(M, full_matrices=False)
    assert abs(dg.alignment(M, U @ Vt) - 1.0) < 1e-12
    assert dg.deviation(U @ Vt, U @ Vt) == 0.0
    # the scale-free forms: any positive multiple of the polar factor scores one
    assert abs(dg.dual_alignment(M, 3.0 * U @ Vt) - 1.0) < 1e-12
    assert abs(dg.cosine(3.0 * U @ Vt, U @ Vt) - 1.0) < 1e-12
    # and M itself scores ||M||_F^2 / (||M||_* ||M||_2) = sum s^2 / (sum s * max s) < 1
    assert abs(dg.dual_alignment(M, M) - np.sum(s ** 2) / (s.sum() * s.max())) < 1e-12


def test_tile_aligned_block_diagonal_converges_to_zero_deviation():
    # two well-conditioned 64x64 blocks exactly on the T = 64 grid: both the tiled and the
    # full cubic iteration converge to the polar factor, which is block diagonal
    rng = np.random.default_rng(0)
    blocks = []
    for k in range(2):
        Uq, _ = np.linalg.qr(rng.standard_normal((64, 64)))
        Vq, _ = np.linalg.qr(rng.standard_normal((64, 64)))
        blocks.append((Uq * np.linspace(0.5, 1.0, 64)) @ Vq.T)
    M = np.zeros((128, 128))
    M[:64, :64], M[64:, 64:] = blocks
    rep = dg.report(M, [64, 0], 40, C)
    assert rep[64]["deviation"] < 1e-12
    assert np.allclose(rep[64]["spectrum"], 1.0, atol=1e-12)
    assert abs(rep[64]["alignment"] - 1.0) < 1e-12
    assert abs(rep[64]["cosine"] - 1.0) < 1e-12 and abs(rep[64]["dual_alignment"] - 1.0) < 1e-12


def test_local_map_differs_from_full_map_on_coupled_matrix():
    # a dense power-law matrix couples rows and columns across tiles: the tiled map is a
    # different function, so the deviation is clearly non-zero and shrinks as T grows
    M, _ = exact_low_rank(256, 256, 9)
    rep = dg.report(M, [32, 64, 128, 0], 5, Q)
    d = [rep[T]["deviation"] for T in (32, 64, 128)]
    assert all(x > 1e-3 for x in d)
    assert d[0] > d[1] > d[2] > rep[0]["deviation"] == 0.0


def test_alignment_scale_invariant():
    M, _ = exact_low_rank(64, 128, 11)
    O = oracle.tiled_ns(M, 32, 5, Q)
    O2 = oracle.tiled_ns(4.0 * M, 32, 5, Q)
    assert abs(dg.alignment(M, O) - dg.alignment(4.0 * M, O2)) < 1e-6


def test_synth_factors_are_exact_svd():
    # the closed-form pins rely on power_law_factors giving orthonormal U, V
    U, s, V = synth.power_law_factors(96, 160, 3)
    assert torch.allclose(U.T @ U, torch.eye(96, dtype=U.dtype), atol=1e-12)
    assert torch.allclose(V.T @ V, torch.eye(96, dtype=V.dtype), atol=1e-12)

"""Matrix-function diagnostics of HiMuon in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the product package never
imports it.

"Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon Optimization"
(Abstract) reports "controlled matrix-function diagnostics" next to its training runs
but does not define them.  The abstract's own framing fixes what is worth measuring:
for T below the matrix dimensions HiMuon is a different (local) matrix function, not an
approximation that converges to the full-matrix map, and a Muon-type map is meant to
push the singular values of the momentum towards one.  The reading taken here, for a
momentum matrix M and its tiled output O_T (O_FULL at T = FULL):

* deviation(T) = ||O_T - O_FULL||_F / ||O_FULL||_F: how far the local map is from the
  full-matrix map;
* spectrum(T) = the singular values of O_T: how close to orthogonal the output is;
* alignment(T) = <M, O_T> / ||M||_*: the share of the steepest-descent value of the
  exact polar factor that O_T keeps (the polar factor U V^T of M = U S V^T gives
  <M, U V^T> = tr S = ||M||_*, so an exact polar factor scores 1).

Each tile is normalised on its own, so O_T carries about sqrt(H / T) times the norm of
O_FULL and the two quantities above mostly measure that scale.  Two scale-free companions
are reported with them:

* cosine(T) = <O_T, O_FULL> / (||O_T||_F ||O_FULL||_F);
* dual alignment(T) = <M, O_T> / (||M||_* ||O_T||_2), in [-1, 1] because the nuclear and
  spectral norms are dual; it is 1 exactly for positive multiples of the polar factor
  (steepest descent under the spectral norm).

Every quantity is a plain definition evaluated with numpy (SVD from LAPACK).
"""
from __future__ import annotations

import numpy as np

from . import himuon_oracle as ho


def deviation(O_T: np.ndarray, O_full: np.ndarray) -> float:
    """||O_T - O_FULL||_F / ||O_FULL||_F."""
    O_T = np.asarray(O_T, dtype=np.float64)
    O_full = np.asarray(O_full, dtype=np.float64)
    return float(np.linalg.norm(O_T - O_full) / np.linalg.norm(O_full))


def spectrum(O: np.ndarray) -> np.ndarray:
    """Singular values of O, descending."""
    return np.linalg.svd(np.asarray(O, dtype=np.float64), compute_uv=False)


def nuclear_norm(M: np.ndarray) -> float:
    return float(spectrum(M).sum())


def alignment(M: np.ndarray, O: np.ndarray) -> float:
    """<M, O> / ||M||_*  (Frobenius inner product over the nuclear norm of M)."""
    M = np.asarray(M, dtype=np.float64)
    return float(np.sum(M * np.asarray(O, dtype=np.float64)) / nuclear_norm(M))


def cosine(O_T: np.ndarray, O_full: np.ndarray) -> float:
    """<O_T, O_FULL> / (||O_T||_F ||O_FULL||_F)."""
    O_T = np.asarray(O_T, dtype=np.float64)
    O_full = np.asarray(O_full, dtype=np.float64)
    return float(np.sum(O_T * O_full) / (np.linalg.norm(O_T) * np.linalg.norm(O_full)))


def dual_alignment(M: np.ndarray, O: np.ndarray) -> float:
    """<M, O> / (||M||_* ||O||_2)."""
    M = np.asarray(M, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    return float(np.sum(M * O) / (nuclear_norm(M) * spectrum(O)[0]))


def report(M: np.ndarray, Ts, K: int, coeffs, eps: float = 1e-7) -> dict:
    """The diagnostics of M at each T in Ts (T = 0 is FULL)."""
    M = np.asarray(M, dtype=np.float64)
    O_full = ho.tiled_ns(M, None, K, coeffs, eps)
    out = {}
    for T in Ts:
        O = O_full if T == 0 else ho.tiled_ns(M, T, K, coeffs, eps)
        sv = spectrum(O)
        out[T] = {"deviation": deviation(O, O_full), "alignment": alignment(M, O),
                  "cosine": cosine(O, O_full), "dual_alignment": dual_alignment(M, O),
                  "sv_min": float(sv.min()), "sv_max": float(sv.max()),
                  "sv_mean": float(sv.mean()), "spectrum": sv}
    return out

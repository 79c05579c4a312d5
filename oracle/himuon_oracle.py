"""Plain fp64 CPU oracle of one HiMuon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg may use it.
It shares no code with the HIP path: numpy only, float64 throughout.

What it computes follows "Hierarchical Muon: Tiled Newton-Schulz Updates for
Efficient Muon Optimization" (Abstract):

* a Muon-type step builds the update direction of a dense weight by a finite
  Newton-Schulz (NS) map applied to the momentum-gradient matrix;
* HiMuon cuts an H x W momentum-gradient matrix into T x T tiles, runs the same
  finite NS map on every tile independently and puts the tile results back in
  place; spectra inside a tile interact, spectra of different tiles do not;
* the leading NS work for fixed T is O(H W T K) instead of O(r^2 s K), with
  r = min(H, W) and s = max(H, W).

The page leaves the following open; the oracle takes the plainest reading:

* momentum: M <- beta * M + G (no Nesterov term); the NS input is the updated M;
* NS step on a short-side tile X (r x s, r <= s): A = X X^T,
  X <- a X + (b A + c A^2) X, with (a, b, c) a parameter; the cubic set
  (1.5, -0.5, 0) is the classical iteration towards the orthogonal polar factor
  (Bjorck & Bowie 1971; Higham 1986, cited by "SignMuon: Communication-Efficient
  Distributed Muon Optimization", References), the quintic set
  (3.4445, -4.7750, 2.0315) is the one used by the Muon blog post cited there;
* each tile is scaled by 1 / (||Y||_F + eps) before the first NS step (a zero tile
  stays zero, also at eps = 0; a tile holding a NaN becomes all NaN);
* a tile with more rows than columns is transposed, iterated, and transposed back;
  a square tile is not transposed;
* tiles are anchored at (0, 0) in row-major order; the last tile row and column
  keep their ragged h x w size; T = 0 (FULL) or T >= max(H, W) is one tile;
* the parameter update is W <- W - lr * O, O the reassembled NS output.
"""
from __future__ import annotations

import numpy as np

COEFFS_CUBIC = (1.5, -0.5, 0.0)
COEFFS_QUINTIC = (3.4445, -4.7750, 2.0315)

TILE_FULL = 0


# ---------------------------------------------------------------- tile partition
def tiles(H: int, W: int, T: int | None):
    """Row-major list of (row0, col0, h, w) covering an H x W matrix with T x T tiles.

    Tiles start at (0, 0); the last row/column of tiles keeps its ragged size.
    T = 0 / None means one tile for the whole matrix (full-matrix Muon).
    (Abstract: partition into T x T tiles.)
    """
    if H < 0 or W < 0:
        raise ValueError("negative shape")
    if H == 0 or W == 0:
        return []
    if not T:
        return [(0, 0, H, W)]
    if T < 0:
        raise ValueError("negative tile size")
    out = []
    for r0 in range(0, H, T):
        for c0 in range(0, W, T):
            out.append((r0, c0, min(T, H - r0), min(T, W - c0)))
    return out


# ---------------------------------------------------------------- the NS map
def frobenius_normalise(Y: np.ndarray, eps: float) -> np.ndarray:
    """X0 = Y / (||Y||_F + eps).  A zero tile maps to zero, also when eps = 0 (the
    divisor is then 0 and the tile is left as it is).  A tile holding a NaN has a NaN
    norm, and the division passes it on to every entry, as IEEE arithmetic does."""
    Y = np.asarray(Y, dtype=np.float64)
    den = np.sqrt(np.sum(Y * Y)) + eps
    return np.zeros_like(Y) if den == 0 else Y / den


def ns_iterate(X: np.ndarray, K: int, coeffs) -> np.ndarray:
    """K Newton-Schulz steps on a short-side matrix X (r x s, r <= s), or on a
    stack of them (n x r x s).  Each step: A = X X^T, B = b A + c A^2,
    X <- a X + B X.  When c == 0 the A^2 term is exactly zero and is not formed.
    """
    a, b, c = (float(v) for v in coeffs)
    X = np.asarray(X, dtype=np.float64)
    for _ in range(int(K)):
        A = X @ np.swapaxes(X, -1, -2)
        B = b * A
        if c != 0.0:
            B = B + c * (A @ A)
        X = a * X + B @ X
    return X


def ns_tile(Y: np.ndarray, K: int, coeffs, eps: float = 1e-7) -> np.ndarray:
    """The finite NS map of one tile: normalise, orient on the short side, K steps,
    orient back.  Same map for every tile (Abstract)."""
    Y = np.asarray(Y, dtype=np.float64)
    tall = Y.shape[0] > Y.shape[1]
    X = frobenius_normalise(np.ascontiguousarray(Y.T if tall else Y), eps)
    X = ns_iterate(X, K, coeffs)
    return X.T if tall else X


def tiled_ns(M: np.ndarray, T: int | None, K: int, coeffs, eps: float = 1e-7) -> np.ndarray:
    """HiMuon map O = reassemble(NS(tile) for tile in tiles(M, T)).

    Tiles of equal shape are stacked and iterated together with batched matmul;
    that groups independent computations and changes no tile's arithmetic.
    """
    M = np.asarray(M, dtype=np.float64)
    H, W = M.shape
    O = np.zeros((H, W), dtype=np.float64)
    groups: dict[tuple[int, int], list[tuple[int, int]]] = {}
    for r0, c0, h, w in tiles(H, W, T):
        groups.setdefault((h, w), []).append((r0, c0))
    for (h, w), origins in groups.items():
        tall = h > w
        # each tile is oriented on its short side (a contiguous copy) before it is
        # normalised, so a tile and its transpose see the same arithmetic
        Y = np.stack([np.ascontiguousarray(M[r0:r0 + h, c0:c0 + w].T if tall else M[r0:r0 + h, c0:c0 + w])
                      for r0, c0 in origins])
        X = np.stack([frobenius_normalise(y, eps) for y in Y])
        X = ns_iterate(X, K, coeffs)
        if tall:
            X = np.swapaxes(X, 1, 2)
        for (r0, c0), blk in zip(origins, X):
            O[r0:r0 + h, c0:c0 + w] = blk
    return O


def tiled_ns_loop(M: np.ndarray, T: int | None, K: int, coeffs, eps: float = 1e-7) -> np.ndarray:
    """Same map as tiled_ns, one tile at a time (reference for the batched form)."""
    M = np.asarray(M, dtype=np.float64)
    O = np.zeros_like(M)
    for r0, c0, h, w in tiles(*M.shape, T):
        O[r0:r0 + h, c0:c0 + w] = ns_tile(M[r0:r0 + h, c0:c0 + w], K, coeffs, eps)
    return O


def phi(x, coeffs):
    """The scalar map a x + b x^3 + c x^5 that one NS step applies to every
    singular value (a polynomial matrix function acts on the spectrum)."""
    a, b, c = coeffs
    return a * x + b * x ** 3 + c * x ** 5


def phi_iterate(x, K: int, coeffs):
    for _ in range(int(K)):
        x = phi(x, coeffs)
    return x


# ---------------------------------------------------------------- momentum / update
def momentum(M: np.ndarray, G: np.ndarray, beta: float) -> np.ndarray:
    """M <- beta M + G, exact in float64."""
    return float(beta) * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32).copy()
    out[nan] = np.float32("nan")
    return out


def momentum_stored(M: np.ndarray, G: np.ndarray, beta: float, storage: str) -> np.ndarray:
    """The stored momentum code: beta*M + G formed once and rounded to float32
    (a fused multiply-add), then, for bfloat16 storage, rounded to bfloat16.
    beta itself is a float32 parameter.  Returns float32 values."""
    b32 = float(np.float32(beta))
    exact = b32 * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    r = exact.astype(np.float32)
    if storage == "bf16":
        r = bf16_round(r)
    elif storage != "f32":
        raise ValueError(storage)
    return r


def apply_update(W: np.ndarray, O: np.ndarray, lr: float) -> np.ndarray:
    """W <- W - lr * O."""
    return np.asarray(W, dtype=np.float64) - float(lr) * np.asarray(O, dtype=np.float64)


def step(layers, T, K, coeffs, beta=0.95, lr=0.02, eps=1e-7):
    """One HiMuon step over a list of (W, M, G) float arrays.

    Returns a list of (W_new, M_new, O) in float64.
    """
    out = []
    for W, M, G in layers:
        M_new = momentum(M, G, beta)
        O = tiled_ns(M_new, T, K, coeffs, eps)
        out.append((apply_update(W, O, lr), M_new, O))
    return out


# ---------------------------------------------------------------- algorithmic work
def tile_flops(h: int, w: int, K: int, coeffs) -> int:
    """Matrix-product flops of K NS steps on one h x w tile (short side r, long
    side s): X X^T costs 2 r^2 s, A^2 costs 2 r^3 (absent when c == 0), B X costs
    2 r^2 s.  Elementwise terms are not counted."""
    r, s = min(h, w), max(h, w)
    per = 4 * r * r * s + (2 * r ** 3 if coeffs[2] != 0 else 0)
    return int(K) * per


def ns_flops(shapes, T, K, coeffs) -> int:
    """Total NS flops of one step over matrices of the given (H, W) shapes."""
    return sum(tile_flops(h, w, K, coeffs) for H, W in shapes for _, _, h, w in tiles(H, W, T))


def step_bytes(shapes, state_bytes: int, weight_bytes: int = 4) -> int:
    """Algorithmic HBM bytes of one step: read G and M, write M (state_bytes each),
    read and write W (weight_bytes each), per element."""
    return sum(H * W for H, W in shapes) * (3 * state_bytes + 2 * weight_bytes)

"""Local pieces of Sign-Muon in plain numpy.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

"Sign-Muon: Communication-Efficient Distributed Muon Optimization" (Figures 1 and 6,
and its remark on practical orthogonalization with 1-bit communication): each worker
takes its Newton-Schulz polar direction U, forms the entrywise sign S in {-1, +1}, packs
S into one bit per entry (ceil(d / 8) bytes) for an all-gather, and every worker then
unpacks the gathered buffers and takes the majority vote S_bar = sign(sum_m S^(m)); a
worker may also run the polar map on S_bar locally.  With HiMuon the direction is the
tiled map O_T = HiMuon_T(M).

Readings where the pages leave a choice:
* sign(0) = +1, so S has no zero entries (the pages require S in {-1, +1});
* the vote of a tie (an even number of workers split evenly) is +1 for the same reason;
* bit k of the packed buffer holds entry k of the matrix in row-major order (k = i W + j),
  byte k // 8, bit k % 8 counted from the least significant bit; 1 means +1.
"""
from __future__ import annotations

import numpy as np


def sign(O: np.ndarray) -> np.ndarray:
    """Entrywise sign in {-1, +1} (int8), sign(0) = +1."""
    return np.where(np.asarray(O) >= 0, 1, -1).astype(np.int8)


def pack(S: np.ndarray) -> np.ndarray:
    """Row-major {-1, +1} matrix -> ceil(d / 8) bytes, entry k at byte k // 8, bit k % 8."""
    flat = (np.asarray(S).reshape(-1) > 0).astype(np.uint8)
    n = flat.size
    out = np.zeros((n + 7) // 8, dtype=np.uint8)
    for b in range(8):
        part = flat[b::8]
        out[:part.size] |= (part << b).astype(np.uint8)
    return out


def unpack(bits: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack for d = n entries: int8 {-1, +1} vector."""
    bits = np.asarray(bits, dtype=np.uint8)
    k = np.arange(n)
    on = (bits[k // 8] >> (k % 8)) & 1
    return np.where(on == 1, 1, -1).astype(np.int8)


def vote(gathered, n: int) -> np.ndarray:
    """Majority vote over the packed buffers of all workers: sign(sum_m S^(m)), ties +1."""
    total = np.zeros(n, dtype=np.int64)
    for bits in gathered:
        total += unpack(bits, n)
    return np.where(total >= 0, 1, -1).astype(np.int8)

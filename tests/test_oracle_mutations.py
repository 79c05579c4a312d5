"""The pins must catch plausible mistakes: each mutant below plants one in a copy of
the oracle's NS step (on the CPU) and must fail the closed-form or tiling checks."""
import numpy as np
import pytest

import oracle
from oracle import COEFFS_QUINTIC as Q

EPS = 1e-7


def closed_form(Y, K, coeffs):
    U, s, Vt = np.linalg.svd(Y / (np.linalg.norm(Y) + EPS), full_matrices=False)
    a, b, c = coeffs
    for _ in range(K):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


def iterate_mutant(kind):
    def it(X, K, coeffs):
        a, b, c = coeffs
        for _ in range(K):
            A = X @ np.swapaxes(X, -1, -2)
            if kind == "drop_c":
                B = b * A
            elif kind == "sign_b":
                B = -b * A + c * (A @ A)
            elif kind == "a_on_B":
                B = b * A + c * (A @ A)
                X = X + a * (B @ X)
                continue
            else:
                B = b * A + c * (A @ A)
            if kind == "right_multiply":      # B on the wrong side of X (square tile)
                X = a * X + X @ B
            else:
                X = a * X + B @ X
        return X
    return it


@pytest.mark.parametrize("kind", ["drop_c", "sign_b", "a_on_B", "right_multiply"])
def test_closed_form_pin_catches_mutant(kind, monkeypatch):
    monkeypatch.setattr(oracle.himuon_oracle, "ns_iterate", iterate_mutant(kind))
    Y = np.random.default_rng(0).standard_normal((64, 64))
    assert np.abs(oracle.himuon_oracle.ns_tile(Y, 5, Q) - closed_form(Y, 5, Q)).max() > 1e-3


def test_tiling_pin_catches_off_by_one(monkeypatch):
    real = oracle.himuon_oracle.tiles

    def shifted(H, W, T):
        return [(r0, c0, h, w) for r0, c0, h, w in real(H, W, T)][:-1]  # drops the last tile

    monkeypatch.setattr(oracle.himuon_oracle, "tiles", shifted)
    M = np.random.default_rng(1).standard_normal((100, 70))
    want = np.zeros_like(M)
    for r0, c0, h, w in real(100, 70, 32):
        want[r0:r0 + h, c0:c0 + w] = closed_form(M[r0:r0 + h, c0:c0 + w], 5, Q)
    assert np.abs(oracle.himuon_oracle.tiled_ns(M, 32, 5, Q) - want).max() > 1e-3

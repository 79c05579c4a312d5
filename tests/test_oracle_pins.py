"""Pins of the fp64 oracle against what the mathematics fixes (no GPU).

Every pin compares the oracle's matrix iteration with something computed another
way: the singular-value closed form (LAPACK SVD + the scalar polynomial), the
polar factor, exact symmetry properties, hand-derivable scalars, brute-force
counts.  A dropped term, a wrong sign, a transposed operand or a wrong tile index
in the oracle breaks at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import COEFFS_CUBIC as C, COEFFS_QUINTIC as Q

EPS = 1e-7
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng_matrix(h, w, seed, spectrum=None):
    rng = np.random.default_rng(seed)
    if spectrum is None:
        return rng.standard_normal((h, w))
    r = min(h, w)
    U, _ = np.linalg.qr(rng.standard_normal((h, r)))
    V, _ = np.linalg.qr(rng.standard_normal((w, r)))
    return (U * spectrum(r)) @ V.T


def closed_form(Y, K, coeffs, eps=EPS):
    """U phi^K(Sigma) V^T of the normalised tile, by SVD (independent of the iteration)."""
    Y = np.asarray(Y, dtype=np.float64)
    U, s, Vt = np.linalg.svd(Y / (np.linalg.norm(Y) + eps), full_matrices=False)
    a, b, c = coeffs
    for _ in range(K):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


# ------------------------------------------------------------------ tiles
@pytest.mark.parametrize("H,W,T", [(256, 512, 64), (250, 500, 64), (37, 53, 16), (5, 3, 2),
                                   (100, 100, 100), (100, 100, 1000), (7, 300, 128), (1, 1, 1)])
def test_tiles_cover_exactly_once(H, W, T):
    cover = np.zeros((H, W), dtype=int)
    prev = (-1, -1)
    for r0, c0, h, w in oracle.tiles(H, W, T):
        assert r0 % T == 0 and c0 % T == 0
        assert h == min(T, H - r0) and w == min(T, W - c0)
        assert (r0, c0) > prev  # row-major order
        prev = (r0, c0)
        cover[r0:r0 + h, c0:c0 + w] += 1
    assert (cover == 1).all()
    assert len(oracle.tiles(H, W, T)) == math.ceil(H / T) * math.ceil(W / T)


def test_tile_counts_of_the_layer_stacks():
    # counts follow from ceil(H/T) * ceil(W/T) per matrix
    assert len(oracle.tiles(256, 512, 64)) == 32
    assert len(oracle.tiles(256, 512, 128)) == 8
    assert len(oracle.tiles(256, 512, 512)) == 1
    assert oracle.tiles(256, 512, 0) == [(0, 0, 256, 512)]
    assert oracle.tiles(256, 512, None) == [(0, 0, 256, 512)]
    gpt2 = [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12
    assert sum(len(oracle.tiles(h, w, 128)) for h, w in gpt2) == 5184
    l8b = ([(4096, 4096)] * 2 + [(4096, 1024)] * 2 + [(4096, 14336)] * 2 + [(14336, 4096)]) * 32
    assert sum(len(oracle.tiles(h, w, 128)) for h, w in l8b) == 425984
    d1b = ([(2048, 2048)] * 4 + [(2048, 8192)] * 2 + [(8192, 2048)]) * 16
    assert [sum(len(oracle.tiles(h, w, T)) for h, w in d1b) for T in (32, 64, 128, 256)] == \
        [1048576, 262144, 65536, 16384]
    assert oracle.tiles(0, 5, 4) == [] and oracle.tiles(5, 0, 4) == []


def test_between_short_and_long_side_still_tiles_both_dimensions():
    assert oracle.tiles(256, 512, 256) == [(0, 0, 256, 256), (0, 256, 256, 256)]
    assert oracle.tiles(256, 512, 300) == [(0, 0, 256, 300), (0, 300, 256, 212)]


# ------------------------------------------------------------------ P1 closed form
@pytest.mark.parametrize("coeffs", [Q, C, (2.0, -1.5, 0.5)])
@pytest.mark.parametrize("shape", [(64, 64), (64, 200), (200, 64), (3, 5), (5, 3), (1, 7), (7, 1), (2, 2)])
@pytest.mark.parametrize("K", [1, 5, 8])
def test_ns_tile_matches_singular_value_closed_form(coeffs, shape, K):
    Y = rng_matrix(*shape, seed=hash((shape, K)) % 1000)
    np.testing.assert_allclose(oracle.ns_tile(Y, K, coeffs), closed_form(Y, K, coeffs), atol=2e-13, rtol=0)


def test_one_step_by_hand():
    # Y = [[3, 4]]: ||Y|| = 5, X0 = [0.6, 0.8] * 5/(5+eps), A = XX^T is the scalar x^2,
    # one step multiplies X by a + b x^2 + c x^4.
    x = 5.0 / (5.0 + EPS)
    for co in (Q, C):
        a, b, c = co
        want = np.array([[0.6, 0.8]]) * x * (a + b * x * x + c * x ** 4)
        np.testing.assert_allclose(oracle.ns_tile(np.array([[3.0, 4.0]]), 1, co), want, rtol=0, atol=1e-15)
        np.testing.assert_allclose(oracle.ns_tile(np.array([[3.0], [4.0]]), 1, co), want.T, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ P2 full matrix
@pytest.mark.parametrize("T", [512, 1000, 0, None])
def test_tile_at_least_matrix_is_full_matrix_ns(T):
    M = rng_matrix(256, 512, 0, spectrum=lambda r: 1.0 / np.arange(1, r + 1))
    np.testing.assert_allclose(oracle.tiled_ns(M, T, 5, Q), closed_form(M, 5, Q), atol=1e-12, rtol=0)


def test_full_matrix_differs_from_tiled():
    # local map, not an approximation of the full update (tiles do not interact)
    M = rng_matrix(256, 512, 0)
    assert np.linalg.norm(oracle.tiled_ns(M, 64, 5, Q) - oracle.tiled_ns(M, 0, 5, Q)) > 0.1


# ------------------------------------------------------------------ tiled = per-tile closed form
@pytest.mark.parametrize("H,W,T", [(250, 500, 64), (97, 131, 32), (130, 70, 64), (64, 64, 16)])
def test_tiled_map_is_per_tile_closed_form(H, W, T):
    M = rng_matrix(H, W, 3)
    want = np.zeros((H, W))
    for r0, c0, h, w in oracle.tiles(H, W, T):
        want[r0:r0 + h, c0:c0 + w] = closed_form(M[r0:r0 + h, c0:c0 + w], 5, Q)
    np.testing.assert_allclose(oracle.tiled_ns(M, T, 5, Q), want, atol=2e-13, rtol=0)
    np.testing.assert_allclose(oracle.tiled_ns_loop(M, T, 5, Q), want, atol=2e-13, rtol=0)


def test_batched_and_loop_forms_agree():
    M = rng_matrix(200, 330, 9)
    np.testing.assert_allclose(oracle.tiled_ns(M, 64, 8, Q), oracle.tiled_ns_loop(M, 64, 8, Q), atol=1e-14, rtol=0)


# ------------------------------------------------------------------ P3 locality
def test_editing_one_tile_leaves_other_tiles_bit_identical():
    M = rng_matrix(250, 330, 4)
    O = oracle.tiled_ns(M, 64, 5, Q)
    M2 = M.copy()
    M2[64:128, 128:192] = rng_matrix(64, 64, 99)
    O2 = oracle.tiled_ns(M2, 64, 5, Q)
    mask = np.ones_like(M, dtype=bool)
    mask[64:128, 128:192] = False
    assert np.array_equal(O[mask], O2[mask])
    assert not np.allclose(O[~mask], O2[~mask])


def test_permuting_tiles_permutes_outputs():
    M = rng_matrix(128, 256, 5)
    P = M.copy()
    P[:64, :64], P[64:, 192:] = M[64:, 192:], M[:64, :64]
    O, OP = oracle.tiled_ns(M, 64, 5, Q), oracle.tiled_ns(P, 64, 5, Q)
    assert np.array_equal(OP[:64, :64], O[64:, 192:]) and np.array_equal(OP[64:, 192:], O[:64, :64])


# ------------------------------------------------------------------ P4 transpose
@pytest.mark.parametrize("H,W,T", [(250, 500, 64), (100, 37, 32), (130, 70, 64)])
def test_transpose_equivariance(H, W, T):
    M = rng_matrix(H, W, 6)
    O = oracle.tiled_ns(M, T, 5, Q)
    Ot = oracle.tiled_ns(M.T.copy(), T, 5, Q)
    np.testing.assert_allclose(Ot, O.T, atol=1e-13, rtol=0)
    # non-square tiles are iterated on the same short-side matrix: bit-identical
    for r0, c0, h, w in oracle.tiles(H, W, T):
        if h != w:
            assert np.array_equal(Ot[c0:c0 + w, r0:r0 + h], O[r0:r0 + h, c0:c0 + w].T)


# ------------------------------------------------------------------ P5 polar factor
@pytest.mark.parametrize("shape", [(16, 24), (24, 16), (32, 32)])
def test_cubic_converges_to_polar_factor(shape):
    r = min(shape)
    Y = rng_matrix(*shape, 7, spectrum=lambda r: np.linspace(1.0, 0.2, r))
    U, _, Vt = np.linalg.svd(Y, full_matrices=False)
    errs = [np.abs(oracle.ns_tile(Y, K, C) - U @ Vt).max() for K in (5, 10, 30)]
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-12, errs
    del r


# ------------------------------------------------------------------ P6 special values
def load_golden():
    with open(os.path.join(GOLDEN, "special_values.json")) as f:
        return json.load(f)


def test_golden_scalars_are_the_closed_form():
    # hand-checkable: cubic phi(1) = 1.5 - 0.5 = 1 exactly; quintic phi(1) = 0.701
    assert oracle.phi(1.0, C) == 1.0
    assert abs(oracle.phi(1.0, Q) - 0.701) < 1e-12
    for case in load_golden()["cases"]:
        co = Q if case["coeffs"] == "quintic" else C
        x = case["x0"]
        for _ in range(case["K"]):
            x = co[0] * x + co[1] * x ** 3 + co[2] * x ** 5
        assert abs(x - case["value"]) < 1e-15


@pytest.mark.parametrize("coeffs,K", [(Q, 5), (Q, 8), (C, 5)])
def test_rank_one_tile(coeffs, K):
    rng = np.random.default_rng(8)
    u, v = rng.standard_normal(40), rng.standard_normal(70)
    u /= np.linalg.norm(u)
    v /= np.linalg.norm(v)
    sig = 3.0
    x0 = sig / (sig + EPS)
    want = oracle.phi_iterate(x0, K, coeffs) * np.outer(u, v)
    # rounding noise in the null space grows by the factor a per step (phi'(0) = a)
    tol = 1e-15 * coeffs[0] ** K * 10
    np.testing.assert_allclose(oracle.ns_tile(sig * np.outer(u, v), K, coeffs), want, atol=tol, rtol=0)
    np.testing.assert_allclose(oracle.ns_tile(sig * np.outer(v, u), K, coeffs), want.T, atol=tol, rtol=0)
    g = {(c["coeffs"], c["K"]): c["value"] for c in load_golden()["cases"] if c["x0"] == 1.0}
    name = "quintic" if coeffs == Q else "cubic"
    assert abs(np.linalg.norm(oracle.ns_tile(np.outer(u, v), K, coeffs)) - g[(name, K)]) < 1e-6


@pytest.mark.parametrize("T", [32, 64, 128])
@pytest.mark.parametrize("coeffs", [Q, C])
def test_orthogonal_tile(T, coeffs):
    Qm, _ = np.linalg.qr(np.random.default_rng(T).standard_normal((T, T)))
    val = {(c["coeffs"], round(c["x0"] ** -2)): c["value"] for c in load_golden()["cases"]
           if c["K"] == 5 and c["x0"] < 1.0}[("quintic" if coeffs == Q else "cubic", T)]
    # ||Qm||_F = sqrt(T): every singular value of the normalised tile is 1/(sqrt(T) + eps)
    assert abs(oracle.phi_iterate(1.0 / (math.sqrt(T) + EPS), 5, coeffs) - val) < 1e-6
    want = oracle.phi_iterate(1.0 / (math.sqrt(T) + EPS), 5, coeffs) * Qm
    np.testing.assert_allclose(oracle.ns_tile(Qm, 5, coeffs), want, atol=1e-13, rtol=0)


def test_tile_size_one_is_sign_momentum():
    M = rng_matrix(9, 13, 10)
    M[2, 3] = 0.0
    O = oracle.tiled_ns(M, 1, 5, C)
    np.testing.assert_allclose(O, np.sign(M), atol=1e-6, rtol=0)  # eps shifts |x| by ~1e-7
    Oq = oracle.tiled_ns(M, 1, 5, Q)
    np.testing.assert_allclose(Oq, oracle.phi_iterate(1.0, 5, Q) * np.sign(M), atol=1e-4, rtol=0)
    np.testing.assert_allclose(Oq, oracle.phi_iterate(M / (np.abs(M) + EPS), 5, Q), atol=1e-13, rtol=0)
    assert O[2, 3] == 0.0


def test_zero_tile_maps_to_zero():
    M = rng_matrix(128, 128, 11)
    M[:64, 64:] = 0.0
    O = oracle.tiled_ns(M, 64, 5, Q)
    assert (O[:64, 64:] == 0.0).all() and np.abs(O[64:, :64]).max() > 0
    # with eps = 0 the divisor of a zero tile is 0; the tile still maps to zero (no NaN),
    # while every other tile is the plain Y / ||Y||_F map
    O0 = oracle.tiled_ns(M, 64, 5, Q, eps=0.0)
    assert (O0[:64, 64:] == 0.0).all() and np.isfinite(O0).all()
    Y = M[64:, :64]
    np.testing.assert_allclose(O0[64:, :64], closed_form(Y, 5, Q, eps=0.0), atol=1e-13, rtol=0)
    # T = 1 at eps = 0 is the sign map phi^K(sign(m)) with sign(0) = 0
    np.testing.assert_array_equal(oracle.tiled_ns(np.array([[0.0, -2.0, 3.0]]), 1, 1, C, eps=0.0),
                                  np.array([[0.0, -1.0, 1.0]]))


def test_nan_stays_in_its_tile():
    # a NaN entry makes its tile's norm NaN, and IEEE division passes it to every entry
    # of that tile; tile locality keeps every other tile as it was (also at eps = 0)
    M = rng_matrix(128, 192, 14)
    ref = oracle.tiled_ns(M, 64, 5, Q)
    M[70, 130] = np.nan
    for eps in (1e-7, 0.0):
        O = oracle.tiled_ns(M, 64, 5, Q, eps=eps)
        assert np.isnan(O[64:, 128:]).all()
        mask = np.ones_like(O, dtype=bool)
        mask[64:, 128:] = False
        assert np.isfinite(O[mask]).all()
        if eps:
            assert np.array_equal(O[mask], ref[mask])


# ------------------------------------------------------------------ P7 invariances
def test_scale_sign_and_orthogonal_invariance():
    Y = rng_matrix(48, 80, 12)
    O = oracle.ns_tile(Y, 5, Q)
    np.testing.assert_allclose(oracle.ns_tile(1e3 * Y, 5, Q), O, atol=1e-9, rtol=0)
    assert np.array_equal(oracle.ns_tile(-Y, 5, Q), -O)
    Qa, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((48, 48)))
    Qb, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((80, 80)))
    np.testing.assert_allclose(oracle.ns_tile(Qa @ Y @ Qb, 5, Q), Qa @ O @ Qb, atol=1e-12, rtol=0)


# ------------------------------------------------------------------ P8 zero padding
def test_zero_padding_a_ragged_tile_is_exact():
    E = rng_matrix(37, 53, 13)
    P = np.zeros((64, 64))
    P[:37, :53] = E
    OP = oracle.ns_tile(P, 5, Q)
    np.testing.assert_allclose(OP[:37, :53], oracle.ns_tile(E, 5, Q), atol=1e-14, rtol=0)
    assert (OP[37:, :] == 0).all() and (OP[:, 53:] == 0).all()


# ------------------------------------------------------------------ P9 work
def test_flops_match_brute_force_count_and_hwtk():
    def brute(H, W, T, K, co):
        total = 0
        for _, _, h, w in oracle.tiles(H, W, T):
            r, s = min(h, w), max(h, w)
            gram = r * r * s * 2          # r x r outputs, s multiply-adds each
            square = r * r * r * 2 if co[2] else 0
            upd = r * s * r * 2           # r x s outputs, r multiply-adds each
            total += K * (gram + square + upd)
        return total
    for H, W, T in [(256, 512, 64), (250, 500, 64), (97, 131, 32), (4096, 14336, 128)]:
        for co in (Q, C):
            assert oracle.ns_flops([(H, W)], T, 5, co) == brute(H, W, T, 5, co)
    # 6 H W T K when T divides H and W (quintic), 4 H W T K for cubic
    assert oracle.ns_flops([(4096, 14336)], 128, 5, Q) == 6 * 4096 * 14336 * 128 * 5
    assert oracle.ns_flops([(2048, 8192)], 32, 5, C) == 4 * 2048 * 8192 * 32 * 5
    # full matrix: K (4 r^2 s + 2 r^3)
    assert oracle.ns_flops([(256, 512)], 0, 5, Q) == 5 * (4 * 256 ** 2 * 512 + 2 * 256 ** 3)
    assert oracle.step_bytes([(10, 20)], 2) == 200 * 14
    assert oracle.step_bytes([(10, 20)], 4) == 200 * 20


# ------------------------------------------------------------------ P10 tiny brute force
@pytest.mark.parametrize("shape", [(1, 1), (2, 2), (3, 5), (5, 3)])
def test_tiny_tiles_brute_force(shape):
    Y = rng_matrix(*shape, 14)
    for co in (Q, C):
        for K in (1, 2, 5):
            np.testing.assert_allclose(oracle.ns_tile(Y, K, co), closed_form(Y, K, co), atol=1e-14, rtol=0)
    # 1x1: x -> phi^K(y / (|y| + eps))
    y = -0.3
    assert abs(oracle.ns_tile(np.array([[y]]), 5, Q)[0, 0]
               - oracle.phi_iterate(y / (abs(y) + EPS), 5, Q)) < 1e-15


# ------------------------------------------------------------------ momentum / update / bf16
def test_bf16_round_matches_torch():
    x = np.random.default_rng(15).standard_normal(100000).astype(np.float32) * 10
    x[:8] = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 65504.0, 1e-40, 3.0e38, -2.5]
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_round(x).view(np.uint32), want.view(np.uint32))
    assert oracle.bf16_round(np.float32(1 + 2 ** -8))[()] == 1.0            # tie to even
    assert oracle.bf16_round(np.float32(1 + 3 * 2 ** -8))[()] == 1 + 2 ** -6  # tie to even (up)


def test_momentum_first_step_is_gradient_and_second_step_combines():
    G1 = rng_matrix(8, 9, 16)
    G2 = rng_matrix(8, 9, 17)
    M1 = oracle.momentum(np.zeros((8, 9)), G1, 0.95)
    assert np.array_equal(M1, G1)
    np.testing.assert_allclose(oracle.momentum(M1, G2, 0.95), 0.95 * G1 + G2, rtol=1e-15)
    Gb = oracle.bf16_round(G1.astype(np.float32))
    assert np.array_equal(oracle.momentum_stored(np.zeros((8, 9)), Gb, 0.95, "bf16"), Gb)
    m2 = oracle.momentum_stored(Gb, Gb, 0.95, "f32")
    np.testing.assert_allclose(m2, np.float32(0.95) * Gb.astype(np.float64) + Gb, rtol=6e-8)


def test_momentum_stored_rounds_once_then_to_bf16():
    """beta M + G is one fused multiply-add: rounded to float32 once, then (bf16 state)
    rounded from that float32 value to bfloat16.  Values derived by hand in exact rational
    arithmetic; a product rounded before the add, or a direct rounding to bf16, fails."""
    from fractions import Fraction as Fr
    b32 = Fr(15938355, 2 ** 24)                      # float32(0.95) = 0x3F733333
    assert b32 == Fr(float(np.float32(0.95)))
    # (1) M = 1 + 2^-23: beta M = 2^-24 (15938356 + 0.89999997...), which float32 rounds
    # to 15938357 2^-24.  With G = -15938357 2^-24 a separate product and add give 0; the
    # fused form keeps the product's rounding error, -838861 2^-47 (exact in float32).
    M = np.array([[1 + 2.0 ** -23]], dtype=np.float32)
    G = np.array([[-15938357 * 2.0 ** -24]], dtype=np.float32)
    assert Fr(float(M[0, 0])) * b32 + Fr(float(G[0, 0])) == Fr(-838861, 2 ** 47)
    out = oracle.momentum_stored(M, G, 0.95, "f32")
    assert out.dtype == np.float32 and out[0, 0] == np.float32(-838861 * 2.0 ** -47)
    assert np.float32(np.float32(b32) * M[0, 0]) + G[0, 0] == 0        # the two-rounding result
    # (2) M = 1 + 5 2^-23: beta M = 2^-24 (15938364 + 0.49999988...), G = 904388 2^-24, so
    # beta M + G = 1 + 2^-8 + 0.49999988 2^-24.  float32 rounds that to 1 + 2^-8 (the
    # remainder is below half an ulp, 2^-24), a bf16 tie that goes to even: 1.0.  Rounded
    # straight to bf16 it would be 1 + 2^-7.
    M = np.array([[1 + 5 * 2.0 ** -23]], dtype=np.float32)
    G = np.array([[904388 * 2.0 ** -24]], dtype=np.float32)
    ex = Fr(float(M[0, 0])) * b32 + Fr(float(G[0, 0]))
    assert 0 < ex - (1 + Fr(1, 256)) < Fr(1, 2 ** 24)
    assert oracle.momentum_stored(M, G, 0.95, "f32")[0, 0] == np.float32(1 + 2.0 ** -8)
    assert oracle.momentum_stored(M, G, 0.95, "bf16")[0, 0] == np.float32(1.0)


def test_step_updates_weights_against_the_direction():
    W = rng_matrix(64, 96, 18)
    G = rng_matrix(64, 96, 19)
    (Wn, Mn, O), = oracle.step([(W, np.zeros_like(W), G)], 32, 5, Q, beta=0.9, lr=0.02)
    np.testing.assert_allclose(O, oracle.tiled_ns(G, 32, 5, Q), rtol=0, atol=0)
    np.testing.assert_allclose(Wn, W - 0.02 * O, rtol=0, atol=1e-16)
    # the update is a descent direction for the linear model <G, W>
    assert np.sum(G * (Wn - W)) < 0

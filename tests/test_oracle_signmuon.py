"""Pins of the oracle's Sign-Muon pieces (CPU): hand-worked bytes, round trips,
brute-force votes on tiny inputs, and agreement with numpy's own bit packing."""
import itertools

import numpy as np
import pytest

from oracle import signmuon as sm


def test_sign_convention():
    assert sm.sign(np.array([-2.0, -0.0, 0.0, 1e-30, -1e-30, 3.0])).tolist() == [-1, 1, 1, 1, -1, 1]


def test_pack_hand_worked_bytes():
    # entries (row-major): + - - + + + - -  | + -   -> 0b00111001, 0b00000001
    S = np.array([[1, -1, -1, 1, 1], [1, -1, -1, 1, -1]], dtype=np.int8)
    assert sm.pack(S).tolist() == [0b00111001, 0b00000001]


@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 64, 65, 1000])
def test_pack_matches_numpy_packbits_and_round_trips(n):
    rng = np.random.default_rng(n)
    S = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
    bits = sm.pack(S)
    assert bits.size == (n + 7) // 8
    assert np.array_equal(bits, np.packbits(S > 0, bitorder="little"))
    assert np.array_equal(sm.unpack(bits, n), S)


def test_vote_brute_force_three_workers_all_patterns():
    # every combination of three signs on 8 entries covers all 2^3 voter patterns
    patterns = list(itertools.product([-1, 1], repeat=3))
    S = np.array(patterns, dtype=np.int8).T            # 3 workers x 8 entries
    want = [1 if sum(p) > 0 else -1 for p in patterns]
    got = sm.vote([sm.pack(s) for s in S], 8)
    assert got.tolist() == want


def test_vote_tie_is_plus_one_and_single_worker_is_identity():
    a = np.array([1, -1, 1, -1], dtype=np.int8)
    b = np.array([-1, 1, 1, -1], dtype=np.int8)
    assert sm.vote([sm.pack(a), sm.pack(b)], 4).tolist() == [1, 1, 1, -1]
    assert np.array_equal(sm.vote([sm.pack(a)], 4), a)

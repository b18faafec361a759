"""Pins for the rotary oracle (FastVideo gemma page: ``precompute_ltx_freqs_cis``
normalises positions by ``max_pos`` with base ``theta``; ``LTXRopeType``
INTERLEAVED rotates channel pairs (2i, 2i+1); the schedule is a stated
reading, pinned here to hand-derived closed forms)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import rope_angles, rope_apply


def _cases(golden_dir):
    return json.load(open(os.path.join(golden_dir, "rope_angles.json")))["cases"]


def test_angles_match_closed_forms(golden_dir):
    for case in _cases(golden_dir):
        pos = np.array([case["pos"]], dtype=np.int32)
        phi = rope_angles(pos, case["max_pos"], case["head_dim"], case["theta"])[0]
        assert phi.shape == (case["head_dim"] // 2,)
        for i, want in case["angles"].items():
            assert phi[int(i)] == pytest.approx(want, rel=1e-13, abs=1e-300), (case["name"], i)
        if case["complete"]:
            assert len(case["angles"]) == case["head_dim"] // 2


def test_rotation_of_unit_vectors_is_cos_sin(golden_dir):
    # (1, 0) -> (cos phi, sin phi) and (0, 1) -> (-sin phi, cos phi): pins the
    # direction of the turn and which channel of the pair is which.
    for case in _cases(golden_dir):
        D = case["head_dim"]
        pos = np.array([case["pos"]], dtype=np.int32)
        e0 = np.zeros((1, 1, 1, D)); e0[..., 0::2] = 1.0
        e1 = np.zeros((1, 1, 1, D)); e1[..., 1::2] = 1.0
        y0 = rope_apply(e0, pos, case["max_pos"], case["theta"])[0, 0, 0]
        y1 = rope_apply(e1, pos, case["max_pos"], case["theta"])[0, 0, 0]
        for i, phi in case["angles"].items():
            i = int(i)
            assert y0[2 * i] == pytest.approx(math.cos(phi), abs=1e-15)
            assert y0[2 * i + 1] == pytest.approx(math.sin(phi), abs=1e-15)
            assert y1[2 * i] == pytest.approx(-math.sin(phi), abs=1e-15)
            assert y1[2 * i + 1] == pytest.approx(math.cos(phi), abs=1e-15)


def test_one_radian_closed_form():
    # One axis, first pair, pos == max_pos: a turn of exactly 1 rad.
    pos = np.array([[7]], dtype=np.int32)
    x = np.zeros((1, 1, 1, 4)); x[..., 0] = 1.0
    y = rope_apply(x, pos, [7], 10000.0)[0, 0, 0]
    assert y[0] == pytest.approx(0.5403023058681398, abs=1e-15)
    assert y[1] == pytest.approx(0.8414709848078965, abs=1e-15)


def test_position_zero_is_identity_bit_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 3, 128))
    pos = np.zeros((5, 3), dtype=np.int32)
    assert np.array_equal(rope_apply(x, pos, [16, 32, 64], 10000.0), x)


def test_pair_norms_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 50, 4, 128))
    pos = rng.integers(0, 64, size=(50, 3)).astype(np.int32)
    y = rope_apply(x, pos, [16, 32, 64], 10000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


@pytest.mark.parametrize("D,A", [(128, 3), (64, 3), (64, 1)])
def test_leftover_pairs_untouched_bit_exact(D, A):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 20, 2, D))
    pos = rng.integers(1, 9, size=(20, A)).astype(np.int32)
    y = rope_apply(x, pos, [9.0] * A, 10000.0)
    n_rot = 2 * A * ((D // 2) // A)
    assert np.array_equal(y[..., n_rot:], x[..., n_rot:])
    assert not np.allclose(y[..., :n_rot], x[..., :n_rot])


def test_relative_position_property_one_axis():
    # <R(m) q, R(n) k> depends only on m - n.
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, 1, D))
    def rot(x, p):
        return rope_apply(x, np.array([[p]], dtype=np.int32), [1000.0], 10000.0)[0, 0, 0]
    for m, n in [(10, 3), (500, 493), (999, 992), (7, 0)]:
        lhs = float(rot(q, m) @ rot(k, n))
        rhs = float(rot(q, m - n) @ k[0, 0, 0])
        assert lhs == pytest.approx(rhs, abs=1e-12)


def test_axes_act_on_their_own_pair_blocks():
    # Moving along x changes only pairs [n_ax, 2 n_ax); the angle is linear in pos.
    D, A = 128, 3
    n_ax = (D // 2) // A
    base = np.array([[3, 5, 7]], dtype=np.int32)
    moved = np.array([[3, 9, 7]], dtype=np.int32)
    mp = [16, 32, 64]
    d = rope_angles(moved, mp, D, 10000.0) - rope_angles(base, mp, D, 10000.0)
    assert np.all(d[0, :n_ax] == 0) and np.all(d[0, 2 * n_ax:] == 0)
    np.testing.assert_allclose(d[0, n_ax:2 * n_ax],
                               rope_angles(np.array([[0, 4, 0]]), mp, D, 10000.0)[0, n_ax:2 * n_ax],
                               rtol=1e-14)


def test_same_rotation_for_every_head_and_batch():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(64)
    x = np.broadcast_to(row, (2, 6, 4, 64)).copy()
    pos = rng.integers(0, 11, size=(6, 3)).astype(np.int32)
    y = rope_apply(x, pos, [3, 7, 11], 10000.0)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(y[b, :, h], y[0, :, 0])


def test_invalid_arguments():
    with pytest.raises(ValueError):
        rope_angles(np.zeros((2, 3), np.int32), [1, 1], 64, 1e4)
    with pytest.raises(ValueError):
        rope_angles(np.zeros((2, 3), np.int32), [1, 0, 1], 64, 1e4)
    with pytest.raises(ValueError):
        rope_angles(np.zeros((2, 3), np.int32), [1, 1, 1], 63, 1e4)

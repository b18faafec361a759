"""Pins for the masked-attention oracle (LTX-2 SP page: global attention over
all tokens per head; padded keys masked out, padded rows discarded; SP is
numerically the single-GPU result)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention


def brute_attention(q, k, v, nk_valid, scale):
    """Scalar loops with exact summation (math.fsum), one query at a time."""
    B, Nq, H, D = q.shape
    o = np.zeros((B, Nq, H, D))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                s = [scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, h, d]) for d in range(D))
                     for j in range(nk_valid)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = math.fsum(w)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(w[j] * float(v[b, j, h, d]) for j in range(nk_valid)) / z
                lse[b, h, i] = m + math.log(z)
    return o, lse


def test_two_key_closed_form(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "attn_two_keys.json")))
    q = np.array(fx["q"])[None, :, None, :]
    k = np.array(fx["k"])[None, :, None, :]
    v = np.array(fx["v"])[None, :, None, :]
    o, lse = attention(q, k, v, fx["nk_valid"], fx["scale"])
    e = math.e
    assert o[0, 0, 0, 0] == pytest.approx(e / (1 + e), abs=1e-15)
    assert o[0, 0, 0, 1] == pytest.approx(1 / (1 + e), abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(1 + e), abs=1e-15)


def test_matches_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(10)
    B, Nq, Nk, H, D = 2, 9, 13, 3, 8
    q = rng.standard_normal((B, Nq, H, D))
    k = rng.standard_normal((B, Nk, H, D))
    v = rng.standard_normal((B, Nk, H, D))
    for nk_valid in (1, 7, 13):
        o, lse = attention(q, k, v, nk_valid, 0.37)
        bo, blse = brute_attention(q, k, v, nk_valid, 0.37)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_matches_brute_force_rows_subset():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 40, 2, 16))
    k = rng.standard_normal((1, 30, 2, 16))
    v = rng.standard_normal((1, 30, 2, 16))
    rows = np.array([0, 5, 39, 17])
    o, lse = attention(q, k, v, 25, 0.25, rows=rows)
    bo, blse = brute_attention(q[:, rows], k, v, 25, 0.25)
    np.testing.assert_allclose(o, bo, atol=1e-12)
    np.testing.assert_allclose(lse, blse, atol=1e-12)


def test_zero_query_gives_mean_of_valid_values():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((1, 50, 2, 32))
    v = rng.standard_normal((1, 50, 2, 32))
    v[:, 40:] = 1e6          # padded values must not leak
    q = np.zeros((1, 8, 2, 32))
    o, lse = attention(q, k, v, 40, 0.125)
    want = v[:, :40].mean(axis=1)                        # [1, 2, 32]
    for i in range(8):
        np.testing.assert_allclose(o[:, i], want, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(40), atol=1e-13)


def test_dominant_logit_selects_its_value_row():
    # Query i points at key perm[i] with a score gap of 60: O[i] = V[perm[i]].
    D = 16
    n = 12
    perm = np.array([3, 0, 11, 7, 7, 2, 9, 1, 5, 10, 4, 6])
    k = np.zeros((1, n, 1, D)); k[0, np.arange(n), 0, np.arange(n)] = 1.0
    q = np.zeros((1, n, 1, D)); q[0, np.arange(n), 0, perm] = 60.0
    rng = np.random.default_rng(14)
    v = rng.standard_normal((1, n, 1, D))
    o, _ = attention(q, k, v, n, 1.0)
    np.testing.assert_allclose(o[0, :, 0], v[0, perm, 0], atol=1e-15)


def test_rows_of_weights_sum_to_one():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 30, 2, 64)) * 3
    k = rng.standard_normal((1, 40, 2, 64)) * 3
    v = np.ones((1, 40, 2, 64))
    o, _ = attention(q, k, v, 33, 0.125)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)


def test_padding_invariance():
    # Valid rows of a padded run equal the unpadded run; padded K/V hold garbage.
    rng = np.random.default_rng(16)
    n = 37
    q = rng.standard_normal((1, n, 2, 16))
    k = rng.standard_normal((1, n, 2, 16))
    v = rng.standard_normal((1, n, 2, 16))
    o_ref, lse_ref = attention(q, k, v, n, 0.25)
    pad = 11
    qp = np.concatenate([q, rng.standard_normal((1, pad, 2, 16))], axis=1)
    kp = np.concatenate([k, np.full((1, pad, 2, 16), 1e300)], axis=1)
    vp = np.concatenate([v, np.full((1, pad, 2, 16), np.nan)], axis=1)
    o, lse = attention(qp, kp, vp, n, 0.25)
    np.testing.assert_array_equal(o[:, :n], o_ref)
    np.testing.assert_array_equal(lse[:, :, :n], lse_ref)


def test_key_permutation_invariance_and_query_equivariance():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((1, 10, 1, 8))
    k = rng.standard_normal((1, 15, 1, 8))
    v = rng.standard_normal((1, 15, 1, 8))
    o, _ = attention(q, k, v, 15, 0.5)
    pk = rng.permutation(15)
    pq = rng.permutation(10)
    o2, _ = attention(q[:, pq], k[:, pk], v[:, pk], 15, 0.5)
    np.testing.assert_allclose(o2, o[:, pq], atol=1e-13)


def test_scale_to_zero_gives_mean():
    rng = np.random.default_rng(18)
    q = rng.standard_normal((1, 4, 1, 8))
    k = rng.standard_normal((1, 9, 1, 8))
    v = rng.standard_normal((1, 9, 1, 8))
    o, _ = attention(q, k, v, 9, 0.0)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (4, 8)), atol=1e-14)


def test_invalid_nk_valid():
    z = np.zeros((1, 4, 1, 8))
    with pytest.raises(ValueError):
        attention(z, z, z, 0, 1.0)
    with pytest.raises(ValueError):
        attention(z, z, z, 5, 1.0)

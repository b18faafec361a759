"""Pins for the rotary oracle's variants (FastVideo gemma page:
``LTXRopeType`` has an interleaved and a split pairing;
``precompute_ltx_freqs_cis`` takes ``dim``, ``num_attention_heads`` and
``use_middle_indices_grid``, and the 1D connector passes the inner dimension
``heads * head_dim``).  The readings are stated in ``oracle/rope.py``; here
they are pinned to hand-derived angles and to identities that tie each
variant to the pinned base case."""

import json
import math
import os

import numpy as np
import pytest

from oracle import rope_angles, rope_apply


def _cases(golden_dir):
    return json.load(open(os.path.join(golden_dir, "rope_variants.json")))["cases"]


def test_variant_angles_match_closed_forms(golden_dir):
    for c in _cases(golden_dir):
        pos = np.array([c["pos"]], dtype=np.int32)
        for h, want in c["heads"].items():
            phi = rope_angles(pos, c["max_pos"], c["head_dim"], c["theta"], grid_heads=c["grid_heads"],
                              head=int(h), middle=c["middle"])[0]
            assert len(want) == c["head_dim"] // 2
            np.testing.assert_allclose(phi, want, rtol=1e-13, atol=0, err_msg=f"{c['name']} head {h}")


@pytest.mark.parametrize("G,D,A", [(4, 64, 3), (32, 128, 1), (3, 10, 3)])
def test_inner_grid_is_the_wide_per_head_grid_cut_into_heads(G, D, A):
    # Head h of a grid over G heads of D channels is slice h of the per-head
    # grid of one head of G*D channels.
    rng = np.random.default_rng(10)
    pos = rng.integers(0, 50, size=(7, A)).astype(np.int32)
    mp = [50.0] * A
    wide = rope_angles(pos, mp, G * D, 10000.0)
    cut = np.concatenate([rope_angles(pos, mp, D, 10000.0, grid_heads=G, head=h) for h in range(G)], axis=1)
    assert np.array_equal(cut, wide)


def test_one_head_grid_is_the_per_head_grid():
    rng = np.random.default_rng(11)
    pos = rng.integers(0, 9, size=(5, 3)).astype(np.int32)
    a = rope_angles(pos, [9, 9, 9], 64, 10000.0)
    b = rope_angles(pos, [9, 9, 9], 64, 10000.0, grid_heads=1, head=0)
    assert np.array_equal(a, b)


def test_inner_grid_head_offset_selects_the_same_heads():
    # Rotating a run of heads with a head offset equals rotating the full
    # G-head tensor and taking those heads.
    rng = np.random.default_rng(12)
    G, D = 8, 32
    x = rng.standard_normal((2, 6, G, D))
    pos = rng.integers(0, 10, size=(6, 3)).astype(np.int32)
    full = rope_apply(x, pos, [10, 10, 10], 10000.0, grid_heads=G)
    for off, H in [(0, 8), (2, 2), (6, 2), (5, 1)]:
        part = rope_apply(x[:, :, off:off + H], pos, [10, 10, 10], 10000.0, grid_heads=G, head_offset=off)
        assert np.array_equal(part, full[:, :, off:off + H])
    with pytest.raises(ValueError):
        rope_apply(x[:, :, :4], pos, [10, 10, 10], 10000.0, grid_heads=G, head_offset=5)


def test_inner_grid_heads_differ_and_per_head_grid_does_not():
    rng = np.random.default_rng(13)
    row = rng.standard_normal(32)
    x = np.broadcast_to(row, (1, 4, 4, 32)).copy()
    pos = np.array([[3], [5], [7], [9]], dtype=np.int32)
    y = rope_apply(x, pos, [10.0], 10000.0, grid_heads=4)
    assert not np.allclose(y[:, :, 0], y[:, :, 1])
    z = rope_apply(x, pos, [10.0], 10000.0)
    assert np.array_equal(z[:, :, 0], z[:, :, 3])


def _split_to_interleaved(x):
    # Channel i -> 2i and channel i + D/2 -> 2i + 1.
    D = x.shape[-1]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., :D // 2]
    y[..., 1::2] = x[..., D // 2:]
    return y


def _interleaved_to_split(y):
    D = y.shape[-1]
    return np.concatenate([y[..., 0::2], y[..., 1::2]], axis=-1)


@pytest.mark.parametrize("grid_heads,middle", [(0, False), (4, False), (0, True)])
def test_split_is_interleaved_on_permuted_channels(grid_heads, middle):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((2, 9, 4, 64))
    pos = rng.integers(0, 12, size=(9, 3)).astype(np.int32)
    kw = dict(grid_heads=grid_heads, middle=middle)
    s = rope_apply(x, pos, [12, 12, 12], 10000.0, rope_type="split", **kw)
    i = rope_apply(_split_to_interleaved(x), pos, [12, 12, 12], 10000.0, **kw)
    assert np.array_equal(s, _interleaved_to_split(i))


def test_split_unit_vectors(golden_dir):
    # (1 at channel i) -> (cos phi_i at i, sin phi_i at i + D/2);
    # (1 at channel i + D/2) -> (-sin phi_i at i, cos phi_i at i + D/2).
    D = 8
    pos = np.array([[4]], dtype=np.int32)
    phis = [1.0, 0.1, 0.01, 0.001]     # one_axis_d8 of rope_angles.json
    for i, phi in enumerate(phis):
        for src, want in ((i, {i: math.cos(phi), i + D // 2: math.sin(phi)}),
                          (i + D // 2, {i: -math.sin(phi), i + D // 2: math.cos(phi)})):
            e = np.zeros((1, 1, 1, D)); e[..., src] = 1.0
            y = rope_apply(e, pos, [4], 10000.0, rope_type="split")[0, 0, 0]
            for ch in range(D):
                assert y[ch] == pytest.approx(want.get(ch, 0.0), abs=1e-15), (src, ch)


def test_split_preserves_pair_norms_and_position_zero():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((1, 20, 2, 128))
    pos = rng.integers(0, 30, size=(20, 3)).astype(np.int32)
    y = rope_apply(x, pos, [30, 30, 30], 10000.0, rope_type="split")
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)
    z = np.zeros((20, 3), dtype=np.int32)
    assert np.array_equal(rope_apply(x, z, [30, 30, 30], 10000.0, rope_type="split"), x)


def test_middle_is_doubled_position_over_doubled_extent():
    # (p + 1/2) / m == (2p + 1) / (2m) exactly in binary floating point.
    rng = np.random.default_rng(16)
    pos = rng.integers(0, 40, size=(11, 3)).astype(np.int32)
    mp = [16, 32, 64]
    a = rope_angles(pos, mp, 128, 10000.0, middle=True)
    b = rope_angles(2 * pos + 1, [2 * m for m in mp], 128, 10000.0)
    assert np.array_equal(a, b)


def test_relative_position_property_holds_per_head_on_the_inner_grid():
    rng = np.random.default_rng(17)
    G, D = 4, 32
    q = rng.standard_normal((1, 1, G, D))
    k = rng.standard_normal((1, 1, G, D))
    def rot(x, p):
        return rope_apply(x, np.array([[p]], dtype=np.int32), [100.0], 10000.0, grid_heads=G)[0, 0]
    for m, n in [(10, 3), (99, 92)]:
        for h in range(G):
            lhs = float(rot(q, m)[h] @ rot(k, n)[h])
            rhs = float(rot(q, m - n)[h] @ k[0, 0, h])
            assert lhs == pytest.approx(rhs, abs=1e-12)


def test_variant_arguments_rejected():
    pos = np.zeros((2, 1), np.int32)
    with pytest.raises(ValueError):
        rope_angles(pos, [1], 8, 1e4, grid_heads=2, head=2)
    with pytest.raises(ValueError):
        rope_apply(np.zeros((1, 2, 1, 8)), pos, [1], 1e4, rope_type="neox")

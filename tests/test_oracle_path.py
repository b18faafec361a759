"""Pins for the end-to-end oracle: the SP procedure over P virtual ranks equals
single-GPU attention (LTX-2 SP page, "What it is": numerically equivalent to
single-GPU inference; "How the forward pass works": pad, exchange heads,
attend, shuffle back, unpad)."""

import numpy as np
import pytest

from oracle import sp_path_single_gpu, sp_path_virtual_ranks
from video_dit_sequence_amd import workloads as wl


def _tiny_inputs(heads):
    w = wl.WORKLOADS["tiny_231"]
    q, k, v = wl.qkv(w, heads=heads)
    n = w.nq_valid
    pos = wl.video_positions(w.q_grid)
    return (wl.to_f64(q)[:, :n], wl.to_f64(k)[:, :n], wl.to_f64(v)[:, :n], pos, w)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_head_share_over_virtual_ranks_equals_single_gpu(P):
    q, k, v, pos, w = _tiny_inputs(heads=4)
    ref = sp_path_single_gpu(q, k, v, pos, pos, w.q_max_pos, w.k_max_pos, w.theta, w.scale)
    got = sp_path_virtual_ranks(q, k, v, pos, pos, w.q_max_pos, w.k_max_pos, w.theta, w.scale,
                                world_size=P, pad_value=np.nan)
    assert got.shape == ref.shape
    # Each head sees the same operands in the same order whatever P is.
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_virtual_ranks_reject_indivisible_heads():
    q, k, v, pos, w = _tiny_inputs(heads=2)
    with pytest.raises(ValueError):
        sp_path_virtual_ranks(q, k, v, pos, pos, w.q_max_pos, w.k_max_pos, w.theta, w.scale, 4)


def test_cross_attention_shapes():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 30, 4, 64))
    k = rng.standard_normal((1, 10, 4, 64))
    v = rng.standard_normal((1, 10, 4, 64))
    qpos = wl.video_positions((2, 3, 5))
    kpos = wl.audio_positions(10)
    ref = sp_path_single_gpu(q, k, v, qpos, kpos, (2, 3, 5), (10,), 1e4, 0.125)
    with np.errstate(invalid="ignore"):   # inf padding turns into NaN under rotation; it is masked
        got = sp_path_virtual_ranks(q, k, v, qpos, kpos, (2, 3, 5), (10,), 1e4, 0.125,
                                    world_size=4, pad_value=np.inf)
    np.testing.assert_allclose(got, ref, atol=1e-13)


def test_workload_positions_layout():
    # Raster order (t slowest, y fastest) and zero positions on padded rows.
    w = wl.WORKLOADS["ragged_32761"]
    qpos, kpos = wl.positions(w)
    assert qpos.shape == (32768, 3) and np.array_equal(qpos, kpos)
    assert w.nq_valid == 32761
    T, X, Y = w.q_grid
    assert tuple(qpos[1]) == (0, 0, 1) and tuple(qpos[Y]) == (0, 1, 0)
    assert tuple(qpos[X * Y]) == (1, 0, 0)
    assert tuple(qpos[T * X * Y]) == (13, 0, 0)
    assert tuple(qpos[32760]) == (13, 5, 18)
    assert np.all(qpos[32761:] == 0)
    assert np.all(qpos[:32761].max(axis=0) < np.array(w.q_max_pos))
    w5 = wl.WORKLOADS["cross_24576x1000"]
    q5, k5 = wl.positions(w5)
    assert q5.shape == (24576, 3) and k5.shape == (1024, 1)
    assert k5[999, 0] == 999 and np.all(k5[1000:] == 0)

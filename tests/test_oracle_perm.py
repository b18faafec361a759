"""Pins for the layout-transform oracle (LTX-2 SP page, "What it is": each rank
ends up with all tokens of a head subset; the exchange moves bytes only and
its round trip is byte-exact; "API / AttentionManager": heads divisible by
world_size; "How the forward pass works" step 1: pad to a multiple of
world_size)."""

import json
import os

import numpy as np
import pytest

from oracle import pad_length, sp_pack, sp_unpack


def test_pack_matches_hand_written_fixture(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "pack_tiny.json")))
    for case in fx["cases"]:
        src = np.array(case["src"], dtype=np.int64)
        want = np.array(case["dst"], dtype=np.int64)
        assert src.shape == (case["B"], case["N"], case["H"], case["D"])
        got = sp_pack(src, case["P"])
        assert got.shape == want.shape, case["name"]
        np.testing.assert_array_equal(got, want, err_msg=case["name"])
        np.testing.assert_array_equal(sp_unpack(want), src, err_msg=case["name"])


@pytest.mark.parametrize("B,N,H,D,P", [(1, 5, 8, 4, 4), (2, 3, 6, 2, 3), (1, 7, 4, 8, 1)])
def test_pack_equals_numpy_transpose(B, N, H, D, P):
    # The packed layout is the head axis split as (P, H/P) and moved to the front.
    rng = np.random.default_rng(7)
    src = rng.integers(0, 2**16, size=(B, N, H, D), dtype=np.uint16)
    want = np.transpose(src.reshape(B, N, P, H // P, D), (2, 0, 1, 3, 4))
    np.testing.assert_array_equal(sp_pack(src, P), want)


def test_pack_brute_force_index_loops():
    rng = np.random.default_rng(11)
    B, N, H, D, P = 2, 3, 4, 3, 2
    src = rng.integers(0, 2**16, size=(B, N, H, D), dtype=np.uint16)
    dst = sp_pack(src, P)
    Hl = H // P
    for p in range(P):
        for b in range(B):
            for n in range(N):
                for j in range(Hl):
                    for d in range(D):
                        assert dst[p, b, n, j, d] == src[b, n, p * Hl + j, d]


def test_round_trip_is_byte_exact_for_bf16_bit_patterns():
    # Every 16-bit pattern, NaNs and infinities included, survives the round trip.
    bits = np.arange(2**16, dtype=np.uint16).reshape(1, 1024, 8, 8)
    for P in (1, 2, 4, 8):
        packed = sp_pack(bits, P)
        assert np.array_equal(sp_unpack(packed), bits)
        assert np.array_equal(sp_pack(sp_unpack(packed), P), packed)


def test_one_rank_is_identity():
    x = np.arange(2 * 3 * 4 * 5, dtype=np.uint16).reshape(2, 3, 4, 5)
    np.testing.assert_array_equal(sp_pack(x, 1)[0], x)


def test_heads_must_divide_by_world_size():
    with pytest.raises(ValueError):
        sp_pack(np.zeros((1, 232, 2, 64), np.uint16), 4)


@pytest.mark.parametrize("n,P,want", [(231, 4, 232), (232, 4, 232), (32761, 8, 32768),
                                      (32761, 2, 32762), (32761, 4, 32764), (0, 8, 0),
                                      (1, 8, 8), (6144, 1, 6144)])
def test_pad_length(n, P, want):
    assert pad_length(n, P) == want

"""Oracle for the token-sharded <-> head-sharded layout transform (one GPU's share
of the sequence-parallel all2all).  Test infrastructure only.

Source: LTX-2 "Sequence Parallelism (SP)" page.
* "What it is": after the exchange each rank holds *all* tokens for a subset
  of the heads; the results are shuffled back afterwards; the exchange moves
  bytes only and its round trip is byte-exact.
* "How the forward pass works", step 1: the video sequence dimension is padded
  up to a multiple of ``world_size`` so that every rank gets an equal shard.
* "API / AttentionManager": ``num_heads`` must be divisible by ``world_size``.

Readings taken where the page is silent:
* Rank ``p`` of ``P`` owns the contiguous head block ``[p*H/P, (p+1)*H/P)``.
* The packed layout is ``[P, B, N, H/P, D]``: rank ``p``'s receive buffer is
  ``dst[p]``, itself a ``[B, N, H/P, D]`` token-major tensor over all tokens.
"""

import numpy as np


def pad_length(n_valid: int, world_size: int) -> int:
    """Padded token count: the smallest multiple of ``world_size`` that is
    >= ``n_valid`` (SP page, "How the forward pass works", step 1)."""
    if n_valid < 0 or world_size < 1:
        raise ValueError("n_valid must be >= 0 and world_size >= 1")
    return -(-n_valid // world_size) * world_size


def sp_pack(src: np.ndarray, world_size: int) -> np.ndarray:
    """Token-major ``[B, N, H, D]`` -> per-rank head shards ``[P, B, N, H/P, D]``.

    Definition: ``dst[p, b, n, j, d] = src[b, n, p*(H/P) + j, d]``.
    Any dtype; a pure copy (SP page, "What it is": the exchange moves bytes only).
    """
    B, N, H, D = src.shape
    P = world_size
    if P < 1 or H % P != 0:
        raise ValueError("num_heads must be divisible by world_size")
    Hl = H // P
    dst = np.empty((P, B, N, Hl, D), dtype=src.dtype)
    for p in range(P):
        dst[p] = src[:, :, p * Hl:(p + 1) * Hl, :]
    return dst


def sp_unpack(src: np.ndarray) -> np.ndarray:
    """Inverse of :func:`sp_pack`: ``[P, B, N, H/P, D]`` -> ``[B, N, H, D]``.

    Definition: ``dst[b, n, p*(H/P) + j, d] = src[p, b, n, j, d]`` (SP page,
    "What it is": the per-head results are shuffled back to token order).
    """
    P, B, N, Hl, D = src.shape
    dst = np.empty((B, N, P * Hl, D), dtype=src.dtype)
    for p in range(P):
        dst[:, :, p * Hl:(p + 1) * Hl, :] = src[p]
    return dst

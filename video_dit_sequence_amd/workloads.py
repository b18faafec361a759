"""Seeded synthetic inputs for the sequence-parallel attention path.

This module only draws numbers and lays out integer token positions; it holds
none of the path's arithmetic.  Both the HIP path's tests/bench and the CPU
oracle's tests take their inputs from here.

Workloads (token counts follow the LTX-2 "Sequence Parallelism (SP)" page,
"Usage": about 6k video tokens for the stage-1 call at 512x768x121, about 24k
for the full-resolution distilled call, and a 32768-token cap):

* ``tiny_231``      -- 3x7x11 = 231 video tokens padded to 232 (a multiple of
                       4 ranks), 2 heads of 64 channels.  Small enough for
                       the oracle and a pure-Python brute force.
* ``full_6144``     -- 8x24x32 = 6144 tokens, 32 heads of 128, no padding.
* ``share_32768``   -- one rank's share at the 32768 cap: 8 ranks, 4 of 32
                       heads of 128 channels, 16x32x64 tokens.  The full
                       32-head tensor is what the layout transform moves.
* ``ragged_32761``  -- 13x49x51 + 274 tokens at t = 13 (32761) padded to
                       32768, 32 heads of 128; split over 2, 4 or 8 ranks.
* ``cross_24576x1000`` -- video queries 12x32x64 = 24576 (3-axis positions)
                       against 1000 audio keys (1-axis positions) padded to
                       1024; 4 heads (of 32) of 64 channels.
* ``connector_1024`` -- the text connector's 1D self-attention (FastVideo
                       gemma page, ``Embeddings1DConnector``): 1024 text
                       tokens at positions 0..1023, 32 heads of 128, batch
                       2.  Its rotary grid spans the inner dimension (32
                       heads x 128).  With learnable registers every slot is
                       valid (the mask is reset to zeros), so all 1024 keys
                       attend.
* ``connector_1024_masked`` -- the same without registers: an additive mask
                       whose valid prefix is 700 tokens, i.e. ``nk_valid`` =
                       700; batch 1.

The pages print no connector sizes; 1024 tokens, 32 x 128 and max_pos 1024
are this library's choices.

Values: independent N(0, 1) draws from ``torch.Generator('cpu')`` seeded per
workload, rounded to bfloat16 (round to nearest even).  Q, K and V are drawn
in that order from one generator.  Token order is raster order (t slowest,
then x, then y); padded tokens carry position 0 on every axis.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    heads: int              # heads in one attention call (one rank's share)
    head_dim: int
    nq: int                 # query rows in the call (padded length for self-attn)
    nk_pad: int             # key rows in memory
    nk_valid: int           # keys that take part in the softmax
    q_grid: Tuple[int, int, int]
    q_extra: int            # extra tokens appended on the t = T plane
    q_max_pos: Tuple[float, ...]
    k_kind: str             # "video" (same positions as the queries), "audio" or "text"
    k_max_pos: Tuple[float, ...]
    full_heads: int         # heads of the token-major tensor before the exchange
    world_sizes: Tuple[int, ...] = field(default=(1,))
    theta: float = 10000.0
    q_kind: str = "video"   # "video": 3-axis grid positions; "text": 1-axis 0..nq-1

    @property
    def nq_valid(self) -> int:
        if self.q_kind == "text":
            return self.nk_valid
        t, x, y = self.q_grid
        return t * x * y + self.q_extra

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS = {
    "tiny_231": Workload(
        name="tiny_231", seed=1000, B=1, heads=2, head_dim=64,
        nq=232, nk_pad=232, nk_valid=231, q_grid=(3, 7, 11), q_extra=0,
        q_max_pos=(3, 7, 11), k_kind="video", k_max_pos=(3, 7, 11),
        full_heads=2, world_sizes=(4,)),
    "full_6144": Workload(
        name="full_6144", seed=1001, B=1, heads=32, head_dim=128,
        nq=6144, nk_pad=6144, nk_valid=6144, q_grid=(8, 24, 32), q_extra=0,
        q_max_pos=(8, 24, 32), k_kind="video", k_max_pos=(8, 24, 32),
        full_heads=32, world_sizes=(1,)),
    "share_32768": Workload(
        name="share_32768", seed=1002, B=1, heads=4, head_dim=128,
        nq=32768, nk_pad=32768, nk_valid=32768, q_grid=(16, 32, 64), q_extra=0,
        q_max_pos=(16, 32, 64), k_kind="video", k_max_pos=(16, 32, 64),
        full_heads=32, world_sizes=(8,)),
    "ragged_32761": Workload(
        name="ragged_32761", seed=1003, B=1, heads=32, head_dim=128,
        nq=32768, nk_pad=32768, nk_valid=32761, q_grid=(13, 49, 51), q_extra=274,
        q_max_pos=(14, 49, 51), k_kind="video", k_max_pos=(14, 49, 51),
        full_heads=32, world_sizes=(2, 4, 8)),
    "cross_24576x1000": Workload(
        name="cross_24576x1000", seed=1004, B=1, heads=4, head_dim=64,
        nq=24576, nk_pad=1024, nk_valid=1000, q_grid=(12, 32, 64), q_extra=0,
        q_max_pos=(12, 32, 64), k_kind="audio", k_max_pos=(1000,),
        full_heads=32, world_sizes=(8,)),
    "connector_1024": Workload(
        name="connector_1024", seed=1005, B=2, heads=32, head_dim=128,
        nq=1024, nk_pad=1024, nk_valid=1024, q_grid=(1, 1, 1024), q_extra=0,
        q_max_pos=(1024,), k_kind="text", k_max_pos=(1024,),
        full_heads=32, world_sizes=(1,), q_kind="text"),
    "connector_1024_masked": Workload(
        name="connector_1024_masked", seed=1006, B=1, heads=32, head_dim=128,
        nq=1024, nk_pad=1024, nk_valid=700, q_grid=(1, 1, 1024), q_extra=0,
        q_max_pos=(1024,), k_kind="text", k_max_pos=(1024,),
        full_heads=32, world_sizes=(1,), q_kind="text"),
}


def video_positions(grid, extra: int = 0, n_total: Optional[int] = None) -> np.ndarray:
    """Integer (t, x, y) positions in raster order, ``int32 [n_total, 3]``.

    ``extra`` tokens continue the raster on the plane ``t = T`` (one past the
    grid).  Rows beyond the valid tokens (padding) are all zero.
    """
    T, X, Y = grid
    n_valid = T * X * Y + extra
    if extra > X * Y:
        raise ValueError("extra tokens must fit on one plane")
    n_total = n_valid if n_total is None else n_total
    if n_total < n_valid:
        raise ValueError("n_total smaller than the number of valid tokens")
    t, x, y = np.meshgrid(np.arange(T + 1), np.arange(X), np.arange(Y), indexing="ij")
    allpos = np.stack([t.ravel(), x.ravel(), y.ravel()], axis=1)
    out = np.zeros((n_total, 3), dtype=np.int32)
    out[:n_valid] = allpos[:n_valid]
    return out


def audio_positions(n_valid: int, n_total: Optional[int] = None) -> np.ndarray:
    """1-axis time positions ``0 .. n_valid-1``, ``int32 [n_total, 1]``;
    padded rows are zero."""
    n_total = n_valid if n_total is None else n_total
    out = np.zeros((n_total, 1), dtype=np.int32)
    out[:n_valid, 0] = np.arange(n_valid, dtype=np.int32)
    return out


def positions(w: Workload):
    """``(q_pos, k_pos)`` for a workload, covering ``nq`` / ``nk_pad`` rows."""
    if w.q_kind == "text":
        # Every slot of the text sequence has its index as position (the
        # connector rotates by arange over the sequence, padding included).
        q_pos = audio_positions(w.nq, w.nq)
        return q_pos, audio_positions(w.nk_pad, w.nk_pad)
    q_pos = video_positions(w.q_grid, w.q_extra, w.nq)
    if w.k_kind == "video":
        k_pos = video_positions(w.q_grid, w.q_extra, w.nk_pad)
    else:
        k_pos = audio_positions(w.nk_valid, w.nk_pad)
    return q_pos, k_pos


def randn_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    """N(0, 1) float32 draws rounded to bfloat16, on the CPU."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def qkv(w: Workload, heads: Optional[int] = None, seed_offset: int = 0):
    """Draw ``(q, k, v)`` bfloat16 CPU tensors for workload ``w``.

    Shapes: q ``[B, nq, heads, D]``, k and v ``[B, nk_pad, heads, D]``;
    ``heads`` defaults to the workload's per-call head count.
    """
    h = w.heads if heads is None else heads
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + seed_offset)
    q = randn_bf16((w.B, w.nq, h, w.head_dim), g)
    k = randn_bf16((w.B, w.nk_pad, h, w.head_dim), g)
    v = randn_bf16((w.B, w.nk_pad, h, w.head_dim), g)
    return q, k, v


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bfloat16/float tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_rows(n_valid: int, seed: int, n_head: int = 128, n_tail: int = 256,
                n_random: int = 512) -> np.ndarray:
    """Query-row sample for large comparisons: the first ``n_head`` rows, the
    last ``n_tail`` valid rows and ``n_random`` seeded random rows (sorted,
    unique)."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(n_head, n_valid))
    tail = np.arange(max(0, n_valid - n_tail), n_valid)
    rand = rng.integers(0, n_valid, size=n_random)
    return np.unique(np.concatenate([head, tail, rand])).astype(np.int64)

"""Oracle for the rotary position embedding on Q and K.
Test infrastructure only.

Source: FastVideo API page ``fastvideo.models.encoders.gemma``:
* ``LTXRopeType`` -- two pairings exist; the INTERLEAVED one rotates the
  channel pairs (2i, 2i+1).
* ``precompute_ltx_freqs_cis(indices_grid, dim, out_dtype, theta=10000.0,
  max_pos=..., ...)`` -- cos/sin grids for (t, x, y) positions, normalised by
  a per-axis ``max_pos``, with base ``theta``; an fp64 grid variant exists.
* ``apply_ltx_rotary_emb(x, (cos, sin), INTERLEAVED)`` -- applies the grids.

The page prints signatures only, so the following readings are taken
(parity with upstream LTX-2 numerics is *unpinned*):

* Schedule.  With ``A`` position axes and ``D/2`` channel pairs, each axis gets
  ``n_ax = floor((D/2)/A)`` consecutive pairs, in axis order (t, x, y).  Pair
  ``i = a*n_ax + k`` (``0 <= k < n_ax``) turns by
  ``phi = (pos[a] / max_pos[a]) * theta ** (-k / n_ax)``.
  The ``(D/2) mod A`` highest pairs are left unrotated (``phi = 0``).
* Rotation.  ``(x0 + i*x1) * exp(i*phi)``: ``y0 = x0 cos - x1 sin``,
  ``y1 = x0 sin + x1 cos``.
* Every head uses the same angles (the grid spans one head's channels).
* Arithmetic in float64 throughout, no intermediate rounding.

Variants (same page; ``precompute_ltx_freqs_cis`` takes ``dim``,
``num_attention_heads``, ``use_middle_indices_grid`` and ``rope_type``, and the
connector passes ``dim = inner_dim = heads * head_dim``; a float64 grid
generator exists beside the float32 one):

* SPLIT pairing (``LTXRopeType``'s second variant).  Reading: pair ``i`` is
  channels ``(i, i + D/2)`` of the head (first half, second half) instead of
  ``(2i, 2i+1)``; the rotation of a pair is unchanged.
* Grid over the inner dimension.  Reading: the schedule above is laid over
  ``G * D`` channels (``G * D / 2`` pairs, ``n_ax = floor((G*D/2)/A)``) and
  head ``h`` of the ``G`` takes global pairs ``[h*D/2, (h+1)*D/2)``, so heads
  turn at different frequencies.  ``G = 1`` is the per-head grid.
* Middle indices.  Reading: integer positions index unit cells and the angle
  uses the cell's middle, ``pos + 1/2``.
* Float64 grid.  A precision choice only: the oracle is float64 throughout,
  so it has no separate function.
"""

import numpy as np


def _schedule(pos: np.ndarray, max_pos, n_pairs: int, theta: float, middle: bool) -> np.ndarray:
    """Angles of all ``n_pairs`` pairs of one grid: ``n_ax = floor(n_pairs/A)``
    pairs per axis in axis order; pair ``a*n_ax + k`` turns by
    ``(pos[a] (+ 1/2) / max_pos[a]) * theta**(-k/n_ax)``; the rest stay at 0."""
    pos = np.asarray(pos)
    if pos.ndim != 2:
        raise ValueError("pos must be [N, A]")
    N, A = pos.shape
    max_pos = [float(m) for m in max_pos]
    if len(max_pos) != A or any(m <= 0 for m in max_pos):
        raise ValueError("max_pos needs one positive entry per axis")
    n_ax = n_pairs // A
    if n_ax < 1:
        raise ValueError("fewer channel pairs than axes")
    phi = np.zeros((N, n_pairs), dtype=np.float64)
    for a in range(A):
        p = pos[:, a].astype(np.float64) + (0.5 if middle else 0.0)
        frac = p / max_pos[a]
        for k in range(n_ax):
            phi[:, a * n_ax + k] = frac * (float(theta) ** (-k / n_ax))
    return phi


def rope_angles(pos: np.ndarray, max_pos, head_dim: int, theta: float, *, grid_heads: int = 1,
                head: int = 0, middle: bool = False) -> np.ndarray:
    """Angles ``phi[n, i]`` (float64) for integer positions ``pos[n, a]``.

    ``pos`` has shape ``[N, A]``; ``max_pos`` has ``A`` positive entries.
    The schedule spans ``grid_heads * head_dim`` channels and the angles of
    head ``head`` are returned (``grid_heads = 1``: the per-head grid).
    ``middle`` uses ``pos + 1/2``.  Returns ``[N, head_dim // 2]``.
    """
    if head_dim % 2 != 0:
        raise ValueError("head_dim must be even")
    if grid_heads < 1 or not 0 <= head < grid_heads:
        raise ValueError("head must lie in [0, grid_heads)")
    hp = head_dim // 2
    phi = _schedule(pos, max_pos, grid_heads * hp, theta, middle)
    return phi[:, head * hp:(head + 1) * hp]


def rope_apply(x: np.ndarray, pos: np.ndarray, max_pos, theta: float, *,
               rope_type: str = "interleaved", grid_heads: int = 0, head_offset: int = 0,
               middle: bool = False) -> np.ndarray:
    """Rotate ``x[B, N, H, D]`` (float64) by the angles of ``pos[N, A]``.

    Returns a new float64 array.  ``rope_type`` "interleaved": channels
    (2i, 2i+1) form pair ``i``; "split": channels (i, i + D/2) do.
    ``grid_heads = 0``: every head uses the per-head grid; ``grid_heads = G``:
    head ``j`` of ``x`` is head ``head_offset + j`` of a grid over ``G`` heads.
    """
    B, N, H, D = x.shape
    if pos.shape[0] != N:
        raise ValueError("one position row per token is required")
    if rope_type not in ("interleaved", "split"):
        raise ValueError("rope_type must be 'interleaved' or 'split'")
    if grid_heads == 0:
        phi = rope_angles(pos, max_pos, D, theta, middle=middle)            # [N, D/2]
        phi = np.broadcast_to(phi[:, None, :], (N, H, D // 2))
    else:
        if head_offset < 0 or head_offset + H > grid_heads:
            raise ValueError("the tensor's heads must lie inside the grid's heads")
        if D % 2 != 0:
            raise ValueError("head_dim must be even")
        hp = D // 2
        wide = _schedule(pos, max_pos, grid_heads * hp, theta, middle)     # [N, G*D/2]
        phi = wide.reshape(N, grid_heads, hp)[:, head_offset:head_offset + H]
    c = np.cos(phi)[None]                                                   # [1, N, H, D/2]
    s = np.sin(phi)[None]
    if rope_type == "interleaved":
        i0, i1 = slice(0, D, 2), slice(1, D, 2)
    else:
        i0, i1 = slice(0, D // 2), slice(D // 2, D)
    x0 = x[..., i0]
    x1 = x[..., i1]
    y = np.empty_like(x, dtype=np.float64)
    y[..., i0] = x0 * c - x1 * s
    y[..., i1] = x0 * s + x1 * c
    return y

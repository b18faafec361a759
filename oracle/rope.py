"""Oracle for the interleaved rotary position embedding on Q and K.
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
"""

import numpy as np


def rope_angles(pos: np.ndarray, max_pos, head_dim: int, theta: float) -> np.ndarray:
    """Angles ``phi[n, i]`` (float64) for integer positions ``pos[n, a]``.

    ``pos`` has shape ``[N, A]``; ``max_pos`` has ``A`` positive entries.
    Returns ``[N, head_dim // 2]``.
    """
    pos = np.asarray(pos)
    if pos.ndim != 2:
        raise ValueError("pos must be [N, A]")
    N, A = pos.shape
    max_pos = [float(m) for m in max_pos]
    if len(max_pos) != A or any(m <= 0 for m in max_pos):
        raise ValueError("max_pos needs one positive entry per axis")
    if head_dim % 2 != 0:
        raise ValueError("head_dim must be even")
    n_pairs = head_dim // 2
    n_ax = n_pairs // A
    if n_ax < 1:
        raise ValueError("fewer channel pairs than axes")
    phi = np.zeros((N, n_pairs), dtype=np.float64)
    for a in range(A):
        frac = pos[:, a].astype(np.float64) / max_pos[a]
        for k in range(n_ax):
            phi[:, a * n_ax + k] = frac * (float(theta) ** (-k / n_ax))
    return phi


def rope_apply(x: np.ndarray, pos: np.ndarray, max_pos, theta: float) -> np.ndarray:
    """Rotate ``x[B, N, H, D]`` (float64) by the angles of ``pos[N, A]``.

    Returns a new float64 array.  Channels (2i, 2i+1) form pair ``i``.
    """
    B, N, H, D = x.shape
    if pos.shape[0] != N:
        raise ValueError("one position row per token is required")
    phi = rope_angles(pos, max_pos, D, theta)          # [N, D/2]
    c = np.cos(phi)[None, :, None, :]
    s = np.sin(phi)[None, :, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x, dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y

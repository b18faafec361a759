"""Oracle for key-padding-masked scaled-dot-product attention, per head.
Test infrastructure only.

Source: LTX-2 "Sequence Parallelism (SP)" page.
* "What it is": each rank runs ordinary (global over all tokens) attention for
  its heads; SP changes only the floating-point reduction order.
* "How the forward pass works", step 1: padded keys are masked out and padded
  query rows are discarded.
The additive-mask convention of the FastVideo connector page
(``_convert_to_additive_mask``: masked entries get ``-finfo.max``) excludes a
key from the softmax; for padding at the end of the sequence that is the same
as summing over the first ``nk_valid`` keys only, which is the reading used.

Definition (per batch ``b``, head ``h``, query row ``i``):
    s_ij   = scale * sum_d q[i, d] * k[j, d]           for j < nk_valid
    O[i,:] = sum_j exp(s_ij - m_i) v[j, :] / sum_j exp(s_ij - m_i),
    m_i    = max_j s_ij
    lse_i  = m_i + log(sum_j exp(s_ij - m_i))

Float64 throughout.  Rows are independent, so they are evaluated in blocks of
``ROW_BLOCK`` to bound memory; that changes no arithmetic within a row.
"""

import numpy as np

ROW_BLOCK = 1024


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, nk_valid: int,
              scale: float, rows=None):
    """Masked attention.

    q: ``[B, Nq, H, D]``, k and v: ``[B, Nk, H, D]`` (float64; widened by the
    caller).  Keys ``j >= nk_valid`` are excluded.  ``rows`` optionally selects
    a subset of query rows (1-D int array); the result then has ``len(rows)``
    rows in that order.

    Returns ``(o, lse)`` with ``o``: ``[B, R, H, D]`` and ``lse``: ``[B, H, R]``.
    """
    B, Nq, H, D = q.shape
    Bk, Nk, Hk, Dk = k.shape
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if not 1 <= nk_valid <= Nk:
        raise ValueError("nk_valid must be in [1, Nk]")
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    o = np.empty((B, R, H, D), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            K = np.ascontiguousarray(k[b, :nk_valid, h, :], dtype=np.float64)
            V = np.ascontiguousarray(v[b, :nk_valid, h, :], dtype=np.float64)
            for r0 in range(0, R, ROW_BLOCK):
                sel = row_idx[r0:r0 + ROW_BLOCK]
                Q = np.ascontiguousarray(q[b, sel, h, :], dtype=np.float64)
                S = scale * (Q @ K.T)                       # [r, nk_valid]
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                denom = E.sum(axis=1, keepdims=True)
                o[b, r0:r0 + len(sel), h, :] = (E @ V) / denom
                lse[b, h, r0:r0 + len(sel)] = (m + np.log(denom))[:, 0]
    return o, lse

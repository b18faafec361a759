"""Oracle for the whole per-layer sequence-parallel attention path.
Test infrastructure only.

Source: LTX-2 "Sequence Parallelism (SP)" page, "How the forward pass works"
(pad -> shard -> exchange heads -> global attention -> shuffle back -> gather
-> unpad) and "What it is" (numerically equivalent to single-GPU attention).

Two definitions are given so that their agreement can be checked:
* :func:`sp_path_single_gpu` -- rotary on Q/K, then attention over all heads
  and all valid keys, with no exchange at all.
* :func:`sp_path_virtual_ranks` -- the page's steps over ``P`` ranks held in
  one process: pad to a multiple of ``P``, hand rank ``p`` its head block of
  every token (:func:`sp_pack`), let each rank rotate and attend on its heads,
  shuffle back (:func:`sp_unpack`) and drop the padded rows.

Both take ``q, k, v`` as ``[B, N, H, D]`` float64 with ``N`` valid tokens and
integer positions ``[N, A]``; ``k``/``v`` may have a different token count
(cross-attention).  Video self-attention pads the key axis along with the
queries (the page's step 1), so padded keys are masked by ``nk_valid``.
"""

import numpy as np

from .attn import attention
from .perm import pad_length, sp_pack, sp_unpack
from .rope import rope_apply


def sp_path_single_gpu(q, k, v, q_pos, k_pos, q_max_pos, k_max_pos, theta, scale):
    """Single-GPU definition: ``attention(rope(q), rope(k), v)`` over all heads."""
    qr = rope_apply(q, q_pos, q_max_pos, theta)
    kr = rope_apply(k, k_pos, k_max_pos, theta)
    o, _ = attention(qr, kr, v, k.shape[1], scale)
    return o


def sp_path_virtual_ranks(q, k, v, q_pos, k_pos, q_max_pos, k_max_pos, theta, scale,
                          world_size, pad_value=0.0):
    """Sequence-parallel definition over ``world_size`` ranks in one process.

    Query and key token axes are each padded up to a multiple of
    ``world_size`` with rows of ``pad_value`` at position 0; padded keys are
    masked by ``nk_valid`` and padded query rows are dropped at the end.
    """
    P = world_size
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    nq_pad, nk_pad = pad_length(Nq, P), pad_length(Nk, P)

    def pad_tokens(x, n_pad):
        out = np.full((x.shape[0], n_pad) + x.shape[2:], pad_value, dtype=np.float64)
        out[:, :x.shape[1]] = x
        return out

    def pad_pos(p, n_pad):
        out = np.zeros((n_pad, p.shape[1]), dtype=p.dtype)
        out[:p.shape[0]] = p
        return out

    qp, kp, vp = pad_tokens(q, nq_pad), pad_tokens(k, nk_pad), pad_tokens(v, nk_pad)
    qpos, kpos = pad_pos(q_pos, nq_pad), pad_pos(k_pos, nk_pad)
    qs, ks, vs = sp_pack(qp, P), sp_pack(kp, P), sp_pack(vp, P)
    outs = np.empty_like(qs)
    for p in range(P):
        qr = rope_apply(qs[p], qpos, q_max_pos, theta)
        kr = rope_apply(ks[p], kpos, k_max_pos, theta)
        outs[p], _ = attention(qr, kr, vs[p], Nk, scale)
    return sp_unpack(outs)[:, :Nq]

"""GPU checks of the fused entry points.

* ``ltxa_sp_pack_rope`` must equal, bit for bit, ``ltxa_sp_pack`` followed
  by ``ltxa_rope_qk`` on the packed tensor (the rotation acts per token and
  pair, so it commutes with the head exchange of the LTX-2 SP page, "What it
  is"), and must sit within the rotary bar of the oracle's
  ``rope_apply`` + ``sp_pack``.
* ``ltxa_attn_fwd_unpack`` must equal, bit for bit, ``ltxa_attn_fwd`` over
  the shards followed by ``ltxa_sp_unpack`` (only the output addressing
  differs), with identical log-sum-exp values.
"""

import numpy as np
import pytest
import torch

import oracle
from parity import bits, f64, rope_ok
from video_dit_sequence_amd import ltxa
from video_dit_sequence_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (workload, heads of the token-major tensor, ranks, which tensor)
PACK_ROPE_CASES = [
    ("tiny_231", 4, 4, "q"),           # D=64, 3 axes: 2 leftover pairs
    ("tiny_231", 4, 1, "k"),           # one rank: a plain rotation
    ("tiny_231", 6, 2, "q"),           # 3 heads per rank
    ("cross_24576x1000", 32, 8, "q"),  # video queries, D=64
    ("cross_24576x1000", 32, 8, "k"),  # audio keys, 1 axis, ragged 1000 of 1024
    ("share_32768", 32, 8, "q"),       # the timed configuration, D=128
    ("connector_1024", 32, 8, "k"),    # batch 2, 1-axis text positions, rows split over grid y
]


@pytest.mark.parametrize("name,heads,P,which", PACK_ROPE_CASES)
def test_pack_rope_equals_pack_then_rope(name, heads, P, which):
    w = wl.WORKLOADS[name]
    print(f"pack_rope {name} H={heads} P={P} {which}", flush=True)
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, kpos = wl.positions(w)
    x, pos, max_pos = (q, qpos, w.q_max_pos) if which == "q" else (k, kpos, w.k_max_pos)
    xg, pg = x.to(DEV), torch.from_numpy(pos).to(DEV)
    B, N, H, D = x.shape

    fused = ltxa.sp_pack_rope(xg, pg, max_pos, P, w.theta)
    two = ltxa.sp_pack(xg, P)
    ltxa.rope_qk(two.view(P * B, N, H // P, D), pg, max_pos, None, None, None, w.theta)
    torch.cuda.synchronize()
    assert fused.shape == (P, B, N, H // P, D)
    assert np.array_equal(bits(fused), bits(two))
    assert np.array_equal(bits(xg), bits(x)), "the source must be left as it was"

    if N * H * D <= 32 * 1024 * 1024:
        x64 = f64(x)
        ref = oracle.sp_pack(oracle.rope_apply(x64, pos, max_pos, w.theta), P)
        ok, exact = rope_ok(f64(fused), ref, oracle.sp_pack(x64, P))
        assert ok.all(), f"{np.count_nonzero(~ok)} outputs off"
        assert exact > 0.995


# (workload, heads of the token-major tensor, ranks)
ATTN_UNPACK_CASES = [
    ("tiny_231", 4, 4),
    ("tiny_231", 2, 1),
    ("tiny_231", 6, 2),                # 3 heads per rank
    ("cross_24576x1000", 32, 8),
    ("full_6144", 32, 8),
    ("connector_1024", 32, 8),         # batch 2: shard entry p * B + b lands in batch b
]


@pytest.mark.parametrize("name,heads,P", ATTN_UNPACK_CASES)
def test_attn_unpack_equals_attn_then_unpack(name, heads, P):
    w = wl.WORKLOADS[name]
    print(f"attn_unpack {name} H={heads} P={P}", flush=True)
    q, k, v = wl.qkv(w, heads=heads)
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    Hl = H // P
    qs, ks, vs = (ltxa.sp_pack(t.to(DEV), P) for t in (q, k, v))

    lse_f = torch.empty((P, B, Hl, Nq), dtype=torch.float32, device=DEV)
    fused = ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, scale=w.scale, lse=lse_f)
    lse_u = torch.empty((P * B, Hl, Nq), dtype=torch.float32, device=DEV)
    o = ltxa.attn_fwd(qs.view(P * B, Nq, Hl, D), ks.view(P * B, Nk, Hl, D), vs.view(P * B, Nk, Hl, D),
                      nk_valid=w.nk_valid, scale=w.scale, lse=lse_u)
    two = ltxa.sp_unpack(o.view(P, B, Nq, Hl, D))
    torch.cuda.synchronize()
    assert fused.shape == (B, Nq, H, D)
    assert np.array_equal(bits(fused), bits(two))
    assert np.array_equal(lse_f.view(-1).cpu().numpy().view(np.uint32),
                          lse_u.view(-1).cpu().numpy().view(np.uint32))


def test_fused_and_unfused_paths_agree_bitwise():
    w = wl.WORKLOADS["ragged_32761"]
    print("fused vs unfused path ragged_32761 P=8", flush=True)
    q, k, v = (t.to(DEV) for t in wl.qkv(w))
    qpos, _ = wl.positions(w)
    pg = torch.from_numpy(qpos).to(DEV)
    share = ltxa.SpShare(max_tokens=32768, num_heads=32, head_dim=128, world_size=8)
    share.set_seqlen(w.nq_valid)
    # The result is a view of the share's output buffer: copy it before the
    # second call overwrites that buffer.
    a = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, fused=True).clone()
    b = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, fused=False)
    torch.cuda.synchronize()
    assert a.shape == b.shape == (1, w.nq_valid, 32, 128)
    assert np.array_equal(bits(a), bits(b))

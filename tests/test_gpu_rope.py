"""GPU parity of ltxa_rope_qk against the fp64 oracle.

Source: FastVideo gemma page (LTXRopeType INTERLEAVED, precompute_ltx_freqs_cis,
apply_ltx_rotary_emb).  Bar: each output is within one bf16 ulp of the exact
rotation, or within 2^-20 * (|x0| + |x1|) of it where the result is tiny
through cancellation (the fp32 evaluation bound).
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


def _rope_case(w, heads=None, which="qk"):
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, kpos = wl.positions(w)
    qg, kg = q.to(DEV), k.to(DEV)
    qp, kp = torch.from_numpy(qpos).to(DEV), torch.from_numpy(kpos).to(DEV)
    ltxa.rope_qk(qg if "q" in which else None, qp, w.q_max_pos,
                 kg if "k" in which else None, kp, w.k_max_pos, w.theta)
    torch.cuda.synchronize()
    out = {}
    if "q" in which:
        out["q"] = (f64(qg), oracle.rope_apply(f64(q), qpos, w.q_max_pos, w.theta), f64(q))
    else:
        assert np.array_equal(bits(qg), bits(q))
    if "k" in which:
        out["k"] = (f64(kg), oracle.rope_apply(f64(k), kpos, w.k_max_pos, w.theta), f64(k))
    else:
        assert np.array_equal(bits(kg), bits(k))
    return out


@pytest.mark.parametrize("name", ["tiny_231", "full_6144", "cross_24576x1000", "share_32768"])
def test_rope_matches_oracle(name):
    w = wl.WORKLOADS[name]
    print(f"rope {name}", flush=True)
    for key, (got, ref, x) in _rope_case(w).items():
        ok, exact = rope_ok(got, ref, x)
        assert ok.all(), f"{name}/{key}: {np.count_nonzero(~ok)} outputs off"
        assert exact > 0.995, f"{name}/{key}: only {exact:.4f} equal the rounded exact value"


@pytest.mark.parametrize("name,heads", [("tiny_231", 2), ("share_32768", 4)])
def test_shared_positions_rotate_q_and_k_in_one_launch(name, heads):
    # Q and K given with the same position buffer, token count and extents
    # (self-attention) are rotated by one launch that computes each angle
    # once: the bits must be those of two separate calls, and K must meet the
    # oracle bar as Q does.
    w = wl.WORKLOADS[name]
    print(f"rope shared positions {name}", flush=True)
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, _ = wl.positions(w)
    pos = torch.from_numpy(qpos).to(DEV)
    q1, k1 = q.to(DEV), k.to(DEV)
    ltxa.rope_qk(q1, pos, w.q_max_pos, k1, pos, w.q_max_pos, w.theta)
    q2, k2 = q.to(DEV), k.to(DEV)
    ltxa.rope_qk(q2, pos, w.q_max_pos, None, None, None, w.theta)
    ltxa.rope_qk(None, None, None, k2, pos, w.q_max_pos, w.theta)
    torch.cuda.synchronize()
    assert np.array_equal(bits(q1), bits(q2))
    assert np.array_equal(bits(k1), bits(k2))
    for got, x in ((q1, q), (k1, k)):
        ok, exact = rope_ok(f64(got), oracle.rope_apply(f64(x), qpos, w.q_max_pos, w.theta), f64(x))
        assert ok.all() and exact > 0.995


@pytest.mark.parametrize("which", ["q", "k"])
def test_rope_one_tensor_only(which):
    w = wl.WORKLOADS["tiny_231"]
    for key, (got, ref, x) in _rope_case(w, which=which).items():
        ok, _ = rope_ok(got, ref, x)
        assert ok.all()


def test_leftover_pairs_and_pad_tokens_untouched():
    # head_dim 128 over 3 axes leaves pair 63 unrotated; padded tokens sit at
    # position 0 and are not rotated at all.
    w = wl.WORKLOADS["tiny_231"]
    q, k, _ = wl.qkv(w)
    x = torch.cat([q, q], dim=3)  # [1, 232, 2, 128]
    qpos, _ = wl.positions(w)
    xg = x.to(DEV)
    ltxa.rope_qk(xg, torch.from_numpy(qpos).to(DEV), w.q_max_pos, None, None, None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(xg)[..., 126:], bits(x)[..., 126:])
    assert np.array_equal(bits(xg)[:, 231], bits(x)[:, 231])


def test_rope_commutes_with_pack_bit_exact():
    w = wl.WORKLOADS["share_32768"]
    g = torch.Generator().manual_seed(77)
    x = wl.randn_bf16((1, 4096, 32, 128), g).to(DEV)
    pos = torch.from_numpy(wl.video_positions((2, 32, 64))).to(DEV)
    a = x.clone()
    ltxa.rope_qk(a, pos, (2, 32, 64), None, None, None)
    a = ltxa.sp_pack(a, 8)
    b = ltxa.sp_pack(x, 8).view(8, 4096, 4, 128)
    ltxa.rope_qk(b, pos, (2, 32, 64), None, None, None)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b.view(8, 1, 4096, 4, 128)))


def test_rope_rejects_bad_arguments():
    x = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((8, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(ltxa.LtxaError):
        ltxa.rope_qk(x, pos, (1, 0, 1), None, None, None)
    with pytest.raises(ltxa.LtxaError):
        ltxa.rope_qk(x, pos, (1, 1, 1), x, pos, (1, 1, 1))  # q and k alias


@pytest.mark.parametrize("B,H,D,P", [(2, 3, 24, 3), (1, 5, 40, 5), (2, 2, 256, 2), (3, 6, 64, 3)])
def test_odd_shapes_match_oracle_and_pack_fusion(B, H, D, P):
    # Head widths whose 16-byte groups do not divide a wave (24, 40), the
    # widest head (256), batches > 1, and the fused pack on each.
    print(f"rope odd shape B={B} H={H} D={D} P={P}", flush=True)
    g = torch.Generator().manual_seed(1000 + D)
    N = 6 * 7 * 5
    x = wl.randn_bf16((B, N, H, D), g)
    pos = wl.video_positions((6, 7, 5))
    pg = torch.from_numpy(pos).to(DEV)
    xg = x.to(DEV)
    ltxa.rope_qk(xg, pg, (6, 7, 5), None, None, None)
    fused = ltxa.sp_pack_rope(x.to(DEV), pg, (6, 7, 5), P)
    torch.cuda.synchronize()
    ref = oracle.rope_apply(f64(x), pos, (6, 7, 5), 10000.0)
    ok, exact = rope_ok(f64(xg), ref, f64(x))
    assert ok.all(), f"{np.count_nonzero(~ok)} outputs off"
    assert exact > 0.995
    assert np.array_equal(bits(fused), bits(ltxa.sp_pack(xg, P)))

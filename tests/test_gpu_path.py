"""End-to-end GPU parity of the SP attention path (pack -> rotary -> attention
-> unpack -> unpad, all through the C ABI) against the oracle's single-GPU
definition (LTX-2 SP page, "What it is": SP is numerically the single-GPU
result; "How the forward pass works": the steps).

The 32768-token case runs the exact launch configuration that bench.py
times: 32 heads, 8 virtual ranks, one call per step kind over all ranks.
"""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_attn_close, f64
from video_dit_sequence_amd import ltxa
from video_dit_sequence_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _path(q, k, v, qpos, kpos, q_max, k_max, n_valid, nk_valid, P, heads, D):
    share = ltxa.SpShare(max_tokens=32768, num_heads=heads, head_dim=D, world_size=P)
    n_pad = share.set_seqlen(n_valid)
    assert n_pad == q.shape[1]
    o = ltxa.sp_attention(q.to(DEV), k.to(DEV), v.to(DEV), share, torch.from_numpy(qpos).to(DEV), q_max,
                          torch.from_numpy(kpos).to(DEV), k_max, nk_valid=nk_valid)
    torch.cuda.synchronize()
    return o


def _oracle_rows(q, k, v, qpos, kpos, q_max, k_max, nq_valid, nk_valid, theta, scale, rows):
    qr = oracle.rope_apply(f64(q)[:, :nq_valid], qpos[:nq_valid], q_max, theta)
    kr = oracle.rope_apply(f64(k)[:, :nk_valid], kpos[:nk_valid], k_max, theta)
    o, _ = oracle.attention(qr, kr, f64(v)[:, :nk_valid], nk_valid, scale, rows=rows)
    return o


def test_tiny_four_heads_four_ranks():
    w = wl.WORKLOADS["tiny_231"]
    print("path tiny_231 H=4 P=4", flush=True)
    q, k, v = wl.qkv(w, heads=4)
    qpos, kpos = wl.positions(w)
    o = _path(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid, 4, 4, 64)
    assert o.shape == (1, 231, 4, 64)
    n = w.nq_valid
    ref = oracle.sp_path_single_gpu(f64(q)[:, :n], f64(k)[:, :n], f64(v)[:, :n], qpos[:n], kpos[:n],
                                    w.q_max_pos, w.k_max_pos, w.theta, w.scale)
    assert_attn_close(f64(o), ref, "path tiny_231")


def test_share_32768_bench_configuration():
    w = wl.WORKLOADS["share_32768"]
    print("path share_32768 H=32 P=8", flush=True)
    q, k, v = wl.qkv(w, heads=w.full_heads)
    qpos, kpos = wl.positions(w)
    o = _path(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid, 8, 32, 128)
    rows = wl.sample_rows(w.nq_valid, w.seed, n_random=384)
    ref = _oracle_rows(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid,
                       w.theta, w.scale, rows)
    e = assert_attn_close(f64(o)[:, rows], ref, "path share_32768")
    print(e, flush=True)


def test_ragged_32761_eight_ranks():
    w = wl.WORKLOADS["ragged_32761"]
    print("path ragged_32761 H=32 P=8", flush=True)
    q, k, v = wl.qkv(w)
    qpos, kpos = wl.positions(w)
    o = _path(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid, 8, 32, 128)
    assert o.shape == (1, 32761, 32, 128)
    rows = wl.sample_rows(w.nq_valid, w.seed, n_random=128)
    ref = _oracle_rows(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid,
                       w.theta, w.scale, rows)
    assert_attn_close(f64(o)[:, rows], ref, "path ragged_32761")


def test_cross_video_to_audio_eight_ranks():
    w = wl.WORKLOADS["cross_24576x1000"]
    print("path cross_24576x1000 H=32 P=8", flush=True)
    q, k, v = wl.qkv(w, heads=w.full_heads)
    qpos, kpos = wl.positions(w)
    o = _path(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid, 8, 32, 64)
    rows = wl.sample_rows(w.nq_valid, w.seed, n_random=512)
    ref = _oracle_rows(q, k, v, qpos, kpos, w.q_max_pos, w.k_max_pos, w.nq_valid, w.nk_valid,
                       w.theta, w.scale, rows)
    assert_attn_close(f64(o)[:, rows], ref, "path cross_24576x1000")


def test_share_rejects_too_many_tokens():
    share = ltxa.SpShare(max_tokens=32768, num_heads=32, head_dim=128, world_size=8)
    with pytest.raises(ValueError, match="smaller resolution or fewer frames"):
        share.set_seqlen(32769)

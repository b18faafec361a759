"""GPU checks of the fused entry points.

* ``ltxa_sp_pack_rope`` must equal, bit for bit, ``ltxa_sp_pack`` followed
  by ``ltxa_rope_qk`` on the packed tensor (the rotation acts per token and
  pair, so it commutes with the head exchange of the LTX-2 SP page, "What it
  is"), and must sit within the rotary bar of the oracle's
  ``rope_apply`` + ``sp_pack``.
* ``ltxa_attn_fwd_unpack`` must equal, bit for bit, ``ltxa_attn_fwd`` over
  the shards followed by ``ltxa_sp_unpack`` (only the output addressing
  differs), with identical log-sum-exp values.
* Log2-domain queries: ``ltxa_sp_pack_rope_ex`` with ``opts->out_scale`` = 1
  equals ``ltxa_sp_pack_rope`` bit for bit, and with c = scale * log2(e)
  sits within the rotary bar of c times the oracle's rotation (so does the
  in-place ``ltxa_rope_ex``); ``ltxa_attn_fwd_unpack_log2q`` and
  ``ltxa_attn_fwd_log2q`` on q' = bf16(q * c) equal ``ltxa_attn_fwd_unpack``
  and ``ltxa_attn_fwd`` on q bit for bit.
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
    ("connector_1024", 32, 4, "q"),    # 8 heads per rank: two row groups per thread
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
    a = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, fused=True, prescale_q=False).clone()
    b = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, fused=False)
    torch.cuda.synchronize()
    assert a.shape == b.shape == (1, w.nq_valid, 32, 128)
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("name,heads,P,which", PACK_ROPE_CASES)
def test_pack_rope_scaled(name, heads, P, which):
    w = wl.WORKLOADS[name]
    print(f"pack_rope_scaled {name} H={heads} P={P} {which}", flush=True)
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, kpos = wl.positions(w)
    x, pos, max_pos = (q, qpos, w.q_max_pos) if which == "q" else (k, kpos, w.k_max_pos)
    xg, pg = x.to(DEV), torch.from_numpy(pos).to(DEV)
    B, N, H, D = x.shape
    plain = ltxa.sp_pack_rope(xg, pg, max_pos, P, w.theta)
    one = ltxa.sp_pack_rope(xg, pg, max_pos, P, w.theta, out_scale=1.0)
    c = ltxa.log2_domain_scale(w.scale)
    scaled = ltxa.sp_pack_rope(xg, pg, max_pos, P, w.theta, out_scale=c)
    torch.cuda.synchronize()
    assert np.array_equal(bits(one), bits(plain))
    if N * H * D <= 32 * 1024 * 1024:
        x64 = f64(x)
        ref = c * oracle.sp_pack(oracle.rope_apply(x64, pos, max_pos, w.theta), P)
        ok, exact = rope_ok(f64(scaled), ref, c * oracle.sp_pack(x64, P))
        assert ok.all(), f"{np.count_nonzero(~ok)} outputs off"
        assert exact > 0.995


@pytest.mark.parametrize("name,heads,P", ATTN_UNPACK_CASES)
def test_attn_unpack_log2q_equals_kernel_scaled(name, heads, P):
    w = wl.WORKLOADS[name]
    print(f"attn_unpack_log2q {name} H={heads} P={P}", flush=True)
    q, k, v = wl.qkv(w, heads=heads)
    B, Nq, H, D = q.shape
    Hl = H // P
    qs, ks, vs = (ltxa.sp_pack(t.to(DEV), P) for t in (q, k, v))
    c = ltxa.log2_domain_scale(w.scale)
    q2 = (qs.float() * c).to(torch.bfloat16)   # the kernel's own fp32 product, rounded once
    lse_a = torch.empty((P, B, Hl, Nq), dtype=torch.float32, device=DEV)
    lse_b = torch.empty_like(lse_a)
    a = ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, scale=w.scale, lse=lse_a)
    b = ltxa.attn_fwd_unpack(q2, ks, vs, nk_valid=w.nk_valid, lse=lse_b, q_log2=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(lse_a.view(-1).cpu().numpy().view(np.uint32),
                          lse_b.view(-1).cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name,heads,P,amp", [("tiny_231", 4, 4, 1), ("tiny_231", 4, 4, 8),
                                              ("full_6144", 8, 8, 4)])
def test_log2q_path_within_single_rounding_model(name, heads, P, amp):
    """Q rotated and scaled by the rotary pack and used as given by the
    attention: against the exact attention of the exactly rotated q (the
    oracle's fp64 rope_apply) and of K as the kernel rotated it, the path
    meets the error model with q rounded once (tests/parity.py).  amp
    multiplies q by a power of two (exact in bf16) to make the logits steep,
    where q's rounding is the largest term.  The unscaled path, where q is
    rounded by the rotation and again by the attention kernel, is measured
    beside it against the same exact result."""
    from parity import assert_within_model, attn_error_bounds
    w = wl.WORKLOADS[name]
    print(f"log2q path {name} H={heads} P={P} amp={amp}", flush=True)
    q, k, v = wl.qkv(w, heads=heads)
    q = q * amp
    qpos, _ = wl.positions(w)
    B, N, H, D = q.shape
    Hl = H // P
    qg, kg, vg = (t.to(DEV) for t in (q, k, v))
    pg = torch.from_numpy(qpos).to(DEV)
    c = ltxa.log2_domain_scale(w.scale)
    ks = ltxa.sp_pack_rope(kg, pg, w.q_max_pos, P, w.theta)
    vs = ltxa.sp_pack(vg, P)
    qs_l2 = ltxa.sp_pack_rope(qg, pg, w.q_max_pos, P, w.theta, out_scale=c)
    qs = ltxa.sp_pack_rope(qg, pg, w.q_max_pos, P, w.theta)
    lse_l2 = torch.empty((P, B, Hl, N), dtype=torch.float32, device=DEV)
    lse_2r = torch.empty_like(lse_l2)
    o_l2 = ltxa.attn_fwd_unpack(qs_l2, ks, vs, nk_valid=w.nk_valid, lse=lse_l2, q_log2=True)
    o_2r = ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, scale=w.scale, lse=lse_2r)
    k_rot = f64(ltxa.sp_unpack(ks))
    torch.cuda.synchronize()

    rows = (np.arange(w.nq_valid) if N <= 512 else wl.sample_rows(w.nq_valid, w.seed, n_random=192))
    q_exact = oracle.rope_apply(f64(q), qpos, w.q_max_pos, w.theta)
    to_bhn = lambda t: t.permute(1, 0, 2, 3).reshape(B, H, N).cpu().numpy().astype(np.float64)
    r_o, r_l = assert_within_model(f64(o_l2)[:, rows], to_bhn(lse_l2)[:, :, rows], q_exact, k_rot, f64(v),
                                   w.nk_valid, w.scale, rows=rows, what=f"log2q {name} amp={amp}")
    lse_b, o_b, o_ex, lse_ex = attn_error_bounds(q_exact, k_rot, f64(v), w.nk_valid, w.scale, rows=rows)
    r2_o = float(np.max(np.abs(f64(o_2r)[:, rows] - o_ex) / o_b))
    r2_l = float(np.max(np.abs(to_bhn(lse_2r)[:, :, rows] - lse_ex) / lse_b))
    e_l2 = float(np.max(np.abs(to_bhn(lse_l2)[:, :, rows] - lse_ex)))
    e_2r = float(np.max(np.abs(to_bhn(lse_2r)[:, :, rows] - lse_ex)))
    print(f"  worst error/bound (q rounded once): o {r_o:.3f} lse {r_l:.3f}; "
          f"(q rounded twice): o {r2_o:.3f} lse {r2_l:.3f}; max |lse err| {e_l2:.2e} vs {e_2r:.2e}", flush=True)


@pytest.mark.parametrize("name,heads", [("tiny_231", 4), ("connector_1024", 32), ("full_6144", 8)])
def test_attn_log2q_equals_kernel_scaled(name, heads):
    w = wl.WORKLOADS[name]
    print(f"attn_log2q {name} H={heads}", flush=True)
    q, k, v = (t.to(DEV) for t in wl.qkv(w, heads=heads))
    B, Nq, H, _ = q.shape
    c = ltxa.log2_domain_scale(w.scale)
    q2 = (q.float() * c).to(torch.bfloat16)
    lse_a = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    lse_b = torch.empty_like(lse_a)
    a = ltxa.attn_fwd(q, k, v, nk_valid=w.nk_valid, scale=w.scale, lse=lse_a)
    b = ltxa.attn_fwd(q2, k, v, nk_valid=w.nk_valid, lse=lse_b, q_log2=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(lse_a.view(-1).cpu().numpy().view(np.uint32),
                          lse_b.view(-1).cpu().numpy().view(np.uint32))


def test_rope_ex_out_scale():
    # The connector's rotation (grid over the inner dimension of all heads)
    # with an output scale: 1 is bit-identical to no scale; c sits within the
    # rotary bar of c times the oracle's rotation.
    w = wl.WORKLOADS["connector_1024"]
    print("rope_ex out_scale connector_1024", flush=True)
    q, _, _ = wl.qkv(w, heads=w.full_heads)
    pos, _ = wl.positions(w)
    pg = torch.from_numpy(pos).to(DEV)
    B, N, H, D = q.shape
    opts = ltxa.rope_opts(grid_heads=H)
    plain, one, scaled = (q.to(DEV) for _ in range(3))
    ltxa.rope(plain, pg, w.q_max_pos, w.theta, opts=opts)
    ltxa.rope(one, pg, w.q_max_pos, w.theta, opts=opts, out_scale=1.0)
    c = ltxa.log2_domain_scale(w.scale)
    ltxa.rope(scaled, pg, w.q_max_pos, w.theta, opts=opts, out_scale=c)
    torch.cuda.synchronize()
    assert np.array_equal(bits(one), bits(plain))
    x64 = f64(q)
    ref = c * oracle.rope_apply(x64, pos, w.q_max_pos, w.theta, grid_heads=H)
    ok, exact = rope_ok(f64(scaled), ref, c * x64)
    assert ok.all(), f"{np.count_nonzero(~ok)} outputs off"
    assert exact > 0.995


# (rope_type, fp64 angles, cell middles, log2-domain output scale)
TABLE_VARIANTS = [("interleaved", False, False, False), ("interleaved", False, False, True),
                  ("split", True, True, False), ("split", False, False, True),
                  ("interleaved", True, False, True), ("interleaved", False, True, False)]


@pytest.mark.parametrize("B,N,H,D,P", [(2, 40, 6, 96, 2), (1, 48, 6, 96, 3), (1, 45, 9, 48, 3)])
def test_table_pack_general_shapes(B, N, H, D, P):
    # The general form of the table pack: pair groups per row that are not a
    # power of two (head_dim 96 and 48), 3 ranks (no shift for the rank), 2 or
    # 3 heads per rank (no whole group of 4), two batch entries.  One and two
    # tensors per launch against the pack with angles computed in the pass.
    print(f"table pack general B={B} N={N} H={H} D={D} P={P}", flush=True)
    g = torch.Generator().manual_seed(N * H + D)
    x = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16).to(DEV)
    y = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16).to(DEV)
    max_pos = (5.0, 7.0, 9.0)
    pos = torch.stack([torch.randint(0, int(m), (N,), generator=g) for m in max_pos], 1).to(torch.int32).to(DEV)
    for rope_type in ("interleaved", "split"):
        if rope_type == "split" and D % 16:
            continue
        table = ltxa.rope_table(pos, max_pos, D, 10000.0)
        for cq, ck in ((0.0, 0.0), (0.25, 0.0)):
            got_x = ltxa.sp_pack_rope_table(x, table, P, rope_type=rope_type, out_scale=cq)
            got_q, got_k = ltxa.sp_pack_rope_qk_table(x, y, table, P, rope_type=rope_type, q_scale=cq, k_scale=ck)
            want_x = ltxa.sp_pack_rope(x, pos, max_pos, P, 10000.0, opts=ltxa.rope_opts(rope_type=rope_type, out_scale=cq))
            want_y = ltxa.sp_pack_rope(y, pos, max_pos, P, 10000.0, opts=ltxa.rope_opts(rope_type=rope_type, out_scale=ck))
            torch.cuda.synchronize()
            assert np.array_equal(bits(got_x), bits(want_x)), (rope_type, cq)
            assert np.array_equal(bits(got_q), bits(want_x)), (rope_type, cq)
            assert np.array_equal(bits(got_k), bits(want_y)), (rope_type, ck)


@pytest.mark.parametrize("prescale_q", [True, False])
def test_self_attention_table_form_equals_per_tensor_form(prescale_q):
    # sp_attention turns self-attention's Q and K with one angle table in one
    # launch; a K position tensor of its own (equal values) takes the
    # one-call-per-tensor form.  The results agree bit for bit, and so does
    # a table the caller built once and passes in.
    w = wl.WORKLOADS["ragged_32761"]
    print(f"sp_attention table form ragged_32761 P=8 prescale={prescale_q}", flush=True)
    q, k, v = (t.to(DEV) for t in wl.qkv(w))
    qpos, _ = wl.positions(w)
    pg = torch.from_numpy(qpos).to(DEV)
    share = ltxa.SpShare(max_tokens=32768, num_heads=32, head_dim=128, world_size=8)
    share.set_seqlen(w.nq_valid)
    a = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, prescale_q=prescale_q).clone()
    table = ltxa.rope_table(pg, w.q_max_pos, 128, w.theta)
    b = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, prescale_q=prescale_q, q_rope_table=table).clone()
    c = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, k_pos=pg.clone(), prescale_q=prescale_q).clone()
    # A separate K position tensor with the caller's table: the table turns Q alone.
    d = ltxa.sp_attention(q, k, v, share, pg, w.q_max_pos, k_pos=pg.clone(), prescale_q=prescale_q,
                          q_rope_table=table)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(c))
    assert np.array_equal(bits(b), bits(c))
    assert np.array_equal(bits(d), bits(c))


@pytest.mark.parametrize("name,heads,P,which", PACK_ROPE_CASES)
def test_pack_rope_table_equals_pack_rope(name, heads, P, which):
    w = wl.WORKLOADS[name]
    print(f"pack_rope_table {name} H={heads} P={P} {which}", flush=True)
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, kpos = wl.positions(w)
    x, pos, max_pos = (q, qpos, w.q_max_pos) if which == "q" else (k, kpos, w.k_max_pos)
    xg, pg = x.to(DEV), torch.from_numpy(pos).to(DEV)
    D = x.shape[3]
    for rope_type, fp64_angles, middle, scaled in TABLE_VARIANTS:
        if rope_type == "split" and D % 16:
            continue
        c = ltxa.log2_domain_scale(w.scale) if scaled else 0.0
        topts = ltxa.rope_opts(fp64_angles=fp64_angles, middle=middle)
        table = ltxa.rope_table(pg, max_pos, D, w.theta, opts=topts)
        got = ltxa.sp_pack_rope_table(xg, table, P, rope_type=rope_type, out_scale=c)
        opts = ltxa.rope_opts(rope_type=rope_type, fp64_angles=fp64_angles, middle=middle, out_scale=c)
        want = ltxa.sp_pack_rope(xg, pg, max_pos, P, w.theta, opts=opts)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(want)), (rope_type, fp64_angles, middle, scaled)


@pytest.mark.parametrize("name,heads,P,which", PACK_ROPE_CASES)
def test_pack_rope_qk_table_equals_two_table_calls(name, heads, P, which):
    # One launch for Q and K (self-attention: the same positions) equals the
    # two one-tensor calls, each with its own scale.  The second tensor is
    # the first with its heads reversed and negated; a third pass hands the
    # same tensor in as both sources.
    w = wl.WORKLOADS[name]
    print(f"pack_rope_qk_table {name} H={heads} P={P} {which}", flush=True)
    q, k, _ = wl.qkv(w, heads=heads)
    qpos, kpos = wl.positions(w)
    x, pos, max_pos = (q, qpos, w.q_max_pos) if which == "q" else (k, kpos, w.k_max_pos)
    xg, pg = x.to(DEV), torch.from_numpy(pos).to(DEV)
    x2 = (-xg.flip(2)).contiguous()
    D = x.shape[3]
    for rope_type, fp64_angles, middle, scaled in TABLE_VARIANTS:
        if rope_type == "split" and D % 16:
            continue
        c = ltxa.log2_domain_scale(w.scale) if scaled else 0.0
        table = ltxa.rope_table(pg, max_pos, D, w.theta, opts=ltxa.rope_opts(fp64_angles=fp64_angles, middle=middle))
        for second, c2 in ((x2, 0.0), (x2, 0.5), (xg, c)):
            got_q, got_k = ltxa.sp_pack_rope_qk_table(xg, second, table, P, rope_type=rope_type, q_scale=c, k_scale=c2)
            want_q = ltxa.sp_pack_rope_table(xg, table, P, rope_type=rope_type, out_scale=c)
            want_k = ltxa.sp_pack_rope_table(second, table, P, rope_type=rope_type, out_scale=c2)
            torch.cuda.synchronize()
            assert np.array_equal(bits(got_q), bits(want_q)), (rope_type, fp64_angles, middle, scaled, c2)
            assert np.array_equal(bits(got_k), bits(want_k)), (rope_type, fp64_angles, middle, scaled, c2)


@pytest.mark.parametrize("name,which", [("share_32768", "q"), ("tiny_231", "q"), ("cross_24576x1000", "k"),
                                        ("ragged_32761", "q")])
@pytest.mark.parametrize("fp64_angles,middle", [(False, False), (True, False), (False, True)])
def test_rope_table_matches_oracle_angles(name, which, fp64_angles, middle):
    # Pins the table to the oracle's angle schedule (not to another kernel):
    # fp32 angles are within a few fp32 ulps of (cos, sin) of the exact
    # angle; fp64 angles are the exact values rounded to fp32.
    w = wl.WORKLOADS[name]
    print(f"rope_table {name} {which} fp64={fp64_angles} middle={middle}", flush=True)
    qpos, kpos = wl.positions(w)
    pos, max_pos = (qpos, w.q_max_pos) if which == "q" else (kpos, w.k_max_pos)
    D = w.head_dim
    table = ltxa.rope_table(torch.from_numpy(pos).to(DEV), max_pos, D, w.theta,
                            opts=ltxa.rope_opts(fp64_angles=fp64_angles, middle=middle))
    torch.cuda.synchronize()
    phi = oracle.rope_angles(pos, max_pos, D, w.theta, middle=middle)
    want = np.stack([np.cos(phi), np.sin(phi)], axis=-1)
    err = np.max(np.abs(f64(table) - want))
    tol = 2.0 ** -23 if fp64_angles else 2.0 ** -20
    assert err <= tol, f"max |table - (cos, sin)| = {err:.3e}"

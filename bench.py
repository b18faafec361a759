"""Throughput of the sequence-parallel masked rotary attention path on one MI355X.

One step = one layer's SP attention for all 8 virtual ranks of the
32768-token, 32-head, head_dim-128 video workload (``share_32768``): pack Q,
K and V to per-rank head shards, rotate Q/K, attend over all 32768 keys for
every rank's 4 heads, and unpack the output.  Every part is exactly 8x one
rank's share, so the rate equals one rank's.  Inputs are seeded synthetic
bf16 N(0,1) tensors already resident in HBM.

The default path takes four launches (``--path fused``): the (cos, sin)
table of the tokens' positions is built (in a model, once per forward pass
for every layer; here once per step), Q and K are packed and rotated with it
in one launch (the Q half also multiplies by scale * log2(e) before its one
rounding), V is packed, and the attention kernel takes those log2-domain
queries as given and writes its output in token order.  ``--path unfused`` times the six-launch sequence (pack x3,
rotary, attention, unpack), in which the attention kernel scales and
rounds Q itself.

Prints one JSON line.  ``value`` is attention TFLOP/s over the whole step
(4 * Nq * Nk_valid * D * H flop per step).  ``roofline`` covers the dominant
kernel (attn_fwd_kernel<128, 8>, launched by ltxa_attn_fwd_unpack_log2q), timed
with HIP events on its own stream inside the timed region.  ``cpu_baseline`` is the fp64 numpy oracle on a bounded row
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "masked RoPE-attention TFLOP/s and % bf16 MFMA peak at 32K tokens, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WORKLOAD = "share_32768"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_share_32768_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "video_dit_sequence_amd", "csrc", "attn_fwd.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--path", choices=("fused", "unfused"), default="fused")
    ap.add_argument("--secondary", type=int, default=1,
                    help="also time the cross-attention and connector workloads (reported apart)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample (0 skips it)")
    ap.add_argument("--cpu-configs", type=float, default=0.0,
                    help="also time the oracle on the other workloads (6144 tokens, 32761 of 32768, "
                         "cross-attention) and its pack, this many CPU seconds each (0 skips it)")
    ap.add_argument("--inputs", choices=("normal", "zeros"), default="normal",
                    help="diagnostic only: 'zeros' runs the same step on all-zero Q/K/V, which "
                         "shows how far the chip's clock under matrix load depends on the data")
    return ap.parse_args()


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_per_launch():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != source_digest(ATTN_SOURCE):
        return None
    return t.get("hbm_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max((i.get("num_threads", 1) for i in threadpool_info()), default=1))
    except Exception:
        return os.cpu_count()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, qpos, kpos, budget_s):
    """Time the oracle on a bounded sample: blocks of 256 query rows of
    successive heads against all valid keys (rotary on the rows and keys,
    then attention), until the time budget is spent."""
    import numpy as np
    import oracle
    threads = blas_threads()
    f64 = lambda t: t.to(torch.float64).numpy()
    rows_per_block = 256
    flops = 0.0
    done_rows = 0
    heads_used = 0
    t0 = time.perf_counter()
    for h in range(q.shape[2]):
        kh = f64(k[:, :, h:h + 1])
        vh = f64(v[:, :, h:h + 1])
        kr = oracle.rope_apply(kh, kpos, w.k_max_pos, w.theta)
        heads_used += 1
        for r0 in range(0, w.nq, rows_per_block):
            rows = np.arange(r0, min(r0 + rows_per_block, w.nq))
            qr = oracle.rope_apply(f64(q[:, r0:r0 + len(rows), h:h + 1]), qpos[rows],
                                   w.q_max_pos, w.theta)
            oracle.attention(qr, kr, vh, w.nk_valid, w.scale)
            flops += 4.0 * len(rows) * w.nk_valid * w.head_dim
            done_rows += len(rows)
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done_rows} query rows over {heads_used} head(s) x {w.nk_valid} keys, "
                      f"head_dim {w.head_dim}, fp64 numpy (rotary + attention), {dt:.1f} s",
            "host_cpus": os.cpu_count()}


def cpu_oracle_configs(wl, budget_s):
    """The oracle on the other workloads (same sampling as cpu_baseline) and
    the oracle pack of one [1, 32768, 32, 128] bf16 tensor to 8 ranks."""
    import numpy as np
    import oracle
    out = {"cpu_model": cpu_model(), "blas_threads": blas_threads(), "host_cpus": os.cpu_count()}
    for name in ("full_6144", "ragged_32761", "cross_24576x1000"):
        w = wl.WORKLOADS[name]
        q, k, v = wl.qkv(w)
        qpos, kpos = wl.positions(w)
        r = cpu_baseline(w, q, k, v, qpos, kpos, budget_s)
        out[name] = {"value": round(r["value"], 4), "unit": "TFLOP/s", "sample": r["sample"]}
    w = wl.WORKLOADS[WORKLOAD]
    x = wl.qkv(w, heads=w.full_heads)[0].view(torch.int16).numpy()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.sp_pack(x, w.world_sizes[0])
        n += 1
    dt = time.perf_counter() - t0
    out["pack_share_32768_P8"] = {"value": round(2.0 * x.nbytes * n / dt / 1e9, 2), "unit": "GB/s",
                                  "sample": f"{n} packs of {x.nbytes} bytes, numpy transpose copy, {dt:.1f} s"}
    return out


def secondary(ltxa, wl, dev, iters):
    """Time the other instantiations of the path (not part of ``value``):
    video->audio cross-attention for all 8 ranks of the 32-head share (fused
    pack+rotary of the video Q and audio K, pack of V, attention into token
    order), and the 1D text connector's attention core (rotary over the
    inner dimension on Q and K, then attention over all 32 heads)."""
    out = {}
    ev = lambda: torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        # These launches are short: run them back to back for ~100 ms first,
        # so that the core clock has settled under the load (right after
        # idle it starts lower), and time at least `iters` launches and 50 ms.
        a, b = ev(), ev()
        fn()
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        one = max(a.elapsed_time(b), 1e-3)
        for _ in range(int(100.0 / one) + 3):
            fn()
        n = max(iters, int(50.0 / one))
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    w = wl.WORKLOADS["cross_24576x1000"]
    P, H = w.world_sizes[0], w.full_heads
    q, k, v = (t.to(dev) for t in wl.qkv(w, heads=H))
    qp, kp = (torch.from_numpy(p).to(dev) for p in wl.positions(w))
    qs = torch.empty((P, w.B, w.nq, H // P, w.head_dim), dtype=torch.bfloat16, device=dev)
    ks = torch.empty((P, w.B, w.nk_pad, H // P, w.head_dim), dtype=torch.bfloat16, device=dev)
    vs, o = torch.empty_like(ks), torch.empty_like(q)

    c = ltxa.log2_domain_scale(w.scale)

    def cross():
        ltxa.sp_pack_rope(q, qp, w.q_max_pos, P, w.theta, out=qs, out_scale=c)
        ltxa.sp_pack_rope(k, kp, w.k_max_pos, P, w.theta, out=ks)
        ltxa.sp_pack(v, P, out=vs)
        ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, out=o, q_log2=True)

    def cross_attn_only():
        ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, out=o, q_log2=True)

    flop = 4.0 * w.nq * w.nk_valid * w.head_dim * H * w.B
    ms, ams = timed(cross), timed(cross_attn_only)
    out["cross_24576x1000"] = {"ms_per_step": round(ms, 4), "attn_ms": round(ams, 4),
                               "attn_tflops": round(flop / (ams * 1e-3) / 1e12, 1),
                               "attn_frac_bf16_peak": round(flop / (ams * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "flop_per_step": flop, "heads": H, "virtual_ranks": P}
    del q, k, v, qs, ks, vs, o

    w = wl.WORKLOADS["connector_1024"]
    q, k, v = (t.to(dev) for t in wl.qkv(w))
    pos = torch.from_numpy(wl.positions(w)[0]).to(dev)
    o = torch.empty_like(q)
    opts = ltxa.rope_opts(grid_heads=w.heads)

    assert list(w.q_max_pos) == list(w.k_max_pos)  # Q and K turn by the same angles

    def connector():
        ltxa.rope_qk_ex(q, k, pos, w.q_max_pos, w.theta, opts=opts)
        ltxa.attn_fwd(q, k, v, nk_valid=w.nk_valid, out=o)

    def connector_attn_only():
        ltxa.attn_fwd(q, k, v, nk_valid=w.nk_valid, out=o)

    flop = 4.0 * w.nq * w.nk_valid * w.head_dim * w.heads * w.B
    ms, ams = timed(connector), timed(connector_attn_only)
    out["connector_1024"] = {"ms_per_step": round(ms, 4), "attn_ms": round(ams, 4),
                             "attn_tflops": round(flop / (ams * 1e-3) / 1e12, 1),
                             "attn_frac_bf16_peak": round(flop / (ams * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "flop_per_step": flop, "heads": w.heads, "batch": w.B}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    global torch
    import numpy as np
    import torch
    from video_dit_sequence_amd import ltxa
    from video_dit_sequence_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[WORKLOAD]
    P, H, D = w.world_sizes[0], w.full_heads, w.head_dim
    q_cpu, k_cpu, v_cpu = wl.qkv(w, heads=H)             # [1, 32768, 32, 128] each
    qpos, kpos = wl.positions(w)
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    if args.inputs == "zeros":
        for t in (q, k, v):
            t.zero_()
    pos = torch.from_numpy(qpos).to(dev)
    share = ltxa.SpShare(max_tokens=32768, num_heads=H, head_dim=D, world_size=P)
    n_pad = share.set_seqlen(w.nq_valid)
    B, N, Hl = w.B, n_pad, H // P

    # The share's own receive and output buffers (the AttentionManager's),
    # allocated once here and reused by every step.
    buf = share.buffers(B, dev)
    qs, ks, vs, os_, out = buf["q"], buf["k"], buf["v"], buf["o_shards"], buf["out"]
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    if args.path == "fused":
        phase_names = ("rope_table", "pack_rope_qk", "pack_v", "attn_fwd")

        c = ltxa.log2_domain_scale(w.scale)
        # Self-attention: Q and K turn by the same angles.  The step builds
        # their table (in a model, once per forward pass for every layer)
        # and then exchanges and rotates Q and K in one launch.
        assert np.array_equal(qpos, kpos) and list(w.q_max_pos) == list(w.k_max_pos)
        table = share.rope_table_buffer(dev)

        def launches():
            yield ltxa.rope_table(pos, w.q_max_pos, D, w.theta, out=table)
            yield ltxa.sp_pack_rope_qk_table(q, k, table, P, q_scale=c, q_out=qs, k_out=ks)
            yield ltxa.sp_pack(v, P, out=vs)
            yield ltxa.attn_fwd_unpack(qs, ks, vs, nk_valid=w.nk_valid, out=out, q_log2=True)
    else:
        phase_names = ("pack_qkv", "rope_qk", "attn_fwd", "unpack_o")

        def launches():
            ltxa.sp_pack(q, P, out=qs)
            ltxa.sp_pack(k, P, out=ks)
            yield ltxa.sp_pack(v, P, out=vs)
            yield ltxa.rope_qk(qs.view(P * B, N, Hl, D), pos, w.q_max_pos, ks.view(P * B, N, Hl, D),
                               pos, w.k_max_pos, w.theta)
            yield ltxa.attn_fwd(qs.view(P * B, N, Hl, D), ks.view(P * B, N, Hl, D),
                                vs.view(P * B, N, Hl, D), nk_valid=w.nk_valid,
                                out=os_.view(P * B, N, Hl, D))
            yield ltxa.sp_unpack(os_, out=out)

    def step(record=None):
        # One event before the step and one after each phase, all on the
        # stream the kernels are launched on.
        if record is None:
            for _ in launches():
                pass
            return
        marks = [ev()]
        marks[0].record(stream)
        for _ in launches():
            marks.append(ev())
            marks[-1].record(stream)
        record.append(marks)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    records = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(records)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    phases = {name: [] for name in phase_names}
    for m in records:
        for i, name in enumerate(phases):
            phases[name].append(m[i].elapsed_time(m[i + 1]))
    avg = {k_: sum(x) / len(x) for k_, x in phases.items()}

    attn_flop = 4.0 * N * w.nk_valid * D * H            # one launch covers all P ranks' heads
    step_tflops = attn_flop / (ms_per_step * 1e-3) / 1e12
    attn_tflops = attn_flop / (avg["attn_fwd"] * 1e-3) / 1e12
    traffic = traffic_per_launch()
    tensor_bytes = 2.0 * B * N * H * D                  # one bf16 [B, N, H, D] tensor
    table_bytes = 4.0 * N * D                           # fp32 (cos, sin) per token and pair
    phase_bytes = {                                     # algorithmic HBM bytes (read + write)
        "rope_table": N * 3 * 4 + table_bytes,
        "pack_rope_qk": 2 * 2 * tensor_bytes + table_bytes,
        "pack_v": 2 * tensor_bytes,
        "pack_qkv": 3 * 2 * tensor_bytes,
        "rope_qk": 2 * 2 * tensor_bytes + 2 * N * 3 * 4,
        "unpack_o": 2 * tensor_bytes,
    }

    line = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic" if args.inputs == "normal" else "synthetic, all zeros (diagnostic, not a result)",
        "config": {"workload": WORKLOAD, "tokens": N, "valid_tokens": w.nq_valid, "heads": H,
                   "head_dim": D, "virtual_ranks": P, "heads_per_rank": Hl, "batch": B,
                   "grid_txy": list(w.q_grid), "rope_theta": w.theta, "path": args.path,
                   "q_operand": ("log2-domain (the rotary pack multiplies by scale*log2(e) before its one rounding)"
                                 if args.path == "fused" else "scaled and rounded inside the attention kernel")},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_kernel<128, 8>",
                     "flop_per_launch": attn_flop, "avg_launch_ms": round(avg["attn_fwd"], 4)},
        "phases_ms": {k_: round(x, 4) for k_, x in avg.items()},
        "hbm_GBps": {**{k_: round(phase_bytes[k_] / (avg[k_] * 1e-3) / 1e9, 1)
                        for k_ in phase_names if k_ in phase_bytes}, "peak": PEAK_HBM_GBS},
        "device": torch.cuda.get_device_name(0),
    }
    if args.secondary:
        line["secondary"] = secondary(ltxa, wl, dev, 20)
    if args.cpu_seconds > 0 and args.inputs == "normal":
        line["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, qpos, kpos, args.cpu_seconds)
    if args.cpu_configs > 0 and args.inputs == "normal":
        line["cpu_oracle_configs"] = cpu_oracle_configs(wl, args.cpu_configs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

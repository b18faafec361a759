"""Stream and graph behaviour of the C ABI: every entry point enqueues on the
stream it is given and keeps no state between calls, so the fused path runs
the same on a side stream, and a HIP graph captured from it replays the same
bits as eager calls (also after its input buffers are refilled).
"""

import numpy as np
import pytest
import torch

from parity import bits
from video_dit_sequence_amd import ltxa
from video_dit_sequence_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class _Step:
    """Preallocated buffers and the four fused calls of one SP attention step."""

    def __init__(self, name, heads, P):
        self.w = w = wl.WORKLOADS[name]
        self.P = P
        q, k, v = wl.qkv(w, heads=heads)
        qpos, kpos = wl.positions(w)
        self.q, self.k, self.v = q.to(DEV), k.to(DEV), v.to(DEV)
        self.qpos, self.kpos = torch.from_numpy(qpos).to(DEV), torch.from_numpy(kpos).to(DEV)
        B, N, H, D = q.shape
        self.qs = torch.empty((P, B, N, H // P, D), dtype=torch.bfloat16, device=DEV)
        self.ks, self.vs = torch.empty_like(self.qs), torch.empty_like(self.qs)
        self.out = torch.empty_like(self.q)

    def run(self):
        w, P = self.w, self.P
        ltxa.sp_pack_rope(self.q, self.qpos, w.q_max_pos, P, w.theta, out=self.qs)
        ltxa.sp_pack_rope(self.k, self.kpos, w.k_max_pos, P, w.theta, out=self.ks)
        ltxa.sp_pack(self.v, P, out=self.vs)
        ltxa.attn_fwd_unpack(self.qs, self.ks, self.vs, nk_valid=w.nk_valid, scale=w.scale, out=self.out)


def test_fused_step_on_a_side_stream():
    print("streams: fused step on a side stream", flush=True)
    st = _Step("tiny_231", 4, 4)
    st.run()
    torch.cuda.synchronize()
    ref = st.out.clone()
    st.out.zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        st.run()
    side.synchronize()
    assert np.array_equal(bits(st.out), bits(ref))


def test_graph_capture_replays_bit_exact():
    print("streams: graph capture of the fused step", flush=True)
    st = _Step("full_6144", 32, 8)
    st.run()
    torch.cuda.synchronize()
    eager = st.out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for i in range(3):
        st.out.fill_(float("nan"))              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(st.out), bits(eager)), f"replay {i}"

    # Refill the captured input buffers: the replay reads them again.
    q2, k2, v2 = wl.qkv(st.w, heads=32, seed_offset=1)
    st.q.copy_(q2.to(DEV))
    st.k.copy_(k2.to(DEV))
    st.v.copy_(v2.to(DEV))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replayed = st.out.clone()
    st.run()                                    # eager on the same new inputs
    torch.cuda.synchronize()
    assert np.array_equal(bits(replayed), bits(st.out))
    assert not np.array_equal(bits(replayed), bits(eager))


def test_concurrent_steps_on_two_streams():
    # No state is shared between calls: two different steps in flight on two
    # streams at once give the bits each gives alone.
    print("streams: two steps on two streams", flush=True)
    a = _Step("tiny_231", 4, 4)
    b = _Step("full_6144", 32, 8)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a, ref_b = a.out.clone(), b.out.clone()
    a.out.zero_()
    b.out.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            b.run()
        with torch.cuda.stream(s2):
            a.run()
    s1.synchronize()
    s2.synchronize()
    assert np.array_equal(bits(a.out), bits(ref_a))
    assert np.array_equal(bits(b.out), bits(ref_b))

"""The 1D text connector's attention core on the GPU against the oracle.

Source: FastVideo gemma page, ``Embeddings1DConnector.forward``: positions
are ``arange`` over the sequence; ``precompute_ltx_freqs_cis`` gets
``dim = inner_dim`` and ``num_attention_heads``, so the rotary grid spans all
heads; the attention mask is additive with valid entries at >= -9000, and
with learnable registers it is reset to zeros (every slot attends).  A valid
prefix mask is ``nk_valid``.  Bar: the attention bar (max-abs 2e-2,
mean-abs 2e-3, relative RMS 1e-2, cosine 0.9999) over every query row, head
and channel.
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


def _oracle(q, k, v, pos, w, rope_type):
    H = q.shape[2]
    qr = oracle.rope_apply(f64(q), pos, w.q_max_pos, w.theta, rope_type=rope_type, grid_heads=H)
    kr = oracle.rope_apply(f64(k), pos, w.k_max_pos, w.theta, rope_type=rope_type, grid_heads=H)
    o, _ = oracle.attention(qr, kr, f64(v), w.nk_valid, w.scale)
    return o


@pytest.mark.parametrize("name,rope_type,fp64", [
    ("connector_1024", "interleaved", False),
    ("connector_1024", "split", True),
    ("connector_1024_masked", "interleaved", True),
    ("connector_1024_masked", "split", False),
])
def test_connector_attention_matches_oracle(name, rope_type, fp64):
    w = wl.WORKLOADS[name]
    print(f"connector {name} {rope_type} fp64={fp64}", flush=True)
    q, k, v = wl.qkv(w)
    pos, _ = wl.positions(w)
    kg, vg = k.clone(), v.clone()
    if w.nk_valid < w.nk_pad:
        # Masked slots hold garbage that must not reach any output.
        kg[:, w.nk_valid:] = float("nan")
        vg[:, w.nk_valid:] = float("inf")
    o = ltxa.connector_attention(q.to(DEV), kg.to(DEV), vg.to(DEV), torch.from_numpy(pos).to(DEV),
                                 w.q_max_pos, nk_valid=w.nk_valid, theta=w.theta, rope_type=rope_type,
                                 fp64_angles=fp64)
    torch.cuda.synchronize()
    ref = _oracle(q, k, v, pos, w, rope_type)
    e = assert_attn_close(f64(o), ref, name)
    print(e, flush=True)

"""GPU parity of ltxa_sp_pack / ltxa_sp_unpack against the oracle: bit-exact.

Source: LTX-2 SP page, "What it is" (the exchange moves bytes only; the round
trip is byte-exact), "API / AttentionManager" (heads divisible by world_size).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity import bits
from video_dit_sequence_amd import ltxa
from video_dit_sequence_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_pack(src_cpu: torch.Tensor, P: int):
    src = src_cpu.to(DEV)
    packed = ltxa.sp_pack(src, P)
    back = ltxa.sp_unpack(packed)
    torch.cuda.synchronize()
    want = oracle.sp_pack(bits(src_cpu), P)
    assert np.array_equal(bits(packed), want)
    assert np.array_equal(bits(back), bits(src_cpu))


@pytest.mark.parametrize("P", [1, 2])
def test_tiny_two_heads(P):
    w = wl.WORKLOADS["tiny_231"]
    q, _, _ = wl.qkv(w)
    print(f"pack tiny_231 H=2 P={P}", flush=True)
    _check_pack(q, P)


def test_tiny_four_heads_four_ranks():
    w = wl.WORKLOADS["tiny_231"]
    q, _, _ = wl.qkv(w, heads=4)
    _check_pack(q, 4)


def test_two_heads_four_ranks_is_rejected():
    # The tiny workload asks for 4 ranks with 2 heads; heads must divide by
    # world_size, so the C ABI refuses it before launching anything.
    x = torch.zeros((1, 232, 2, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((4, 1, 232, 1, 64), dtype=torch.bfloat16, device=DEV)
    rc = ltxa.lib().ltxa_sp_pack(x.data_ptr(), y.data_ptr(), 1, 232, 2, 64, 4, 2, None)
    assert rc == ltxa.LTXA_E_DIVISIBILITY
    with pytest.raises(ltxa.LtxaError):
        ltxa.sp_pack(x, 4)


def test_every_bf16_bit_pattern_round_trips():
    pat = torch.arange(2 ** 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = pat.reshape(1, 1024, 8, 8).contiguous()
    for P in (2, 4, 8):
        _check_pack(x, P)


def test_share_32768_full_tensor_eight_ranks():
    w = wl.WORKLOADS["share_32768"]
    g = torch.Generator().manual_seed(w.seed)
    x = wl.randn_bf16((1, 32768, 32, 128), g)
    print("pack share_32768 [1,32768,32,128] P=8", flush=True)
    _check_pack(x, 8)


@pytest.mark.parametrize("B,N,H,D,P,dtype", [
    (2, 6, 6, 3, 3, torch.uint8),        # 3-byte head blocks: byte path
    (1, 10, 4, 5, 2, torch.int16),       # 10-byte blocks: 2-byte path
    (3, 4, 8, 3, 4, torch.float32),      # 12-byte blocks: 4-byte path
    (1, 8, 4, 1, 2, torch.float64),      # 16-byte blocks, 8-byte elements
    (2, 12, 12, 16, 3, torch.bfloat16),  # 4 heads per rank, 128-byte blocks
])
def test_generic_widths(B, N, H, D, P, dtype):
    g = torch.Generator().manual_seed(5)
    raw = torch.randint(0, 255, (B, N, H, D * torch.tensor([], dtype=dtype).element_size()),
                        generator=g, dtype=torch.uint8)
    src_cpu = raw.view(dtype).contiguous()
    src = src_cpu.to(DEV)
    packed = ltxa.sp_pack(src, P)
    back = ltxa.sp_unpack(packed)
    torch.cuda.synchronize()
    want = oracle.sp_pack(src_cpu.view(torch.uint8).numpy(), P)
    assert np.array_equal(packed.cpu().view(torch.uint8).numpy(), want)
    assert np.array_equal(back.cpu().view(torch.uint8).numpy(), src_cpu.view(torch.uint8).numpy())


def test_unaligned_views_use_narrow_path():
    # Sub-tensors starting 2 bytes into an allocation: still exact.
    base = torch.arange(2 * 4 * 4 * 8 + 1, dtype=torch.int32).to(torch.int16).to(DEV)
    src = base[1:].view(2, 4, 4, 8)
    out_base = torch.empty(2 * 4 * 4 * 8 + 1, dtype=torch.int16, device=DEV)
    out = out_base[1:].view(2, 2, 4, 2, 8)
    ltxa.sp_pack(src, 2, out=out)
    torch.cuda.synchronize()
    want = oracle.sp_pack(src.cpu().numpy(), 2)
    assert np.array_equal(out.cpu().numpy(), want)


def test_overlapping_buffers_are_rejected():
    x = torch.zeros(1 << 12, dtype=torch.bfloat16, device=DEV)
    rc = ltxa.lib().ltxa_sp_pack(x.data_ptr(), x.data_ptr() + 64, 1, 8, 4, 64, 2, 2, None)
    assert rc == ltxa.LTXA_E_ALIAS

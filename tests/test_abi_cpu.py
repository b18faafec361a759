"""CPU checks of the C ABI: the library loads, exports exactly what
include/ltxa.h declares, and rejects bad arguments with the documented codes
before touching the GPU.  Also the host-side SpShare bookkeeping (LTX-2 SP
page, "API / AttentionManager" and "Usage")."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

from video_dit_sequence_amd import ltxa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ltxa.h")

# Fake, 256-byte aligned device addresses: validation never dereferences them
# and no call below passes validation, so nothing is launched.
A, B, C, D_, E = (0x10000000 * i for i in range(1, 6))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ltxa.LIB_PATH):
        from video_dit_sequence_amd import build
        build.build()
    return ltxa.lib()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(ltxa_\w+)\s*\(", text, re.M)))


def header_constant(name):
    text = open(HEADER).read()
    m = re.search(rf"{name}\s*=?\s*(-?\d+)", text)
    return int(m.group(1))


def test_exports_match_header(L):
    declared = header_functions()
    assert declared == sorted(ltxa.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ltxa.LIB_PATH], capture_output=True, text=True)
    exported = sorted(l.split()[-1] for l in out.stdout.splitlines() if " T ltxa_" in l)
    assert exported == declared


def test_version_and_status_strings(L):
    assert ltxa.version() == header_constant("LTXA_VERSION")
    for code in (ltxa.LTXA_OK, ltxa.LTXA_E_NULL, ltxa.LTXA_E_SHAPE, ltxa.LTXA_E_DIVISIBILITY,
                 ltxa.LTXA_E_ALIGN, ltxa.LTXA_E_ALIAS, ltxa.LTXA_E_HIP, ltxa.LTXA_E_RANGE):
        s = ltxa.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in ltxa.status_string(12345)
    for name, val in (("LTXA_E_NULL", -1), ("LTXA_E_SHAPE", -2), ("LTXA_E_DIVISIBILITY", -3),
                      ("LTXA_E_ALIGN", -4), ("LTXA_E_ALIAS", -5), ("LTXA_E_HIP", -6),
                      ("LTXA_E_RANGE", -7)):
        assert header_constant(name) == val == getattr(ltxa, name)


@pytest.mark.parametrize("fn", ["ltxa_sp_pack", "ltxa_sp_unpack"])
def test_perm_errors(L, fn):
    f = getattr(L, fn)
    assert f(None, B, 1, 8, 4, 64, 2, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, None, 1, 8, 4, 64, 2, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, B, 0, 8, 4, 64, 2, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, 1, 8, 4, 0, 2, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, 1, 8, 4, 64, 0, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, 1, 8, 4, 64, 2, 3, None) == ltxa.LTXA_E_SHAPE
    # heads % world_size (the AttentionManager rule) and tokens % world_size
    # (the sequence is padded to a multiple of world_size first).
    assert f(A, B, 1, 232, 2, 64, 4, 2, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, 1, 231, 4, 64, 4, 2, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, A + 64, 1, 8, 4, 64, 2, 2, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, 1 << 40, 1 << 20, 64, 128, 8, 2, None) == ltxa.LTXA_E_RANGE


def _mp(*vals):
    return (ctypes.c_double * len(vals))(*vals)


def test_rope_errors(L):
    f = L.ltxa_rope_qk
    mp3 = _mp(3, 7, 11)
    ok_q = (A, C, 232, 3, mp3)
    none = (None, None, 0, 0, None)
    assert f(*none, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, None, 232, 3, mp3, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, C, 232, 3, None, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(*ok_q, *none, 0, 2, 64, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(*ok_q, *none, 1, 2, 63, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(*ok_q, *none, 1, 2, 512, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, C, 232, 4, _mp(1, 1, 1, 1), *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, C, 232, 3, _mp(3, 0, 11), *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, C, 232, 3, _mp(3, float("nan"), 11), *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(*ok_q, *none, 1, 2, 64, 0.0, None) == ltxa.LTXA_E_SHAPE
    assert f(*ok_q, *none, 1, 2, 64, float("inf"), None) == ltxa.LTXA_E_SHAPE
    assert f(A, C, 0, 3, mp3, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(*ok_q, *none, 1, 2, 4, 1e4, None) == ltxa.LTXA_E_ALIGN       # 8-byte rows
    assert f(A + 2, C, 232, 3, mp3, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_ALIGN
    assert f(A, C + 4, 232, 3, mp3, *none, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_ALIGN
    assert f(*ok_q, A + 256, C, 232, 3, mp3, 1, 2, 64, 1e4, None) == ltxa.LTXA_E_ALIAS


def test_attn_errors(L):
    f = L.ltxa_attn_fwd
    good = (1, 2, 128, 232, 232, 231, 0.088)
    assert f(None, B, C, D_, None, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, None, None, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, D_, None, 1, 2, 96, 232, 232, 231, 0.1, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 2, 128, 232, 232, 0, 0.1, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 2, 128, 232, 232, 233, 0.1, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 2, 128, 0, 232, 231, 0.1, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 0, 2, 128, 232, 232, 231, 0.1, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 2, 128, 232, 232, 231, 0.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 2, 128, 232, 232, 231, float("nan"), None) == ltxa.LTXA_E_SHAPE
    assert f(A + 8, B, C, D_, None, *good, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, D_, E + 4, *good, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, A + 64, None, *good, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, D_, C + 128, *good, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, D_, None, 1 << 30, 1 << 10, 128, 1 << 20, 1 << 20, 1, 0.1, None) == ltxa.LTXA_E_RANGE


def test_pack_rope_errors(L):
    f = L.ltxa_sp_pack_rope
    mp3 = _mp(3, 7, 11)
    # src, dst, pos, n, axes, max_pos, batch, heads, head_dim, world_size, theta
    assert f(None, B, C, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, None, C, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, B, None, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, 232, 3, None, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, 232, 3, mp3, 0, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 3, mp3, 1, 4, 64, 0, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 3, mp3, 1, 4, 63, 2, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 4, _mp(1, 1, 1, 1), 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 3, mp3, 1, 4, 64, 2, -1.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 0, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 3, mp3, 1, 6, 64, 4, 1e4, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, C, 231, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, C, 232, 3, mp3, 1, 4, 4, 2, 1e4, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B + 8, C, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C + 4, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_ALIGN
    assert f(A, A + 256, C, 232, 3, mp3, 1, 4, 64, 2, 1e4, None) == ltxa.LTXA_E_ALIAS


def test_attn_unpack_errors(L):
    f = L.ltxa_attn_fwd_unpack
    good = (1, 8, 128, 232, 232, 231, 0.088)
    assert f(None, B, C, D_, None, *good, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, None, None, *good, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, D_, None, *good, 0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, *good, 3, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, C, D_, None, 1, 8, 96, 232, 232, 231, 0.1, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 8, 128, 232, 232, 0, 0.1, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A + 8, B, C, D_, None, *good, 2, None) == ltxa.LTXA_E_ALIGN
    # o spans world_size * batch * nq * (heads/world_size) rows, as q does.
    assert f(A, B, C, A + 64, None, *good, 2, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, D_, None, 1 << 40, 1 << 13, 128, 232, 232, 231, 0.1, 1 << 13, None) == ltxa.LTXA_E_RANGE


def test_rope_opts_out_scale_layout():
    # out_scale took the place of a reserved int32 that had to be 0: the
    # struct keeps its size and offsets, and 0 still means "as before".
    assert ctypes.sizeof(ltxa.RopeOpts) == 6 * 4
    assert ltxa.RopeOpts.out_scale.offset == 5 * 4
    text = open(HEADER).read()
    assert re.search(r"float out_scale;", text) and "reserved" not in text
    o = ltxa.rope_opts()
    assert o.out_scale == 0.0


def test_attn_log2q_errors(L):
    f = L.ltxa_attn_fwd_log2q
    good = (1, 8, 128, 232, 232, 231)  # no scale argument
    assert f(None, B, C, D_, None, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, None, None, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, D_, None, 0, 8, 128, 232, 232, 231, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 8, 96, 232, 232, 231, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 8, 128, 232, 232, 0, None) == ltxa.LTXA_E_SHAPE
    assert f(A + 8, B, C, D_, None, *good, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, A + 64, None, *good, None) == ltxa.LTXA_E_ALIAS


def test_attn_unpack_log2q_errors(L):
    f = L.ltxa_attn_fwd_unpack_log2q
    good = (1, 8, 128, 232, 232, 231)  # no scale argument
    assert f(None, B, C, D_, None, *good, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, None, None, *good, 2, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, D_, None, *good, 0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, *good, 3, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, C, D_, None, 1, 8, 96, 232, 232, 231, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, D_, None, 1, 8, 128, 232, 232, 0, 2, None) == ltxa.LTXA_E_SHAPE
    assert f(A + 8, B, C, D_, None, *good, 2, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, A + 64, None, *good, 2, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, D_, None, 1 << 40, 1 << 13, 128, 232, 232, 231, 1 << 13, None) == ltxa.LTXA_E_RANGE


def test_log2_domain_scale_matches_kernel_rounding():
    import numpy as np
    for d in (64, 128):
        sc = 1.0 / d ** 0.5
        c = ltxa.log2_domain_scale(sc)
        assert c == float(np.float32(c))                       # an fp32 value
        assert abs(c - sc * 1.4426950408889634) <= 2 ** -24 * c  # the nearest one, to within rounding
    assert ltxa.log2_domain_scale(1.0) == float(np.float32(1.4426950408889634))


def _opts(**kw):
    return ctypes.byref(ltxa.rope_opts(**kw)) if kw else None


def _raw_opts(*vals):
    return ctypes.byref(ltxa.RopeOpts(*vals))


def test_rope_ex_errors(L):
    f = L.ltxa_rope_ex
    mp3 = _mp(3, 7, 11)
    # x, pos, n, axes, max_pos, batch, heads, head_dim, theta, opts
    assert f(None, C, 232, 3, mp3, 1, 4, 64, 1e4, None, None) == ltxa.LTXA_E_NULL
    assert f(A, None, 232, 3, mp3, 1, 4, 64, 1e4, None, None) == ltxa.LTXA_E_NULL
    assert f(A, C, 232, 3, None, 1, 4, 64, 1e4, None, None) == ltxa.LTXA_E_NULL
    assert f(A, C, 232, 3, mp3, 0, 4, 64, 1e4, None, None) == ltxa.LTXA_E_SHAPE
    assert f(A, C, 232, 3, mp3, 1, 4, 62, 1e4, None, None) == ltxa.LTXA_E_ALIGN
    assert f(A + 2, C, 232, 3, mp3, 1, 4, 64, 1e4, None, None) == ltxa.LTXA_E_ALIGN
    bad = [(2, 0, 0, 0, 0, 0), (0, 0, 0, 2, 0, 0), (0, 0, 0, 0, 2, 0), (0, 0, 0, 0, 0, -1.0),
           (0, 0, 0, 0, 0, float("inf")), (0, 0, 0, 0, 0, float("nan")),
           (0, -1, 0, 0, 0, 0), (0, 4, -1, 0, 0, 0), (0, 4, 1, 0, 0, 0), (0, 3, 0, 0, 0, 0)]
    for vals in bad:
        assert f(A, C, 232, 3, mp3, 1, 4, 64, 1e4, _raw_opts(*vals), None) == ltxa.LTXA_E_SHAPE, vals
    # Fewer grid pairs than axes: one head of 4 channels has 2 pairs.
    assert f(A, C, 232, 3, mp3, 1, 1, 4, 1e4, _opts(grid_heads=1), None) in (ltxa.LTXA_E_SHAPE,
                                                                            ltxa.LTXA_E_ALIGN)
    # SPLIT needs 16-element halves-of-8: head_dim % 16 == 0.
    assert f(A, C, 232, 3, mp3, 1, 4, 24, 1e4, _opts(rope_type="split"), None) == ltxa.LTXA_E_ALIGN


def test_pack_rope_ex_errors(L):
    f = L.ltxa_sp_pack_rope_ex
    mp3 = _mp(3, 7, 11)
    args = (232, 3, mp3, 1, 4, 64, 2, 1e4)
    assert f(None, B, C, *args, None, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, 231, 3, mp3, 1, 4, 64, 2, 1e4, None, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, A + 256, C, *args, None, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, *args, _opts(grid_heads=3), None) == ltxa.LTXA_E_SHAPE     # 4 heads > 3
    assert f(A, B, C, *args, _opts(grid_heads=5, head_offset=2), None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, *args, _raw_opts(0, 0, 0, 0, 0, -7.0), None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 3, mp3, 1, 4, 40, 2, 1e4, _opts(rope_type="split"), None) == ltxa.LTXA_E_ALIGN


def test_rope_table_errors(L):
    f = L.ltxa_rope_table
    mp3 = _mp(3, 7, 11)
    # pos, n, axes, max_pos, head_dim, theta, opts, table, stream
    assert f(None, 232, 3, mp3, 64, 1e4, None, B, None) == ltxa.LTXA_E_NULL
    assert f(C, 232, 3, None, 64, 1e4, None, B, None) == ltxa.LTXA_E_NULL
    assert f(C, 232, 3, mp3, 64, 1e4, None, None, None) == ltxa.LTXA_E_NULL
    assert f(C, 0, 3, mp3, 64, 1e4, None, B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 4, mp3, 64, 1e4, None, B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 3, mp3, 63, 1e4, None, B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 3, mp3, 64, -1.0, None, B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 3, mp3, 62, 1e4, None, B, None) == ltxa.LTXA_E_ALIGN
    assert f(C, 232, 3, mp3, 64, 1e4, None, B + 4, None) == ltxa.LTXA_E_ALIGN
    # The table serves the head-shared grid and holds unscaled angles.
    assert f(C, 232, 3, mp3, 64, 1e4, _opts(grid_heads=4), B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 3, mp3, 64, 1e4, _opts(out_scale=0.5), B, None) == ltxa.LTXA_E_SHAPE
    assert f(C, 232, 3, mp3, 64, 1e4, _raw_opts(2, 0, 0, 0, 0, 0), B, None) == ltxa.LTXA_E_SHAPE
    # 232 tokens x 3 axes of int32 positions start 16 bytes below the table.
    assert f(B - 16, 232, 3, mp3, 64, 1e4, None, B, None) == ltxa.LTXA_E_ALIAS
    assert f(C, 1 << 38, 3, mp3, 64, 1e4, None, B, None) == ltxa.LTXA_E_RANGE


def test_pack_rope_table_errors(L):
    f = L.ltxa_sp_pack_rope_table
    # src, dst, table, n, batch, heads, head_dim, world_size, rope_type, out_scale, stream
    good = (232, 1, 4, 64, 2, 0, 0.0)
    assert f(None, B, C, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, None, C, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, None, *good, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, 0, 1, 4, 64, 2, 0, 0.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 1, 4, 63, 2, 0, 0.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 1, 4, 64, 0, 0, 0.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, 232, 1, 4, 64, 2, 2, 0.0, None) == ltxa.LTXA_E_SHAPE
    for sc in (-1.0, float("inf"), float("nan")):
        assert f(A, B, C, 232, 1, 4, 64, 2, 0, sc, None) == ltxa.LTXA_E_SHAPE, sc
    assert f(A, B, C, 232, 1, 4, 62, 2, 0, 0.0, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, 232, 1, 4, 40, 2, 1, 0.0, None) == ltxa.LTXA_E_ALIGN  # SPLIT: head_dim % 16
    assert f(A + 8, B, C, *good, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C + 8, *good, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, C, 232, 1, 4, 64, 3, 0, 0.0, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, C, 231, 1, 4, 64, 2, 0, 0.0, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, A + 256, C, *good, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, B + 256, *good, None) == ltxa.LTXA_E_ALIAS
    assert f(A, B, C, 1 << 40, 1 << 13, 4, 64, 2, 0, 0.0, None) == ltxa.LTXA_E_RANGE


def test_pack_rope_qk_table_errors(L):
    f = L.ltxa_sp_pack_rope_qk_table
    # q, q_dst, q_scale, k, k_dst, k_scale, table, n, batch, heads, head_dim, world_size, rope_type, stream
    sizes = (232, 1, 4, 64, 2, 0)
    assert f(A, B, 0.0, None, E, 0.0, C, *sizes, None) == ltxa.LTXA_E_NULL
    assert f(A, B, 0.0, D_, None, 0.0, C, *sizes, None) == ltxa.LTXA_E_NULL
    assert f(A, B, 0.0, D_, E, 0.0, None, *sizes, None) == ltxa.LTXA_E_NULL
    assert f(A, B, 0.0, D_, E, -1.0, C, *sizes, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, float("nan"), D_, E, 0.0, C, *sizes, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, 0.0, D_ + 8, E, 0.0, C, *sizes, None) == ltxa.LTXA_E_ALIGN
    assert f(A, B, 0.0, D_, E, 0.0, C, 231, 1, 4, 64, 2, 0, None) == ltxa.LTXA_E_DIVISIBILITY
    assert f(A, B, 0.0, B + 256, E, 0.0, C, *sizes, None) == ltxa.LTXA_E_ALIAS   # q_dst on k
    assert f(A, B, 0.0, D_, B + 256, 0.0, C, *sizes, None) == ltxa.LTXA_E_ALIAS  # both destinations
    assert f(A, B, 0.0, D_, A + 256, 0.0, C, *sizes, None) == ltxa.LTXA_E_ALIAS  # k_dst on q
    assert f(A, B, 0.0, D_, C + 256, 0.0, C, *sizes, None) == ltxa.LTXA_E_ALIAS  # k_dst on the table


def test_rope_qk_ex_errors(L):
    f = L.ltxa_rope_qk_ex
    mp = (ctypes.c_double * 3)(5.0, 7.0, 9.0)
    # q, k, pos, n, axes, max_pos, batch, heads, head_dim, theta, opts, k_scale, stream
    sizes = (232, 3, mp, 1, 4, 64, 10000.0, None)
    assert f(A, None, C, *sizes, 0.0, None) == ltxa.LTXA_E_NULL
    assert f(None, B, C, *sizes, 0.0, None) == ltxa.LTXA_E_NULL
    assert f(A, B, C, *sizes, -1.0, None) == ltxa.LTXA_E_SHAPE
    assert f(A, B, C, *sizes, float("nan"), None) == ltxa.LTXA_E_SHAPE
    assert f(A, B + 8, C, *sizes, 0.0, None) == ltxa.LTXA_E_ALIGN
    assert f(A, A + 256, C, *sizes, 0.0, None) == ltxa.LTXA_E_ALIAS   # k overlaps q
    assert f(A, C, C, *sizes, 0.0, None) == ltxa.LTXA_E_ALIAS         # k on the positions
    assert f(A, B, C, 232, 3, mp, 1, 4, 63, 10000.0, None, 0.0, None) == ltxa.LTXA_E_SHAPE


def test_sp_share_bookkeeping():
    s = ltxa.SpShare(max_tokens=32768, num_heads=32, head_dim=128, world_size=8)
    assert s.heads_per_rank == 4 and s.tokens_per_rank_max == 4096
    assert s.set_seqlen(32761) == 32768 and s.tokens_per_rank == 4096
    assert s.set_seqlen(6144) == 6144
    assert s.set_seqlen(32768) == 32768
    with pytest.raises(ValueError, match="smaller resolution or fewer frames"):
        s.set_seqlen(32769)
    with pytest.raises(ValueError):
        s.set_seqlen(0)
    with pytest.raises(ValueError, match="divisible"):
        ltxa.SpShare(max_tokens=232, num_heads=2, head_dim=64, world_size=4)
    t = ltxa.SpShare(max_tokens=231, num_heads=4, head_dim=64, world_size=4)
    assert t.tokens_per_rank_max == 58 and t.set_seqlen(231) == 232
    with pytest.raises(TypeError):
        ltxa.SpShare(max_tokens=64, num_heads=4, head_dim=64, world_size=2, tensor_dtype=torch.float32)


def test_sp_share_owns_and_reuses_buffers():
    # The page's AttentionManager owns the exchange buffers, sized for
    # ceil(max_tokens / world_size) tokens per rank.  The sizing and reuse
    # logic is host code; CPU tensors stand in for device memory here.
    s = ltxa.SpShare(max_tokens=32761, num_heads=32, head_dim=128, world_size=8)
    with pytest.raises(ValueError, match="set_seqlen"):
        s.buffers(1, "cpu")
    s.set_seqlen(32761)                       # 32768 after padding
    b = s.buffers(1, "cpu")
    assert b["q"].shape == (8, 1, 32768, 4, 128) and b["out"].shape == (1, 32768, 32, 128)
    assert b["k"].shape == b["v"].shape == (8, 1, 32768, 4, 128)
    cap = 4096 * 8 * 32 * 128                 # per-rank ceil(32761 / 8) = 4096 tokens x 8 ranks
    assert all(s._store[n].numel() == cap for n in ("q", "k", "v", "out"))
    ptrs = {n: t.data_ptr() for n, t in b.items()}
    s.set_seqlen(6000)                        # a shorter step reuses the same memory
    b2 = s.buffers(1, "cpu")
    assert b2["q"].shape == (8, 1, 6000, 4, 128)
    assert {n: t.data_ptr() for n, t in b2.items()} == ptrs
    b3 = s.buffers(1, "cpu", nk=1024)         # cross-attention keys: a view of the same K/V buffers
    assert b3["k"].shape == (8, 1, 1024, 4, 128) and b3["k"].data_ptr() == ptrs["k"]
    b4 = s.buffers(2, "cpu")                  # batch 2 of 6000 tokens still fits
    assert b4["q"].shape == (8, 2, 6000, 4, 128) and b4["q"].data_ptr() == ptrs["q"]
    s.set_seqlen(32761)
    b5 = s.buffers(2, "cpu")                  # batch 2 at max_tokens grows them once
    assert b5["q"].shape == (8, 2, 32768, 4, 128) and s._store["q"].numel() == 2 * cap


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 8, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        ltxa.sp_pack(x, 2)
    with pytest.raises(ValueError, match="GPU"):
        ltxa.attn_fwd(x, x, x)

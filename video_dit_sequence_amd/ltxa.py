"""Thin ctypes binding over ``libltxa.so`` (C ABI in ``include/ltxa.h``).

Argument marshalling only: each function checks that it got torch tensors of
the right dtype on a GPU, passes their device pointers, sizes and the current
HIP stream to the C entry point of the same name, and raises
:class:`LtxaError` on a non-zero status.  Every step of the computation runs
in the library's HIP kernels; there is no fallback.  If the library is
missing, :func:`lib` raises.

``SpShare`` is the host-side bookkeeping of one sequence-parallel attention
group (LTX-2 "Sequence Parallelism (SP)" page, "API / AttentionManager":
``max_tokens`` bound, ``num_heads`` divisible by ``world_size``, per-rank
buffers of ``ceil(max_tokens / world_size)`` tokens; "How the forward pass
works" step 1: pad to a multiple of ``world_size``; "Usage": exceeding
``max_tokens`` raises and asks for a smaller resolution or fewer frames).
"""

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libltxa.so")

LTXA_OK = 0
LTXA_E_NULL = -1
LTXA_E_SHAPE = -2
LTXA_E_DIVISIBILITY = -3
LTXA_E_ALIGN = -4
LTXA_E_ALIAS = -5
LTXA_E_HIP = -6
LTXA_E_RANGE = -7

EXPORTS = ("ltxa_version", "ltxa_status_string", "ltxa_sp_pack", "ltxa_sp_unpack",
           "ltxa_rope_qk", "ltxa_attn_fwd", "ltxa_sp_pack_rope", "ltxa_attn_fwd_unpack",
           "ltxa_rope_ex", "ltxa_sp_pack_rope_ex", "ltxa_attn_fwd_log2q",
           "ltxa_attn_fwd_unpack_log2q", "ltxa_rope_table", "ltxa_sp_pack_rope_table",
           "ltxa_sp_pack_rope_qk_table", "ltxa_rope_qk_ex")

LTXA_ROPE_INTERLEAVED = 0
LTXA_ROPE_SPLIT = 1


class RopeOpts(ctypes.Structure):
    """``ltxa_rope_opts``: the rotary variants (see ``include/ltxa.h``)."""
    _fields_ = [("rope_type", ctypes.c_int32), ("grid_heads", ctypes.c_int32),
                ("head_offset", ctypes.c_int32), ("fp64_angles", ctypes.c_int32),
                ("middle", ctypes.c_int32), ("out_scale", ctypes.c_float)]


def rope_opts(rope_type: str = "interleaved", grid_heads: int = 0, head_offset: int = 0,
              fp64_angles: bool = False, middle: bool = False, out_scale: float = 0.0) -> RopeOpts:
    """Build an ``ltxa_rope_opts``.  ``rope_type`` is "interleaved" or "split";
    ``grid_heads = 0`` shares one head_dim-wide grid across heads, ``G > 0``
    lays the grid over ``G`` heads (head ``j`` of a tensor is grid head
    ``head_offset + j``).  ``out_scale`` (0: none) multiplies every output
    value before its one rounding to bf16."""
    types = {"interleaved": LTXA_ROPE_INTERLEAVED, "split": LTXA_ROPE_SPLIT}
    if rope_type not in types:
        raise ValueError("rope_type must be 'interleaved' or 'split'")
    return RopeOpts(types[rope_type], int(grid_heads), int(head_offset), int(bool(fp64_angles)),
                    int(bool(middle)), float(out_scale))


class LtxaError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed with status {status}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if ``libltxa.so`` has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_dit_sequence_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.ltxa_version.restype = ctypes.c_int
        L.ltxa_version.argtypes = []
        L.ltxa_status_string.restype = ctypes.c_char_p
        L.ltxa_status_string.argtypes = [ctypes.c_int]
        perm_args = [vp, vp, i64, i64, i32, i32, i32, i32, vp]
        for name in ("ltxa_sp_pack", "ltxa_sp_unpack"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = perm_args
        L.ltxa_rope_qk.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        L.ltxa_rope_qk.argtypes = [vp, vp, i64, i32, dp, vp, vp, i64, i32, dp,
                                   i64, i32, i32, ctypes.c_double, vp]
        L.ltxa_attn_fwd.restype = ctypes.c_int
        L.ltxa_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i64, i64,
                                    ctypes.c_float, vp]
        L.ltxa_sp_pack_rope.restype = ctypes.c_int
        L.ltxa_sp_pack_rope.argtypes = [vp, vp, vp, i64, i32, dp, i64, i32, i32, i32,
                                        ctypes.c_double, vp]
        op = ctypes.POINTER(RopeOpts)
        L.ltxa_rope_ex.restype = ctypes.c_int
        L.ltxa_rope_ex.argtypes = [vp, vp, i64, i32, dp, i64, i32, i32, ctypes.c_double, op, vp]
        L.ltxa_sp_pack_rope_ex.restype = ctypes.c_int
        L.ltxa_sp_pack_rope_ex.argtypes = [vp, vp, vp, i64, i32, dp, i64, i32, i32, i32,
                                           ctypes.c_double, op, vp]
        L.ltxa_attn_fwd_unpack.restype = ctypes.c_int
        L.ltxa_attn_fwd_unpack.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i64, i64,
                                           ctypes.c_float, i32, vp]
        L.ltxa_attn_fwd_log2q.restype = ctypes.c_int
        L.ltxa_attn_fwd_log2q.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i64, i64, vp]
        L.ltxa_attn_fwd_unpack_log2q.restype = ctypes.c_int
        L.ltxa_attn_fwd_unpack_log2q.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i64, i64,
                                                 i32, vp]
        L.ltxa_rope_table.restype = ctypes.c_int
        L.ltxa_rope_table.argtypes = [vp, i64, i32, dp, i32, ctypes.c_double, op, vp, vp]
        L.ltxa_sp_pack_rope_table.restype = ctypes.c_int
        L.ltxa_sp_pack_rope_table.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, ctypes.c_float, vp]
        L.ltxa_rope_qk_ex.restype = ctypes.c_int
        L.ltxa_rope_qk_ex.argtypes = [vp, vp, vp, i64, i32, ctypes.POINTER(ctypes.c_double), i64, i32, i32,
                                      ctypes.c_double, vp, ctypes.c_float, vp]
        L.ltxa_sp_pack_rope_qk_table.restype = ctypes.c_int
        L.ltxa_sp_pack_rope_qk_table.argtypes = [vp, vp, ctypes.c_float, vp, vp, ctypes.c_float, vp, i64, i64,
                                                 i32, i32, i32, i32, vp]
        _lib = L
    return _lib


def version() -> int:
    return lib().ltxa_version()


def status_string(status: int) -> str:
    return lib().ltxa_status_string(status).decode()


def _check(call: str, status: int):
    if status != LTXA_OK:
        raise LtxaError(call, status)


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _gpu(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def sp_pack(src: torch.Tensor, world_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``[B, N, H, D]`` -> ``[P, B, N, H/P, D]`` (``ltxa_sp_pack``)."""
    _gpu(src, "src")
    B, N, H, D = src.shape
    P = int(world_size)
    if out is None:
        if P < 1 or H % P:
            _check("ltxa_sp_pack", LTXA_E_DIVISIBILITY if P >= 1 else LTXA_E_SHAPE)
        out = torch.empty((P, B, N, H // P, D), dtype=src.dtype, device=src.device)
    _gpu(out, "out", src.dtype)
    if out.numel() != src.numel():
        raise ValueError("out has the wrong number of elements")
    _check("ltxa_sp_pack", lib().ltxa_sp_pack(src.data_ptr(), out.data_ptr(), B, N, H, D, P,
                                              src.element_size(), _stream_ptr(src)))
    return out


def sp_unpack(src: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``[P, B, N, H/P, D]`` -> ``[B, N, H, D]`` (``ltxa_sp_unpack``)."""
    _gpu(src, "src")
    P, B, N, Hl, D = src.shape
    if out is None:
        out = torch.empty((B, N, P * Hl, D), dtype=src.dtype, device=src.device)
    _gpu(out, "out", src.dtype)
    if out.numel() != src.numel():
        raise ValueError("out has the wrong number of elements")
    _check("ltxa_sp_unpack", lib().ltxa_sp_unpack(src.data_ptr(), out.data_ptr(), B, N, P * Hl, D, P,
                                                  src.element_size(), _stream_ptr(src)))
    return out


def _max_pos_array(max_pos: Sequence[float]):
    return (ctypes.c_double * len(max_pos))(*[float(x) for x in max_pos])


def rope_qk(q: Optional[torch.Tensor], q_pos: Optional[torch.Tensor], q_max_pos,
            k: Optional[torch.Tensor], k_pos: Optional[torch.Tensor], k_max_pos,
            theta: float = 10000.0) -> None:
    """Rotate bf16 ``q`` and/or ``k`` (``[B, N, H, D]``) in place (``ltxa_rope_qk``).

    ``q_pos``/``k_pos`` are int32 ``[N, A]`` GPU tensors; ``*_max_pos`` hold
    ``A`` positive numbers.  Either ``q`` or ``k`` may be ``None``.
    """
    ref = q if q is not None else k
    if ref is None:
        _check("ltxa_rope_qk", LTXA_E_NULL)
    B, _, H, D = ref.shape
    args = []
    for x, pos, mp, name in ((q, q_pos, q_max_pos, "q"), (k, k_pos, k_max_pos, "k")):
        if x is None:
            args += [None, None, 0, 0, None]
            continue
        _gpu(x, name, torch.bfloat16)
        _gpu(pos, f"{name}_pos", torch.int32)
        if x.dim() != 4 or x.shape[0] != B or x.shape[2] != H or x.shape[3] != D:
            raise ValueError("q and k must be [B, N, H, D] with the same B, H and D")
        if pos.dim() != 2 or pos.shape[0] != x.shape[1] or pos.shape[1] != len(mp):
            raise ValueError(f"{name}_pos must be [N, A] with one max_pos per axis")
        args += [x.data_ptr(), pos.data_ptr(), x.shape[1], pos.shape[1], _max_pos_array(mp)]
    _check("ltxa_rope_qk", lib().ltxa_rope_qk(*args, B, H, D, float(theta), _stream_ptr(ref)))


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, nk_valid: Optional[int] = None,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, q_log2: bool = False) -> torch.Tensor:
    """Masked attention (``ltxa_attn_fwd``) over bf16 BSHD tensors.

    Keys ``>= nk_valid`` (default: all) are excluded.  ``scale`` defaults to
    ``1/sqrt(D)``.  ``lse``, if given, is a float32 ``[B, H, Nq]`` tensor.
    With ``q_log2`` the queries are already multiplied by ``scale * log2(e)``
    (:func:`log2_domain_scale`) and ``scale`` is not used
    (``ltxa_attn_fwd_log2q``).
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _gpu(t, name, torch.bfloat16)
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    if k.shape != (B, Nk, H, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Nk, H, D] matching q")
    nk_valid = Nk if nk_valid is None else int(nk_valid)
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _gpu(out, "out", torch.bfloat16)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    lse_ptr = None
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
        if lse.shape != (B, H, Nq):
            raise ValueError("lse must be [B, H, Nq]")
        lse_ptr = lse.data_ptr()
    if q_log2:
        _check("ltxa_attn_fwd_log2q", lib().ltxa_attn_fwd_log2q(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, H, D, Nq, Nk, nk_valid,
            _stream_ptr(q)))
    else:
        _check("ltxa_attn_fwd", lib().ltxa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                    out.data_ptr(), lse_ptr, B, H, D, Nq, Nk, nk_valid,
                                                    scale, _stream_ptr(q)))
    return out


def rope(x: torch.Tensor, pos: torch.Tensor, max_pos, theta: float = 10000.0,
         opts: Optional[RopeOpts] = None, out_scale: Optional[float] = None) -> None:
    """Rotate bf16 ``x`` (``[B, N, H, D]``) in place with the variants of
    ``opts`` (:func:`rope_opts`; ``None`` = the rotation of :func:`rope_qk`)
    (``ltxa_rope_ex``).  ``out_scale`` overrides ``opts.out_scale``."""
    opts = _with_scale(opts, out_scale)
    _gpu(x, "x", torch.bfloat16)
    _gpu(pos, "pos", torch.int32)
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, D]")
    B, N, H, D = x.shape
    if pos.dim() != 2 or pos.shape[0] != N or pos.shape[1] != len(max_pos):
        raise ValueError("pos must be [N, A] with one max_pos per axis")
    _check("ltxa_rope_ex", lib().ltxa_rope_ex(
        x.data_ptr(), pos.data_ptr(), N, pos.shape[1], _max_pos_array(max_pos), B, H, D, float(theta),
        None if opts is None else ctypes.byref(opts), _stream_ptr(x)))


def rope_qk_ex(q: torch.Tensor, k: torch.Tensor, pos: torch.Tensor, max_pos, theta: float = 10000.0,
               opts: Optional[RopeOpts] = None, q_scale: Optional[float] = None, k_scale: float = 0.0) -> None:
    """Rotate bf16 ``q`` and ``k`` (both ``[B, N, H, D]``) in place by the same
    positions and options in one launch (``ltxa_rope_qk_ex``): equal, bit for
    bit, to :func:`rope` of each.  ``q_scale`` overrides ``opts.out_scale``
    for ``q``; ``k_scale`` (0: none) scales ``k``."""
    opts = _with_scale(opts, q_scale)
    _gpu(q, "q", torch.bfloat16)
    _gpu(k, "k", torch.bfloat16)
    _gpu(pos, "pos", torch.int32)
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must be [B, N, H, D] of one shape")
    B, N, H, D = q.shape
    if pos.dim() != 2 or pos.shape[0] != N or pos.shape[1] != len(max_pos):
        raise ValueError("pos must be [N, A] with one max_pos per axis")
    _check("ltxa_rope_qk_ex", lib().ltxa_rope_qk_ex(
        q.data_ptr(), k.data_ptr(), pos.data_ptr(), N, pos.shape[1], _max_pos_array(max_pos), B, H, D,
        float(theta), None if opts is None else ctypes.byref(opts), float(k_scale), _stream_ptr(q)))


def _with_scale(opts: Optional[RopeOpts], out_scale: Optional[float]) -> Optional[RopeOpts]:
    """``opts`` with ``out_scale`` set (a copy; ``opts`` None: the defaults)."""
    if out_scale is None:
        return opts
    o = rope_opts() if opts is None else RopeOpts.from_buffer_copy(opts)
    o.out_scale = float(out_scale)
    return o


def log2_domain_scale(scale: float) -> float:
    """``scale * log2(e)`` as the attention kernel forms it: the fp32 scale
    widened to double, multiplied, rounded to fp32.  Passed as ``out_scale``
    to :func:`sp_pack_rope`, it makes the log2-domain queries that
    :func:`attn_fwd_unpack` takes with ``q_log2=True``."""
    return float(np.float32(np.float64(np.float32(scale)) * 1.4426950408889634))


def sp_pack_rope(src: torch.Tensor, pos: torch.Tensor, max_pos, world_size: int,
                 theta: float = 10000.0, out: Optional[torch.Tensor] = None,
                 opts: Optional[RopeOpts] = None, out_scale: Optional[float] = None) -> torch.Tensor:
    """bf16 ``[B, N, H, D]`` -> rotated ``[P, B, N, H/P, D]`` (``ltxa_sp_pack_rope``,
    or ``ltxa_sp_pack_rope_ex`` when ``opts`` or ``out_scale`` is given).

    Equal, bit for bit, to :func:`sp_pack` followed by the rotation of each
    rank's shard.  ``pos`` is an int32 ``[N, A]`` GPU tensor.  ``out_scale``
    multiplies every output value before its one rounding to bf16.
    """
    _gpu(src, "src", torch.bfloat16)
    _gpu(pos, "pos", torch.int32)
    B, N, H, D = src.shape
    P = int(world_size)
    if pos.dim() != 2 or pos.shape[0] != N or pos.shape[1] != len(max_pos):
        raise ValueError("pos must be [N, A] with one max_pos per axis")
    if out is None:
        if P < 1 or H % P:
            _check("ltxa_sp_pack_rope", LTXA_E_DIVISIBILITY if P >= 1 else LTXA_E_SHAPE)
        out = torch.empty((P, B, N, H // P, D), dtype=src.dtype, device=src.device)
    _gpu(out, "out", torch.bfloat16)
    if out.numel() != src.numel():
        raise ValueError("out has the wrong number of elements")
    opts = _with_scale(opts, out_scale)
    if opts is None:
        _check("ltxa_sp_pack_rope", lib().ltxa_sp_pack_rope(
            src.data_ptr(), out.data_ptr(), pos.data_ptr(), N, pos.shape[1], _max_pos_array(max_pos),
            B, H, D, P, float(theta), _stream_ptr(src)))
    else:
        _check("ltxa_sp_pack_rope_ex", lib().ltxa_sp_pack_rope_ex(
            src.data_ptr(), out.data_ptr(), pos.data_ptr(), N, pos.shape[1], _max_pos_array(max_pos),
            B, H, D, P, float(theta), ctypes.byref(opts), _stream_ptr(src)))
    return out


def rope_table(pos: torch.Tensor, max_pos, head_dim: int, theta: float = 10000.0,
               opts: Optional[RopeOpts] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cos and sin of every (token, pair) of the head-shared grid
    (``ltxa_rope_table``): float32 ``[N, head_dim/2, 2]``.

    ``pos`` is an int32 ``[N, A]`` GPU tensor.  Of ``opts`` only ``fp64_angles``
    and ``middle`` act; ``grid_heads`` and ``out_scale`` must be 0.  Rotating
    with the table (:func:`sp_pack_rope_table`) equals rotating with the
    positions, bit for bit.
    """
    _gpu(pos, "pos", torch.int32)
    if pos.dim() != 2 or pos.shape[1] != len(max_pos):
        raise ValueError("pos must be [N, A] with one max_pos per axis")
    N = pos.shape[0]
    if out is None:
        out = torch.empty((N, max(int(head_dim) // 2, 1), 2), dtype=torch.float32, device=pos.device)
    _gpu(out, "out", torch.float32)
    if out.numel() != N * (int(head_dim) // 2) * 2:
        raise ValueError("out must hold N * head_dim/2 * 2 floats")
    _check("ltxa_rope_table", lib().ltxa_rope_table(
        pos.data_ptr(), N, pos.shape[1], _max_pos_array(max_pos), int(head_dim), float(theta),
        ctypes.byref(opts) if opts is not None else None, out.data_ptr(), _stream_ptr(pos)))
    return out


def sp_pack_rope_table(src: torch.Tensor, table: torch.Tensor, world_size: int, rope_type: str = "interleaved",
                       out_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 ``[B, N, H, D]`` -> rotated ``[P, B, N, H/P, D]`` with the angles of
    a :func:`rope_table` (``ltxa_sp_pack_rope_table``).

    Equal, bit for bit, to :func:`sp_pack_rope` with the positions and options
    the table was made from, this ``rope_type`` and ``out_scale``.
    """
    _gpu(src, "src", torch.bfloat16)
    _gpu(table, "table", torch.float32)
    B, N, H, D = src.shape
    P = int(world_size)
    types = {"interleaved": LTXA_ROPE_INTERLEAVED, "split": LTXA_ROPE_SPLIT}
    if rope_type not in types:
        raise ValueError("rope_type must be 'interleaved' or 'split'")
    if table.numel() != N * (D // 2) * 2:
        raise ValueError("table must be [N, D/2, 2]")
    if out is None:
        if P < 1 or H % P:
            _check("ltxa_sp_pack_rope_table", LTXA_E_DIVISIBILITY if P >= 1 else LTXA_E_SHAPE)
        out = torch.empty((P, B, N, H // P, D), dtype=src.dtype, device=src.device)
    _gpu(out, "out", torch.bfloat16)
    if out.numel() != src.numel():
        raise ValueError("out has the wrong number of elements")
    _check("ltxa_sp_pack_rope_table", lib().ltxa_sp_pack_rope_table(
        src.data_ptr(), out.data_ptr(), table.data_ptr(), N, B, H, D, P, types[rope_type], float(out_scale),
        _stream_ptr(src)))
    return out


def sp_pack_rope_qk_table(q: torch.Tensor, k: torch.Tensor, table: torch.Tensor, world_size: int,
                          rope_type: str = "interleaved", q_scale: float = 0.0, k_scale: float = 0.0,
                          q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None):
    """Q and K, each bf16 ``[B, N, H, D]``, -> rotated ``[P, B, N, H/P, D]`` with
    one :func:`rope_table`, in one launch (``ltxa_sp_pack_rope_qk_table``).

    Returns ``(q_out, k_out)``, equal, bit for bit, to
    :func:`sp_pack_rope_table` of each with its own scale.
    """
    _gpu(q, "q", torch.bfloat16)
    _gpu(k, "k", torch.bfloat16)
    _gpu(table, "table", torch.float32)
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    B, N, H, D = q.shape
    P = int(world_size)
    types = {"interleaved": LTXA_ROPE_INTERLEAVED, "split": LTXA_ROPE_SPLIT}
    if rope_type not in types:
        raise ValueError("rope_type must be 'interleaved' or 'split'")
    if table.numel() != N * (D // 2) * 2:
        raise ValueError("table must be [N, D/2, 2]")
    outs = []
    for o in (q_out, k_out):
        if o is None:
            if P < 1 or H % P:
                _check("ltxa_sp_pack_rope_qk_table", LTXA_E_DIVISIBILITY if P >= 1 else LTXA_E_SHAPE)
            o = torch.empty((P, B, N, H // P, D), dtype=q.dtype, device=q.device)
        _gpu(o, "out", torch.bfloat16)
        if o.numel() != q.numel():
            raise ValueError("out has the wrong number of elements")
        outs.append(o)
    _check("ltxa_sp_pack_rope_qk_table", lib().ltxa_sp_pack_rope_qk_table(
        q.data_ptr(), outs[0].data_ptr(), float(q_scale), k.data_ptr(), outs[1].data_ptr(), float(k_scale),
        table.data_ptr(), N, B, H, D, P, types[rope_type], _stream_ptr(q)))
    return outs[0], outs[1]


def attn_fwd_unpack(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, nk_valid: Optional[int] = None,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, q_log2: bool = False) -> torch.Tensor:
    """Attention over head shards ``[P, B, N, H/P, D]`` with the output in token
    order ``[B, Nq, H, D]`` (``ltxa_attn_fwd_unpack``).

    Equal, bit for bit, to :func:`attn_fwd` over the ``P * B`` shard entries
    followed by :func:`sp_unpack`.  ``lse``, if given, is float32
    ``[P, B, H/P, Nq]``.  With ``q_log2`` the queries are already multiplied by
    ``scale * log2(e)`` (:func:`log2_domain_scale`) and ``scale`` is not used
    (``ltxa_attn_fwd_unpack_log2q``).
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _gpu(t, name, torch.bfloat16)
    if q.dim() != 5:
        raise ValueError("q must be [P, B, Nq, H/P, D]")
    P, B, Nq, Hl, D = q.shape
    Nk = k.shape[2]
    if k.shape != (P, B, Nk, Hl, D) or v.shape != k.shape:
        raise ValueError("k and v must be [P, B, Nk, H/P, D] matching q")
    nk_valid = Nk if nk_valid is None else int(nk_valid)
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, Nq, P * Hl, D), dtype=q.dtype, device=q.device)
    _gpu(out, "out", torch.bfloat16)
    if out.shape != (B, Nq, P * Hl, D):
        raise ValueError("out must be [B, Nq, H, D]")
    lse_ptr = None
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
        if lse.shape != (P, B, Hl, Nq):
            raise ValueError("lse must be [P, B, H/P, Nq]")
        lse_ptr = lse.data_ptr()
    if q_log2:
        _check("ltxa_attn_fwd_unpack_log2q", lib().ltxa_attn_fwd_unpack_log2q(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, P * Hl, D, Nq, Nk,
            nk_valid, P, _stream_ptr(q)))
    else:
        _check("ltxa_attn_fwd_unpack", lib().ltxa_attn_fwd_unpack(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr, B, P * Hl, D, Nq, Nk,
            nk_valid, scale, P, _stream_ptr(q)))
    return out


class SpShare:
    """Bookkeeping and exchange buffers of one SP attention group held as
    ``world_size`` virtual ranks on one GPU (an ``AttentionManager`` analogue).

    It checks ``num_heads % world_size``, pads each step's sequence to a
    multiple of ``world_size`` (:meth:`set_seqlen`) and owns the per-rank
    receive buffers: Q, K, V head shards ``[P, B, N_pad, H/P, D]`` and the
    token-order output ``[B, N_pad, H, D]``.  They are allocated once, on
    first use, for ``ceil(max_tokens / world_size)`` tokens per rank (K/V
    buffers grow only if a call brings more keys, as cross-attention to a
    longer sequence can), and every later step reuses them.

    ``copy_out``: with ``False`` (the default) :func:`sp_attention` returns a
    view of the owned output buffer, valid until the next call on this share;
    with ``True`` it returns a tensor of its own.
    """

    _NAMES = ("q", "k", "v", "o_shards", "out")

    def __init__(self, max_tokens: int, num_heads: int, head_dim: int, world_size: int,
                 tensor_dtype: torch.dtype = torch.bfloat16, copy_out: bool = False):
        if max_tokens < 1 or num_heads < 1 or head_dim < 1 or world_size < 1:
            raise ValueError("max_tokens, num_heads, head_dim and world_size must be positive")
        if num_heads % world_size:
            raise ValueError(f"num_heads ({num_heads}) must be divisible by world_size ({world_size})")
        if tensor_dtype != torch.bfloat16:
            raise TypeError("the attention kernels take bfloat16 tensors")
        self.max_tokens = int(max_tokens)
        self.num_heads = int(num_heads)
        self.head_dim = int(head_dim)
        self.world_size = int(world_size)
        self.tensor_dtype = tensor_dtype
        self.copy_out = bool(copy_out)
        self.heads_per_rank = self.num_heads // self.world_size
        self.tokens_per_rank_max = -(-self.max_tokens // self.world_size)
        self.n_valid = 0
        self.n_pad = 0
        self._store = {}      # name -> flat device tensor

    def set_seqlen(self, n_valid: int) -> int:
        """Record this step's token count; returns the padded length."""
        if n_valid < 1:
            raise ValueError("the sequence must hold at least one token")
        if n_valid > self.max_tokens:
            raise ValueError(f"{n_valid} video tokens exceed max_tokens={self.max_tokens}: "
                             "use a smaller resolution or fewer frames")
        self.n_valid = int(n_valid)
        self.n_pad = -(-self.n_valid // self.world_size) * self.world_size
        return self.n_pad

    @property
    def tokens_per_rank(self) -> int:
        return self.n_pad // self.world_size

    def _view(self, name: str, shape, device) -> torch.Tensor:
        numel = 1
        for x in shape:
            numel *= int(x)
        buf = self._store.get(name)
        if buf is None or buf.numel() < numel or buf.device != torch.device(device):
            # First use: size for max_tokens (per rank ceil(max_tokens / P)
            # tokens from each of P ranks) at this batch size, or the request
            # if that is larger.
            B = int(shape[1]) if name in ("q", "k", "v", "o_shards") else int(shape[0])
            cap = B * self.tokens_per_rank_max * self.world_size * self.num_heads * self.head_dim
            buf = torch.empty(max(numel, cap), dtype=self.tensor_dtype, device=device)
            self._store[name] = buf
        return buf[:numel].view(*shape)

    def buffers(self, batch: int, device, nk: Optional[int] = None) -> dict:
        """Views of the owned buffers for this step (:meth:`set_seqlen` first):
        ``q``/``o_shards`` ``[P, B, n_pad, H/P, D]``, ``k``/``v``
        ``[P, B, nk, H/P, D]`` (``nk`` defaults to ``n_pad``) and ``out``
        ``[B, n_pad, H, D]``."""
        if self.n_pad < 1:
            raise ValueError("call set_seqlen before asking for buffers")
        P, Hl, D, N = self.world_size, self.heads_per_rank, self.head_dim, self.n_pad
        nk = N if nk is None else int(nk)
        return {"q": self._view("q", (P, batch, N, Hl, D), device),
                "k": self._view("k", (P, batch, nk, Hl, D), device),
                "v": self._view("v", (P, batch, nk, Hl, D), device),
                "o_shards": self._view("o_shards", (P, batch, N, Hl, D), device),
                "out": self._view("out", (batch, N, self.num_heads, D), device)}

    def rope_table_buffer(self, device) -> torch.Tensor:
        """A view of the owned float32 ``[n_pad, head_dim/2, 2]`` buffer for
        the step's angle table (:func:`rope_table`), sized on first use for
        ``ceil(max_tokens / world_size) * world_size`` tokens."""
        if self.n_pad < 1:
            raise ValueError("call set_seqlen before asking for buffers")
        half = max(self.head_dim // 2, 1)
        numel = self.n_pad * half * 2
        buf = self._store.get("rope_table")
        if buf is None or buf.numel() < numel or buf.device != torch.device(device):
            cap = self.tokens_per_rank_max * self.world_size * half * 2
            buf = torch.empty(max(numel, cap), dtype=torch.float32, device=device)
            self._store["rope_table"] = buf
        return buf[:numel].view(self.n_pad, half, 2)


def sp_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, share: "SpShare",
                 q_pos: torch.Tensor, q_max_pos, k_pos: Optional[torch.Tensor] = None,
                 k_max_pos=None, nk_valid: Optional[int] = None, theta: float = 10000.0,
                 scale: Optional[float] = None, fused: bool = True, prescale_q: bool = True,
                 q_rope_table: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One layer's SP attention for every virtual rank of ``share`` on one GPU.

    ``q``: token-major bf16 ``[B, N_pad, H, D]`` padded to ``share.n_pad``
    tokens; ``k``/``v``: ``[B, Nk_pad, H, D]`` (the same tensors' token count
    for self-attention).  Steps (SP page, "How the forward pass works"):
    exchange heads (``ltxa_sp_pack``) into the share's receive buffers,
    rotate Q/K (``ltxa_rope_qk``), attend over every valid key
    (``ltxa_attn_fwd``), shuffle back (``ltxa_sp_unpack``) into the share's
    output buffer and drop padded rows (a view).  Returns
    ``[B, share.n_valid, H, D]``: a view of the share's output buffer, or a
    copy with ``share.copy_out``.

    With ``fused`` (the default) the same steps take four launches: Q and K
    are exchanged and rotated in one pass each (``ltxa_sp_pack_rope``), V is
    exchanged, and attention writes token order directly
    (``ltxa_attn_fwd_unpack``).  With ``prescale_q`` (the default) the Q pass
    also multiplies by ``scale * log2(e)`` before its one rounding
    (``ltxa_sp_pack_rope_ex`` with ``out_scale``) and the attention takes those queries as
    given (``ltxa_attn_fwd_unpack_log2q``): Q is rounded once instead of
    twice.  With ``prescale_q=False`` the fused result is bit-identical to the
    unfused one.

    Self-attention (``k_pos`` absent or the same tensor as ``q_pos``, the same
    ``max_pos`` and token count) takes the fused path's table form, with the
    same result bit for bit: the angles of ``q_pos`` go into a table
    (``ltxa_rope_table``) and one launch exchanges and rotates Q and K with it
    (``ltxa_sp_pack_rope_qk_table``).  ``q_rope_table`` is such a table made
    by the caller (:func:`rope_table`, default options), once per forward
    pass for every layer, as the pages precompute the rotary frequencies;
    without it the table is built into the share's buffer on each call.
    For cross-attention such a table rotates Q alone.
    """
    P = share.world_size
    B, N, H, D = q.shape
    Nk = k.shape[1]
    if N != share.n_pad or H != share.num_heads or D != share.head_dim:
        raise ValueError("q must be [B, share.n_pad, num_heads, head_dim]")
    same_angles = ((k_pos is None or k_pos is q_pos) and Nk == N and
                   (k_max_pos is None or [float(x) for x in k_max_pos] == [float(x) for x in q_max_pos]))
    k_pos = q_pos if k_pos is None else k_pos
    k_max_pos = q_max_pos if k_max_pos is None else k_max_pos
    nk_valid = share.n_valid if nk_valid is None else nk_valid
    Hl = H // P
    buf = share.buffers(B, q.device, nk=Nk)
    qs, ks, vs, out = buf["q"], buf["k"], buf["v"], buf["out"]
    if fused:
        c = log2_domain_scale((1.0 / D ** 0.5) if scale is None else float(scale)) if prescale_q else 0.0
        if same_angles:
            table = q_rope_table
            if table is None:
                table = rope_table(q_pos, q_max_pos, D, theta, out=share.rope_table_buffer(q.device))
            sp_pack_rope_qk_table(q, k, table, P, q_scale=c, q_out=qs, k_out=ks)
        else:
            if q_rope_table is not None:
                sp_pack_rope_table(q, q_rope_table, P, out_scale=c, out=qs)
            else:
                sp_pack_rope(q, q_pos, q_max_pos, P, theta, out=qs, out_scale=c if prescale_q else None)
            sp_pack_rope(k, k_pos, k_max_pos, P, theta, out=ks)
        sp_pack(v, P, out=vs)
        attn_fwd_unpack(qs, ks, vs, nk_valid=nk_valid, scale=scale, out=out, q_log2=prescale_q)
    else:
        sp_pack(q, P, out=qs)
        sp_pack(k, P, out=ks)
        sp_pack(v, P, out=vs)
        rope_qk(qs.view(P * B, N, Hl, D), q_pos, q_max_pos, ks.view(P * B, Nk, Hl, D), k_pos, k_max_pos, theta)
        os_ = buf["o_shards"]
        attn_fwd(qs.view(P * B, N, Hl, D), ks.view(P * B, Nk, Hl, D), vs.view(P * B, Nk, Hl, D),
                 nk_valid=nk_valid, scale=scale, out=os_.view(P * B, N, Hl, D))
        sp_unpack(os_, out=out)
    res = out[:, :share.n_valid]
    return res.clone() if share.copy_out else res


def connector_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, max_pos,
                        nk_valid: Optional[int] = None, theta: float = 10000.0,
                        rope_type: str = "interleaved", fp64_angles: bool = False,
                        scale: Optional[float] = None, prescale_q: bool = True) -> torch.Tensor:
    """The attention core of the 1D text connector (FastVideo gemma page,
    ``Embeddings1DConnector.forward``): rotate Q and K in place by 1D
    positions with the grid over the inner dimension (all ``H`` heads,
    ``num_attention_heads = H``), then masked attention over every head.

    ``q``, ``k``, ``v``: bf16 ``[B, N, H, D]`` on one GPU (no sequence
    parallelism); ``pos``: int32 ``[N, 1]``; an additive mask with a valid
    prefix of ``nk_valid`` keys is ``nk_valid`` (default: all keys, as after
    the learnable registers replace the padding).  Returns ``[B, N, H, D]``.
    With ``prescale_q`` (the default) Q's rotation also multiplies by
    ``scale * log2(e)`` before its one rounding and the attention takes Q as
    given (``ltxa_attn_fwd_log2q``), so Q is rounded once; Q then holds those
    log2-domain values.
    """
    H, D = q.shape[2], q.shape[3]
    opts = rope_opts(rope_type=rope_type, grid_heads=H, fp64_angles=fp64_angles)
    c = log2_domain_scale((1.0 / D ** 0.5) if scale is None else float(scale)) if prescale_q else 0.0
    # Q and K share the positions: one launch evaluates each angle once for both.
    rope_qk_ex(q, k, pos, max_pos, theta, opts=opts, q_scale=c)
    return attn_fwd(q, k, v, nk_valid=nk_valid, scale=scale, q_log2=prescale_q)

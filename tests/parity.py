"""Comparison helpers shared by the GPU parity tests (no GPU needed to import)."""

import numpy as np
import torch

# Acceptance bar for bf16 attention outputs on unit-variance inputs, over
# valid query rows, all heads and channels.
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
# Extra bars of this library (the output std at 32k keys is ~0.009, so the
# absolute bars alone are loose): relative RMS error and cosine similarity.
ATTN_REL_RMS = 1e-2
ATTN_COSINE = 0.9999
# Unit roundoffs: bfloat16 keeps 8 significant bits, float32 24.
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24
LOG2E = 1.4426950408889634


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor (CPU numpy uint16)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def attn_errors(got: np.ndarray, want: np.ndarray) -> dict:
    d = got - want
    rms_ref = float(np.sqrt(np.mean(want ** 2)))
    cos = float(np.sum(got * want) / (np.linalg.norm(got) * np.linalg.norm(want)))
    return {
        "max_abs": float(np.max(np.abs(d))),
        "mean_abs": float(np.mean(np.abs(d))),
        "rel_rms": float(np.sqrt(np.mean(d ** 2)) / rms_ref),
        "cosine": cos,
    }


def assert_attn_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    e = attn_errors(got, want)
    msg = f"{what}: {e}"
    assert e["max_abs"] <= ATTN_MAX_ABS, msg
    assert e["mean_abs"] <= ATTN_MEAN_ABS, msg
    assert e["rel_rms"] <= ATTN_REL_RMS, msg
    assert e["cosine"] >= ATTN_COSINE, msg
    return e


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest-even bfloat16, returned as float64."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rope_ok(got: np.ndarray, ref: np.ndarray, x: np.ndarray):
    """Rotary acceptance: within 1 bf16 ulp of the exact result, or within
    the fp32 computation bound 2^-20 * (|x0| + |x1|) of the pair (this covers
    results that are tiny through cancellation).  Returns (ok mask, fraction
    exactly equal to the exact result rounded to bf16)."""
    mag = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    mag = np.repeat(mag, 2, axis=-1)
    d = np.abs(got - ref)
    ok = (d <= bf16_ulp(ref)) | (d <= 2.0 ** -20 * mag)
    exact = float(np.mean(got == bf16_round(ref)))
    return ok, exact


def kernel_scaled_q(q: np.ndarray, scale: float) -> np.ndarray:
    """The attention kernel's documented rounding of q (include/ltxa.h,
    ltxa_attn_fwd "Arithmetic"): c = fp32(scale * log2 e), the product
    fp32(q * c), rounded once to bf16.  Returned in log2-score units divided
    back by log2 e (float64), so that ``kernel_scaled_q(q, s) @ k.T`` is the
    natural-log score the kernel works with, before accumulation error."""
    c = np.float32(scale * LOG2E)
    prod = (q.astype(np.float32) * c).astype(np.float32)
    return bf16_round(prod.astype(np.float64)) / LOG2E


def attn_error_bounds(q: np.ndarray, k: np.ndarray, v: np.ndarray, nk_valid: int, scale: float,
                      rows=None, q_prerounded: bool = False):
    """Per-row LSE bound and per-element output bound of ltxa_attn_fwd against
    the exact attention of the same bf16 inputs (``oracle.attention``),
    derived from the kernel's arithmetic as include/ltxa.h states it.

    With c = scale * log2(e), A_ij = sum_d |q_id k_jd| (valid keys j) and
    T = ceil(nk_valid / 64) key tiles, the kernel's log-weight of key j in row
    i differs from the exact scale * <q_i, k_j> (up to a shift common to the
    row) by at most
        delta_i = scale * A_i * (U_BF16 (1 + 2^-14) + 2 D U_F32)   q rounded to bf16 once (c and
                                                                  the product in fp32), fp32
                                                                  accumulation of D products
                  - ln(1 - U_BF16) + 4 U_F32                      fp32 exp2; the probabilities
                                                                  weighting V rounded to bf16
                                                                  (the row sum adds them
                                                                  unrounded, which this covers)
    where A_i = max_j A_ij (``q_prerounded``: q already carries the
    kernel's rounding, so the first term drops to the accumulation part).
    Every weight w_j = p_j / sum p then moves by a factor in
    [e^{-2 delta}, e^{2 delta}], the log of the row sum by at most delta, and:
        |lse - exact| <= delta_i + (T + 20) U_F32 + 8 U_F32 (|lse| + 1)
        |o_d - exact| <= ((e^{2 delta_i} - 1) + (5 T + 20) U_F32 e^{2 delta_i}) W_id
                         + U_BF16 (|o_d| + that)
    with W_id = sum_j w_ij |v_jd| (the oracle's weights applied to |v|);
    (T + 20) U_F32 and (5 T + 20) U_F32 cover the fp32 row-sum and P*V
    accumulations (at most 16 keys per chain step, one step per tile and
    rescale) and the final reciprocal; U_BF16 |o| is the output rounding.
    These are worst-case bounds (every rounding error aligned), not
    expected errors.

    Returns ``(lse_bound [B, H, R], o_bound [B, R, H, D], o_exact, lse_exact)``.
    """
    import oracle  # test infrastructure
    B, Nq, H, D = q.shape
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    o_ex, lse_ex = oracle.attention(q, k, v, nk_valid, scale, rows=row_idx)
    w_abs_v, _ = oracle.attention(q, k, np.abs(v), nk_valid, scale, rows=row_idx)
    T = -(-nk_valid // 64)
    a_max = np.empty((B, H, len(row_idx)))
    for b in range(B):
        for h in range(H):
            Kabs = np.abs(k[b, :nk_valid, h, :])
            for r0 in range(0, len(row_idx), 1024):
                sel = row_idx[r0:r0 + 1024]
                a_max[b, h, r0:r0 + len(sel)] = (np.abs(q[b, sel, h, :]) @ Kabs.T).max(axis=1)
    q_term = 0.0 if q_prerounded else U_BF16 * (1.0 + 2.0 ** -14)
    delta = scale * a_max * (q_term + 2.0 * D * U_F32) - np.log1p(-U_BF16) + 4.0 * U_F32
    lse_bound = delta + (T + 20) * U_F32 + 8.0 * U_F32 * (np.abs(lse_ex) + 1.0)
    d_o = np.transpose(delta, (0, 2, 1))[..., None]              # [B, R, H, 1]
    grow = np.exp(2.0 * d_o)
    o_core = ((grow - 1.0) + (5 * T + 20) * U_F32 * grow) * w_abs_v
    o_bound = o_core + U_BF16 * (np.abs(o_ex) + o_core)
    return lse_bound, o_bound, o_ex, lse_ex


def assert_within_model(got_o: np.ndarray, got_lse, q, k, v, nk_valid, scale, rows=None,
                        what: str = "", q_prerounded: bool = False):
    """Assert the kernel's output (and LSE, if given) against the exact
    attention within :func:`attn_error_bounds`.  Returns the worst ratio of
    error to bound for the output and the LSE (each must be <= 1)."""
    lse_b, o_b, o_ex, lse_ex = attn_error_bounds(q, k, v, nk_valid, scale, rows, q_prerounded)
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    r_o = float(np.max(np.abs(got_o - o_ex) / o_b))
    assert r_o <= 1.0, f"{what}: output error exceeds the model bound (worst ratio {r_o:.3f})"
    r_l = None
    if got_lse is not None:
        r_l = float(np.max(np.abs(got_lse - lse_ex) / lse_b))
        assert r_l <= 1.0, f"{what}: lse error exceeds the model bound (worst ratio {r_l:.3f})"
    return r_o, r_l

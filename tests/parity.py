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
# Log-sum-exp: the kernel's row sum adds the bf16-rounded probabilities (the
# same values that weight V), each within a relative 2^-9 of the exact one,
# so the sum is within a relative 2^-9 and its log within ~2^-9 ~= 2e-3
# (plus fp32 rounding, ~1e-6).  Bar: twice that.
LSE_ABS = 4e-3


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

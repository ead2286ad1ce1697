"""Row operations of the oracle: FP16 residual sum and fixed-width LayerNorm.

TEST INFRASTRUCTURE (see the package docstring): float64 numpy, slow and plain.
"""
from __future__ import annotations

import numpy as np

# LayerNorm epsilon; the pages give none, 1e-5 is the framework default that the
# replaced native_layer_norm calls used.
EPS = 1e-5
# Section 3 of the BW1000 page: the model's hidden widths are 192 and 384, and
# any width without its own tests is refused rather than served by an untested
# path. 768 is the patch-merge width of the same model (four neighbouring
# 192-channel tokens concatenated before the merge), added with its own tests.
WIDTHS = (192, 384, 768)


def fp16_round(values) -> np.ndarray:
    """Round float64 values to IEEE binary16, to nearest with ties to even
    (overflow goes to +-inf, NaN stays NaN)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(values, dtype=np.float64).astype(np.float16)


def residual_sum(residual: np.ndarray, branch: np.ndarray) -> np.ndarray:
    """FP16 residual of section 4 (fused residual add + norm) of the BW1000 page:
    residual <- FP16(residual + branch), one rounding of the exact sum.

    Two binary16 values have 11-bit significands with exponents in [-24, 15], so
    their sum is exact in float64 (at most 40 significant bits); the only
    rounding is the final cast."""
    r = np.asarray(residual, dtype=np.float16).astype(np.float64)
    b = np.asarray(branch, dtype=np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return fp16_round(r + b)


def layer_norm(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """Fixed-width LayerNorm of section 3 of the BW1000 page, per row of ``[rows, C]``:
    mean over the row, biased variance of the deviations (divide by C), then
    (x - mean) / sqrt(var + eps), rounded once to binary16. No scale and no
    shift: the page folds the affine parameters into the next Linear at load time.

    Statistics are taken in float64 from the binary16 inputs; a row holding
    Inf or NaN gives a NaN row."""
    a = np.asarray(x, dtype=np.float16)
    if a.ndim != 2 or a.shape[1] not in WIDTHS:
        raise ValueError(f"layer_norm expects [rows, C] with C in {WIDTHS}, got {a.shape}")
    v = a.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        mean = v.mean(axis=1, keepdims=True)
        dev = v - mean
        var = (dev * dev).mean(axis=1, keepdims=True)
        y = dev / np.sqrt(var + eps)
    return fp16_round(y)


def add_ln(branch: np.ndarray, residual: np.ndarray, eps: float = EPS):
    """Section 4 of the BW1000 page: the FP16 residual sum is written out, and the
    LayerNorm reads that rounded residual. Returns (residual_out, y)."""
    r = residual_sum(residual, branch)
    return r, layer_norm(r, eps)


def layer_norm_affine(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = EPS) -> np.ndarray:
    """LayerNorm with a per-channel scale and shift, for callers that do not fold
    the affine parameters into the next Linear (section 3 of the BW1000 page
    folds them; this is the unfolded form): y = (x - mean) / sqrt(var + eps) *
    gamma + beta, computed in float64 from binary16 x, gamma and beta, rounded
    once to binary16."""
    a = np.asarray(x, dtype=np.float16)
    if a.ndim != 2 or a.shape[1] not in WIDTHS:
        raise ValueError(f"layer_norm_affine expects [rows, C] with C in {WIDTHS}, got {a.shape}")
    g = np.asarray(gamma, dtype=np.float16).astype(np.float64).reshape(1, -1)
    b = np.asarray(beta, dtype=np.float16).astype(np.float64).reshape(1, -1)
    if g.shape[1] != a.shape[1] or b.shape[1] != a.shape[1]:
        raise ValueError("gamma and beta must have one entry per channel")
    v = a.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        mean = v.mean(axis=1, keepdims=True)
        dev = v - mean
        var = (dev * dev).mean(axis=1, keepdims=True)
        y = dev / np.sqrt(var + eps) * g + b
    return fp16_round(y)


def add_ln_affine(branch: np.ndarray, residual: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                  eps: float = EPS):
    """Residual add (section 4) followed by the affine LayerNorm. Returns (residual_out, y)."""
    r = residual_sum(residual, branch)
    return r, layer_norm_affine(r, gamma, beta, eps)

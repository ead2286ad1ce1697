"""Bias + tanh-approximated GELU of the oracle.

TEST INFRASTRUCTURE (see the package docstring). The operation is the fused
bias + GELU of the page "PyTorch + HIP custom fused operator" (Hygon DCU
practice series), sections 3-6: input [rows, hidden] float32 plus a bias
[hidden] float32, then the tanh form of GELU,
0.5 * x * (1 + tanh(sqrt(2/pi) * (x + 0.044715 * x^3))). The page's eager
reference adds the bias as its own float32 tensor operation, so the sum is
rounded to float32 once before the activation.
"""
from __future__ import annotations

import numpy as np

GELU_K0 = np.sqrt(2.0 / np.pi)
GELU_K1 = 0.044715


def bias_gelu(x: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """float32 result of gelu_tanh(float32(x + bias)); the activation itself is
    evaluated in float64 and rounded once."""
    a = np.asarray(x, dtype=np.float32)
    b = np.asarray(bias, dtype=np.float32)
    if a.ndim != 2 or b.shape != (a.shape[1],):
        raise ValueError("bias_gelu expects x [rows, hidden] and bias [hidden]")
    with np.errstate(over="ignore", invalid="ignore"):
        t = (a + b[None, :]).astype(np.float64)          # float32 add, exactly rounded
        y = 0.5 * t * (1.0 + np.tanh(GELU_K0 * (t + GELU_K1 * t ** 3)))
    return y.astype(np.float32)

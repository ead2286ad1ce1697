"""Window index tables and gathers of the oracle.

TEST INFRASTRUCTURE (see the package docstring): plain numpy, no blocking or
fusion. The table follows the steps of a shifted-window transformer in their
natural order -- pad the token grid, shift it cyclically, cut it into windows --
with the padding carried as index -1, as section 5 of the page "Pangu-Weather
inference optimisation on Hygon BW1000 (gfx936)" describes (an INT32 index per
gathered token, padding folded into the index protocol).

Readings of what the page leaves open (each also listed in the design notes):
* padding goes at the high end of each axis, up to the next multiple of the
  window extent;
* the cyclic shift is applied to the padded grid, after padding; a shift s
  moves content toward lower indices (gathered position p reads padded
  position (p + s) mod P), shifts are taken modulo the padded extent;
* windows are ordered row-major over (z, h, w) window coordinates, tokens inside
  a window row-major over (dz, dh, dw); the gathered tensor is [windows, wz*wh*ww, C]
  flattened to rows;
* an index outside [0, n_src) -- -1 or any other -- yields a zero row (+0.0).
"""
from __future__ import annotations

import numpy as np

from .rowops import layer_norm


def padded_extent(extent: int, window: int) -> int:
    """Extent rounded up to a multiple of the window extent (high-end padding)."""
    return -(-extent // window) * window


def window_token_count(grid, window) -> int:
    """Rows of the gathered tensor: the product of the padded extents."""
    return int(np.prod([padded_extent(g, w) for g, w in zip(grid, window)]))


def window_index_table(grid, window, shift=(0, 0, 0)) -> np.ndarray:
    """INT32 table, one entry per gathered row: the source token index, or -1
    for a padding position.

    Steps: token ids of the (Z,H,W) grid (z slowest) -> pad each axis at the high
    end with -1 -> roll by -shift on each axis -> split into windows and list them
    window by window."""
    Z, H, W = grid
    wz, wh, ww = window
    if min(Z, H, W) < 1 or min(wz, wh, ww) < 1 or min(shift) < 0:
        raise ValueError("grid and window extents must be >= 1 and shifts >= 0")
    ids = np.arange(Z * H * W, dtype=np.int64).reshape(Z, H, W)
    pad = [(0, padded_extent(g, w) - g) for g, w in zip(grid, window)]
    padded = np.pad(ids, pad, mode="constant", constant_values=-1)
    rolled = np.roll(padded, shift=tuple(-s for s in shift), axis=(0, 1, 2))
    Zp, Hp, Wp = padded.shape
    windows = rolled.reshape(Zp // wz, wz, Hp // wh, wh, Wp // ww, ww)
    windows = windows.transpose(0, 2, 4, 1, 3, 5)
    return np.ascontiguousarray(windows.reshape(-1)).astype(np.int32)


def window_gather(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Section 5 of the BW1000 page: row j of the output is x[table[j]] when the
    entry is a valid source index, otherwise a row of +0.0."""
    x = np.asarray(x, dtype=np.float16)
    table = np.asarray(table, dtype=np.int64)
    out = np.zeros((table.shape[0], x.shape[1]), dtype=np.float16)
    valid = (table >= 0) & (table < x.shape[0])
    out[valid] = x[table[valid]]
    return out


def norm_gather(x: np.ndarray, table: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """Section 5 of the BW1000 page (norm-gather): norm1's output is only ever
    gathered, so the result is the gather of the LayerNorm of x."""
    return window_gather(layer_norm(x, eps), table)


def norm_gather_rows(x: np.ndarray, table: np.ndarray, rows: np.ndarray,
                     eps: float = 1e-5) -> np.ndarray:
    """Selected output rows of ``norm_gather`` (for checks at full size):
    row j is LayerNorm(x[table[j]]) for a valid entry, else +0.0."""
    x = np.asarray(x, dtype=np.float16)
    t = np.asarray(table, dtype=np.int64)[np.asarray(rows, dtype=np.int64)]
    out = np.zeros((t.shape[0], x.shape[1]), dtype=np.float16)
    valid = (t >= 0) & (t < x.shape[0])
    if valid.any():
        out[valid] = layer_norm(x[t[valid]], eps)
    return out

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


def window_reverse(rows: np.ndarray, grid, window, shift=(0, 0, 0)) -> np.ndarray:
    """Undo the window partition: the gathered rows [M, C] (window-major) are put
    back on the padded grid, rolled back by +shift, and the padding is cropped,
    giving [Z*H*W, C] in token order. This is the step that follows attention in a
    shifted-window block; the pages describe only the forward gather, so the
    reverse is read as the forward steps undone in the opposite order."""
    Z, H, W = grid
    wz, wh, ww = window
    Zp, Hp, Wp = (padded_extent(g, w) for g, w in zip(grid, window))
    rows = np.asarray(rows)
    c = rows.shape[1]
    if rows.shape[0] != Zp * Hp * Wp:
        raise ValueError("row count differs from the window token count")
    g = rows.reshape(Zp // wz, Hp // wh, Wp // ww, wz, wh, ww, c)
    g = g.transpose(0, 3, 1, 4, 2, 5, 6).reshape(Zp, Hp, Wp, c)
    g = np.roll(g, shift=tuple(shift), axis=(0, 1, 2))
    return np.ascontiguousarray(g[:Z, :H, :W].reshape(Z * H * W, c))


def window_inverse_table(grid, window, shift=(0, 0, 0)) -> np.ndarray:
    """INT32 table, one entry per source token: the gathered row that holds it.
    Obtained by running window_reverse on the column of gathered-row numbers."""
    m = window_token_count(grid, window)
    ids = np.arange(m, dtype=np.int64)[:, None]
    return window_reverse(ids, grid, window, shift)[:, 0].astype(np.int32)


def window_reverse_add_ln(rows: np.ndarray, residual: np.ndarray, grid, window, shift=(0, 0, 0),
                          eps: float = 1e-5):
    """Window reverse of the attention output used as the branch of the residual
    add + LayerNorm of section 4 of the BW1000 page: returns (FP16(residual +
    reversed rows), LayerNorm of that)."""
    from .rowops import add_ln
    branch = window_reverse(np.asarray(rows, dtype=np.float16), grid, window, shift)
    return add_ln(branch, residual, eps)


def add_norm_gather(branch: np.ndarray, residual: np.ndarray, table: np.ndarray, eps: float = 1e-5):
    """Residual add + LayerNorm + window gather: the FP16 residual sum of section 4
    of the BW1000 page is written out, and its LayerNorm is only ever gathered
    (section 5). Returns (residual_out, gathered rows)."""
    from .rowops import residual_sum
    r = residual_sum(residual, branch)
    return r, norm_gather(r, table, eps)

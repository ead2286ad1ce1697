"""Seeded synthetic inputs for the row pipeline (shared by tests, bench and smoke).

This module only draws random numbers and casts them to IEEE binary16. It holds
none of the method's arithmetic: no LayerNorm, no residual sum, no padding or
window rule. The oracle and the HIP path both receive exactly the arrays built
here, so the two sides see the same bits.

The shapes are those of the Pangu-Weather student model as measured on the
page "Pangu-Weather inference optimisation on Hygon BW1000 (gfx936)"
(l189.com/news/2144533), section 3 (LayerNorm microbenchmark table: [1,131040,192]
and [1,32760,384]) and section 5 (shifted-window gather). The pages publish no
activations, so the value distributions below are stand-ins; each recipe is
stated in its docstring.

Every array is drawn in float64 with numpy's PCG64 ``default_rng(seed)`` and cast
to float16 with ``astype`` (round to nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

EPS = 1e-5


@dataclass(frozen=True)
class Level:
    """One hidden width of the model with the token grid it runs on."""

    name: str
    grid: tuple  # (Z, H, W) token grid, z slowest
    channels: int

    @property
    def tokens(self) -> int:
        z, h, w = self.grid
        return z * h * w


# Level 1: [1,131040,192] on an 8 x 182 x 90 grid; level 2: [1,32760,384] on 8 x 91 x 45.
LEVEL1 = Level("level1", (8, 182, 90), 192)
LEVEL2 = Level("level2", (8, 91, 45), 384)
# Patch merging from level 1 to level 2 normalises 4 x 192 = 768 concatenated
# channels of each merged token, on the level-2 grid.
PATCH_MERGE = Level("patch_merge", (8, 91, 45), 768)
# The tiny case: a 2 x 12 x 24 grid, exactly four (2,6,12) windows with no padding.
TINY = Level("tiny", (2, 12, 24), 192)

WINDOW = (2, 6, 12)
SHIFT = (1, 3, 6)
NO_SHIFT = (0, 0, 0)


def _f16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.astype(np.float16))


def normal_rows(seed: int, rows: int, channels: int, mean: float = 0.0,
                std: float = 1.0) -> np.ndarray:
    """``[rows, channels]`` float16 drawn i.i.d. from N(mean, std**2)."""
    rng = np.random.default_rng(seed)
    return _f16(rng.normal(mean, std, size=(rows, channels)))


def tiny_inputs(seed: int = 0):
    """Tiny case: x and residual i.i.d. N(0,1), 576 x 192."""
    rng = np.random.default_rng(seed)
    n, c = TINY.tokens, TINY.channels
    x = _f16(rng.normal(0.0, 1.0, size=(n, c)))
    residual = _f16(rng.normal(0.0, 1.0, size=(n, c)))
    return x, residual


def level1_inputs(seed: int = 1):
    """Level-1 standalone: x ~ N(0,1) (also the add_ln branch), residual ~ N(0, 0.5**2)."""
    rng = np.random.default_rng(seed)
    n, c = LEVEL1.tokens, LEVEL1.channels
    x = _f16(rng.normal(0.0, 1.0, size=(n, c)))
    residual = _f16(rng.normal(0.0, 0.5, size=(n, c)))
    return x, residual


def level2_inputs(seed: int = 2):
    """Level-2 standalone: x ~ N(0.5, 2**2) with floor(1% of rows) seeded rows
    multiplied by 50 before the cast (a large-variance stress); residual ~ N(0, 0.5**2).
    Returns (x, residual, scaled_row_indices)."""
    rng = np.random.default_rng(seed)
    n, c = LEVEL2.tokens, LEVEL2.channels
    x = rng.normal(0.5, 2.0, size=(n, c))
    scaled = np.sort(rng.choice(n, size=n // 100, replace=False))
    x[scaled] *= 50.0
    residual = rng.normal(0.0, 0.5, size=(n, c))
    return _f16(x), _f16(residual), scaled


def fused_level1_inputs(seed: int = 3):
    """Fused norm_gather at level 1: x ~ N(0,1), 131040 x 192."""
    return normal_rows(seed, LEVEL1.tokens, LEVEL1.channels)


def stress_row_classes(seed: int, rows: int):
    """Pick disjoint row sets for the block-stack replay: floor(1%) near-constant
    rows and floor(1%) offset-mean rows. Returns (near_constant_idx, offset_idx)."""
    rng = np.random.default_rng(seed)
    k = rows // 100
    picked = rng.choice(rows, size=2 * k, replace=False)
    return np.sort(picked[:k]), np.sort(picked[k:])


def mixed_rows(seed: int, rows: int, channels: int, near_constant: np.ndarray,
               offset: np.ndarray, offset_mean: float = 100.0) -> np.ndarray:
    """Rows N(0,1), except near-constant rows c + 1e-3*z (c ~ N(0,1) per row,
    z ~ N(0,1)) and offset rows offset_mean + z. ``offset_mean=0`` gives plain
    N(0,1) rows there (used for the replay's branch tensors so that the offset
    rows keep a mean near 100 through the residual stream)."""
    rng = np.random.default_rng(seed)
    a = rng.normal(0.0, 1.0, size=(rows, channels))
    c = rng.normal(0.0, 1.0, size=(len(near_constant), 1))
    z = rng.normal(0.0, 1.0, size=(len(near_constant), channels))
    a[near_constant] = c + 1e-3 * z
    a[offset] = offset_mean + rng.normal(0.0, 1.0, size=(len(offset), channels))
    return _f16(a)


@dataclass(frozen=True)
class ReplayCall:
    """One call of the block-stack replay."""

    op: str          # "ln_fixed" | "norm_gather" | "add_ln"
    level: Level
    shift: tuple     # window shift for norm_gather, else NO_SHIFT
    seed: int        # seed of the branch tensor for add_ln, else -1


def replay_schedule(blocks: int = 32):
    """The 66-call block-stack replay: one ln_fixed per level, then for each block
    b a norm_gather followed by an add_ln (residual updated in place). Block b runs
    at level 1 when b is even, else level 2; its window is shifted by (1,3,6) when
    floor(b/2) is odd. Gives 34 LayerNorm-family calls and 32 norm_gather calls."""
    calls = [ReplayCall("ln_fixed", LEVEL1, NO_SHIFT, -1),
             ReplayCall("ln_fixed", LEVEL2, NO_SHIFT, -1)]
    for b in range(blocks):
        level = LEVEL1 if b % 2 == 0 else LEVEL2
        shift = SHIFT if (b // 2) % 2 == 1 else NO_SHIFT
        calls.append(ReplayCall("norm_gather", level, shift, -1))
        calls.append(ReplayCall("add_ln", level, NO_SHIFT, 4 + b))
    return calls


def replay_streams(seed: int = 4):
    """Initial residual streams of the replay, one per level, with the stress
    row classes. Returns {level name: (stream, near_constant_idx, offset_idx)}."""
    out = {}
    for k, level in enumerate((LEVEL1, LEVEL2)):
        nc, off = stress_row_classes(seed * 10 + k, level.tokens)
        out[level.name] = (mixed_rows(seed * 100 + k, level.tokens, level.channels, nc, off),
                           nc, off)
    return out


def replay_branch(call: ReplayCall, near_constant: np.ndarray, offset: np.ndarray) -> np.ndarray:
    """Branch tensor of a replay add_ln call: the same row classes as the stream,
    with offset rows drawn around 0 so the stream's offset rows keep their mean."""
    lv = call.level
    return mixed_rows(call.seed, lv.tokens, lv.channels, near_constant, offset, offset_mean=0.0)


# Grids whose tensors pass 2**31 elements and 2**32 bytes (64-bit offsets),
# with ragged extents so the window tables pad at both levels' widths.
LARGE_192 = Level("large_192", (8, 1093, 1297), 192)   # 11,340,968 rows, 4.35 GB
LARGE_384 = Level("large_384", (4, 1093, 1297), 384)   # 5,670,484 rows, 4.35 GB


def id_tagged_rows(seed: int, rows: int, channels: int, block: int = 4096) -> np.ndarray:
    """``[rows, channels]`` float16 whose rows are all distinct and carry their own
    index: columns 0..2 hold the base-1024 digits of the row index (exact binary16
    integers, least significant first), column 3 holds 1.0 as a marker, and
    columns 4.. repeat a block of ``block`` i.i.d. N(0,1) rows. Built in place,
    block by block, so a multi-GB array costs one pass over memory."""
    rng = np.random.default_rng(seed)
    base = _f16(rng.normal(0.0, 1.0, size=(block, channels)))
    out = np.empty((rows, channels), np.float16)
    for s in range(0, rows, block):
        e = min(rows, s + block)
        out[s:e] = base[: e - s]
    ids = np.arange(rows, dtype=np.int64)
    out[:, 0] = ids % 1024
    out[:, 1] = (ids >> 10) % 1024
    out[:, 2] = ids >> 20
    out[:, 3] = 1.0
    return out


def gelu_inputs(seed: int, rows: int, cols: int):
    """float32 ``x`` [rows, cols] and ``bias`` [cols], both i.i.d. N(0,1) drawn
    in float64 and rounded to float32 (the bias + GELU operator takes float32)."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(rows, cols)).astype(np.float32)
    bias = rng.normal(0.0, 1.0, size=cols).astype(np.float32)
    return x, bias


def fp16_bit_pattern_pairs(seed: int, rows: int, cols: int):
    """(residual, branch) float16 [rows, cols] with every bit pattern possible:
    uniformly random 16-bit words (so subnormals, infinities and NaNs occur),
    and on even rows a branch within a few ulps of the negated residual, so that
    sums cancel and land on subnormals and zeros."""
    rng = np.random.default_rng(seed)
    res = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    br = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    near = (res[::2].astype(np.int32) ^ 0x8000) + rng.integers(-3, 4, size=(len(res[::2]), cols))
    br[::2] = near.astype(np.uint16)
    return res.view(np.float16), br.view(np.float16)


def table_with_bad_entries(seed: int, n_out: int, n_src: int) -> np.ndarray:
    """int32 [n_out] gather table of random entries in [-1, n_src), with entries
    outside [0, n_src) planted at fixed strides: n_src, -5, INT32_MIN, INT32_MAX."""
    rng = np.random.default_rng(seed)
    table = rng.integers(-1, n_src, size=n_out).astype(np.int32)
    table[::7] = n_src
    table[::11] = -5
    table[::13] = np.iinfo(np.int32).min
    table[::17] = np.iinfo(np.int32).max
    return table

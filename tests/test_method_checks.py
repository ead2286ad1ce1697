"""CPU checks of the arithmetic methods the kernels rely on (not of the kernels
themselves, which the GPU tests compare with the oracle).

Narrowing binary64 to binary16 in one rounding: the kernels cut the binary64
value to binary32 with round-to-odd (keep the top 23 fraction bits, OR a sticky
bit for the 29 dropped ones), then round that to binary16 to nearest-even.
binary32 keeps 13 bits beyond binary16, more than the 2 extra bits round-to-odd
needs, so the two steps must equal a direct correctly rounded conversion. Here
the bit manipulation is redone in numpy and compared with numpy's own
float64 -> float16 conversion (correctly rounded) on values chosen to sit on,
and a hair off, every kind of binary16 rounding boundary.
"""
import numpy as np


def two_step(y: np.ndarray) -> np.ndarray:
    b = y.view(np.uint64)
    low29 = b & np.uint64(0x1FFFFFFF)
    sticky = ((low29 + np.uint64(0x1FFFFFFF)) & np.uint64(0x20000000))
    t = (b & np.uint64(0xFFFFFFFFE0000000)) | sticky
    with np.errstate(over="ignore"):
        return t.view(np.float64).astype(np.float32).astype(np.float16)


def boundary_values(rng) -> np.ndarray:
    """binary16 values, the midpoints between neighbours, and points a few
    binary64 ulps either side of each midpoint, across normal and subnormal
    binary16 and the overflow threshold; plus random doubles of every
    magnitude near the binary16 range."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)   # +0 .. 65504
    mids = (h[:-1] + h[1:]) / 2                                                        # exact in binary64
    mids = np.concatenate([mids, [65520.0]])                                           # 65504 / +Inf midpoint
    off = []
    for k in (1, 2, 3, 1 << 20, 1 << 28, 1 << 29, (1 << 29) + 1):
        off.append(np.nextafter(mids, np.inf) if k == 1 else mids * (1 + k * 2.0 ** -52))
        off.append(np.nextafter(mids, -np.inf) if k == 1 else mids * (1 - k * 2.0 ** -52))
    rand = rng.standard_normal(400_000) * np.exp2(rng.uniform(-30, 17, 400_000))
    v = np.concatenate([h, mids, *off, rand])
    return np.concatenate([v, -v, [np.inf, -np.inf, np.nan, 0.0, -0.0, 1e300, -1e300, 1e-300]])


def test_round_to_odd_binary32_then_binary16_is_one_correct_rounding():
    rng = np.random.default_rng(20260716)
    y = boundary_values(rng)
    with np.errstate(over="ignore", invalid="ignore"):
        direct = y.astype(np.float16)
    got = two_step(y)
    nan = np.isnan(direct)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.flatnonzero(got[~nan].view(np.uint16) != direct[~nan].view(np.uint16))
    assert bad.size == 0, f"{bad.size} values differ, e.g. {y[~nan][bad[:5]]}"


def test_plain_double_rounding_would_be_wrong():
    """The same values cut to binary32 with nearest-even instead of round-to-odd
    disagree with the direct conversion somewhere, so the test above can tell
    the two methods apart."""
    rng = np.random.default_rng(20260716)
    y = boundary_values(rng)
    with np.errstate(over="ignore", invalid="ignore"):
        direct = y.astype(np.float16)
        naive = y.astype(np.float32).astype(np.float16)
    ok = ~np.isnan(direct)
    assert (naive[ok].view(np.uint16) != direct[ok].view(np.uint16)).any()

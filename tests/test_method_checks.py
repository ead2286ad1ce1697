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


def test_one_newton_step_on_the_hardware_rsqrt_estimate():
    """rstd = 1/sqrt(var + eps) in the kernels is the hardware estimate r0
    refined once: r = r0 + r0*(1/2 - (a*r0/2)*r0), with two fused multiply-adds.
    From a relative error e the step leaves about -1.5 e^2. With the estimate
    good to 2^-22, the refined value is within 2^-40 of 1/sqrt(a), far below the
    2^-11 of a binary16 result, so the binary16 rounding of y is unaffected
    except within 2^-40 of a rounding midpoint. Checked here with estimates
    perturbed by +-2^-22 over the range of (var + eps) a row can give. (The
    gfx950 binary64 estimate, measured over 2^20 log-uniform arguments in
    [1e-5, 2^34], is off by at most 2^-24.2, inside the margin assumed here.)"""
    from fractions import Fraction
    rng = np.random.default_rng(20260716)
    a = np.concatenate([np.exp2(rng.uniform(np.log2(1e-5), 34, 2000)), [1e-5, 1.0, 2.0, 4.3e9]])

    def fma(x, y, z):      # one rounding, as the hardware fused multiply-add
        return float(Fraction(x) * Fraction(y) + Fraction(z))

    worst = 0.0
    for ai in a:
        exact = 1.0 / np.sqrt(np.float64(ai))
        for e in (2.0 ** -22, -(2.0 ** -22)):
            r0 = float(exact * (1 + e))
            h = 0.5 * ai * r0
            r = fma(r0, fma(-h, r0, 0.5), r0)
            rel = abs(Fraction(r) * Fraction(r) * Fraction(float(ai)) - 1)   # |r^2 a - 1| ~ 2 |rel. error|
            worst = max(worst, float(rel) / 2)
    assert worst < 2.0 ** -40, worst
    # a much worse estimate would not be enough after one step
    ai = 3.0
    r0 = float(1.0 / np.sqrt(ai) * (1 + 2.0 ** -12))
    r = fma(r0, fma(-0.5 * ai * r0, r0, 0.5), r0)
    assert abs(r * r * ai - 1) / 2 > 2.0 ** -26

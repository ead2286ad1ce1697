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


def fma(x, y, z):
    """One rounding of x*y + z, as the hardware fused multiply-add (exact
    rationals, then Python's correctly rounded int/int division)."""
    from fractions import Fraction
    return float(Fraction(x) * Fraction(y) + Fraction(z))


def newton(a, r):
    h = a * (0.5 * r)
    return fma(r, fma(-h, r, 0.5), r)


def test_two_newton_steps_on_the_hardware_rsqrt_estimate():
    """rstd = 1/sqrt(var + eps) in the kernels is the hardware estimate r0
    refined twice with r' = r + r*(1/2 - (a*r/2)*r), two fused multiply-adds
    per step (h = a*(r/2), so a subnormal a does not underflow). From a
    relative error e one step leaves about -1.5 e^2: from the
    estimate's 2^-22 (assumed here; the gfx950 binary64 estimate measured over
    2^20 log-uniform arguments in [1e-5, 2^34] is off by at most 2^-24.2) to
    below 2^-40 after the first step and to binary64's own rounding level after
    the second. Checked with estimates perturbed by +-2^-22 over the range of
    (var + eps) a row can give."""
    from fractions import Fraction
    rng = np.random.default_rng(20260716)
    a = np.concatenate([np.exp2(rng.uniform(np.log2(1e-5), 34, 1000)), [1e-5, 1.0, 2.0, 4.3e9, 5e-324]])

    def rel(r, ai):          # |r^2 a - 1| ~ 2 |relative error of r|
        return float(abs(Fraction(r) * Fraction(r) * Fraction(float(ai)) - 1)) / 2

    worst1 = worst2 = 0.0
    for ai in a:
        exact = 1.0 / np.sqrt(np.float64(ai))
        for e in (2.0 ** -22, -(2.0 ** -22)):
            r0 = float(exact * (1 + e))
            r1 = newton(ai, r0)
            worst1 = max(worst1, rel(r1, ai))
            worst2 = max(worst2, rel(newton(ai, r1), ai))
    assert worst1 < 2.0 ** -40, worst1
    assert worst2 < 2.0 ** -51, worst2
    # a much worse estimate would not be enough after one step
    ai = 3.0
    r0 = float(1.0 / np.sqrt(ai) * (1 + 2.0 ** -12))
    assert rel(newton(ai, r0), ai) > 2.0 ** -26


WIDTH_LANES = {192: (3, 8), 384: (6, 8), 768: (6, 16)}    # C -> (chunks per lane K, lanes per row)


def lane_order(x: np.ndarray, C: int) -> np.ndarray:
    """[rows, C] -> [rows, lanes, 8K]: the values each lane of a row holds, in
    the order it holds them (its chunks l, l + lanes, ..., 8 values each)."""
    K, L = WIDTH_LANES[C]
    ch = x.reshape(x.shape[0], C // 8, 8)
    return np.stack([ch[:, l::L].reshape(x.shape[0], 8 * K) for l in range(L)], axis=1)


def lane_tree(v: np.ndarray) -> np.ndarray:
    """The DPP sum over the lanes of a row (last axis): lane ^ 1, lane ^ 2, the
    mirror within 8 lanes, the mirror within 16; every lane ends with the same
    value (IEEE addition commutes)."""
    L = v.shape[-1]
    for perm in ([l ^ 1 for l in range(L)], [l ^ 2 for l in range(L)],
                 [(l & ~7) | (7 - (l & 7)) for l in range(L)], [15 - l for l in range(L)]):
        if max(perm) >= L:
            break
        v = v + v[..., perm]
    return v[..., 0]


def row_sum(x_lanes: np.ndarray) -> np.ndarray:
    """The kernels' binary64 sum of a row: two accumulators per lane over its
    even and odd positions, their sum, then the lane tree."""
    s0, s1 = x_lanes[..., 0].copy(), x_lanes[..., 1].copy()
    for i in range(2, x_lanes.shape[-1], 2):
        s0 = s0 + x_lanes[..., i]
        s1 = s1 + x_lanes[..., i + 1]
    return lane_tree(s0 + s1)


def kernel_layer_norm(x16: np.ndarray, eps: float, estimate_error: float):
    """The kernels' LayerNorm method, emulated: the exact binary64 sums in the
    kernels' order; the one-pass variance m2 - mean^2 (one fused rounding) on
    rows with m2 <= 16 var (or all-zero rows), else the two-pass variance over
    the deviations (fused multiply-adds, same order); rstd from an estimate off
    by `estimate_error` and two Newton steps, 0 for a zero variance; every
    output fma(x, rstd, -mean*rstd), rounded to binary16 through round-to-odd
    binary32. Returns the outputs and the number of two-pass rows."""
    from fractions import Fraction
    C = x16.shape[1]
    x = x16.astype(np.float64)
    xl = lane_order(x, C)
    inv_c = 1.0 / C
    mean = row_sum(xl) * inv_c
    m2 = row_sum(xl * xl) * inv_c        # squares of binary16 values are exact in binary64
    out = np.empty(x.shape, np.float16)
    two_pass_rows = 0
    for i in range(x.shape[0]):
        mu = float(mean[i])
        var = float(Fraction(float(m2[i])) - Fraction(mu) ** 2)
        if not ((var > 0 and m2[i] <= 16.0 * var) or m2[i] == 0.0):
            two_pass_rows += 1
            lanes = []
            for lane in xl[i]:
                p0 = p1 = 0.0
                for j in range(0, lane.size, 2):
                    d0, d1 = lane[j] - mu, lane[j + 1] - mu
                    p0, p1 = fma(d0, d0, p0), fma(d1, d1, p1)
                lanes.append(p0 + p1)
            var = float(lane_tree(np.array(lanes))) * inv_c
        a = var + eps
        if var == 0.0:
            rstd = 0.0
        else:
            r0 = float(1.0 / np.sqrt(a)) * (1 + estimate_error)
            rstd = newton(a, newton(a, r0))
        shift = -mu * rstd
        out[i] = two_step(np.array([fma(float(v), rstd, shift) for v in x[i]]))
    return out, two_pass_rows


def test_one_pass_layer_norm_method_matches_the_oracle():
    """The emulated kernel method gives the oracle's binary16 outputs (equal
    values; only the sign of a zero may differ) on rows of every class the
    bench and the tests use: N(0,1), N(0.5,2), x50-scaled, near-constant
    (c + 1e-3 z), offset (100 + z), constant, all-zero, +-1, subnormal inputs,
    extreme two-valued rows, and rows at the one-pass limit (|mean| = 3.8 and
    4.0 standard deviations), at all three widths, with eps 1e-5 and two
    subnormal values, and with the hardware estimate off by +-2^-22 either
    way. The offset, near-constant, constant and
    4-sigma rows must take the second pass; the others must not."""
    import oracle
    rng = np.random.default_rng(7)
    for C in (192, 384, 768):
        z = rng.standard_normal((4, C))
        at_limit = [3.8 + z[0] / z[0].std() - z[0].mean() / z[0].std(), 4.0 + (z[1] - z[1].mean()) / z[1].std()]
        rows = [rng.standard_normal(C), rng.normal(0.5, 2.0, C), 50 * rng.standard_normal(C),
                rng.standard_normal() + 1e-3 * rng.standard_normal(C), 100 + rng.standard_normal(C),
                np.full(C, 1.5), np.full(C, -3.5), np.zeros(C), (np.arange(C) % 2 * 2 - 1.0),
                2.0 ** -24 * (np.arange(C) % 3), np.where(np.arange(C) % 2, 65504.0, -65504.0),
                at_limit[0], at_limit[1]]
        x = np.array(rows).astype(np.float16)
        for eps in (1e-5, 1e-320, 5e-324):  # subnormal eps: constant rows need rstd = 0, not 1/sqrt(eps)
            ref = oracle.layer_norm(x, eps)
            for e in (2.0 ** -22, -(2.0 ** -22)):
                got, two_pass = kernel_layer_norm(x, eps, e)
                assert np.array_equal(got.astype(np.float64), ref.astype(np.float64)), \
                    (C, eps, np.argwhere(got.astype(np.float64) != ref.astype(np.float64))[:5])
                assert two_pass == 5, (C, two_pass)        # near-constant, offset, two constants, 4-sigma
            assert not ref[5].view(np.uint16).any() and not ref[6].view(np.uint16).any()


def test_constant_row_mean_is_exact():
    """A constant row c has the exact binary64 sum C*c (any order), and the
    kernels' mean (C*c) * RN(1/C) is exactly c for every finite binary16 c at
    each served width, so the row's deviations and second-pass variance are
    exactly 0 and its outputs exactly +0 (rstd = 0)."""
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    c = h[np.isfinite(h)].astype(np.float64)
    for C in (192, 384, 768):
        mean = (c * C) * (1.0 / C)
        assert np.array_equal(mean, c), C

"""Pins of the CPU oracle to things other than itself.

Each test fixes one oracle function against what the pages and the mathematics
determine: IEEE binary16 rounding done in exact rational arithmetic, closed
forms of LayerNorm on special rows, a library LayerNorm, invariants, tables
derived by hand (tests/golden/), and brute force on tiny grids. A plausible slip
in the oracle (a dropped eps, an unbiased variance, a wrong roll sign, a swapped
window order, padding at the wrong end) fails at least one of them.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

# ---------------------------------------------------------------------------
# helpers that are independent of the oracle's arithmetic


def f16_from_bits(bits):
    return np.array(bits, dtype=np.uint16).view(np.float16)


def bits_of(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def rne_binary16_exact(q: Fraction):
    """Round an exact rational to binary16, ties to even, by counting ulps.
    Returns a Python float holding the rounded value (or +-inf)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    if a >= Fraction(65520):           # midpoint of 65504 and 2**16: ties go to 2**16 -> inf
        return sign * float("inf")
    if a < Fraction(1, 2 ** 14):
        ulp = Fraction(1, 2 ** 24)     # subnormal spacing
    else:
        e = a.numerator.bit_length() - a.denominator.bit_length()
        if Fraction(2) ** e > a:
            e -= 1
        ulp = Fraction(2) ** (e - 10)
    m = a / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * ulp)


# ---------------------------------------------------------------------------
# residual_sum: FP16(residual + branch), rounded once


def test_residual_golden_cases(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "fp16_residual_cases.json")))
    for case in spec["cases"]:
        r = f16_from_bits([int(case["residual"], 16)])
        b = f16_from_bits([int(case["branch"], 16)])
        got = oracle.residual_sum(r, b)
        if case["expect"] == "nan":
            assert np.isnan(got[0]), case
        else:
            assert int(bits_of(got)[0]) == int(case["expect"], 16), case


def _finite_f16_bits(rng, n):
    bits = rng.integers(0, 1 << 16, size=4 * n, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]
    return bits[:n]


def test_residual_matches_exact_rational_rounding():
    rng = np.random.default_rng(11)
    n = 6000
    a = _finite_f16_bits(rng, n)
    b = _finite_f16_bits(rng, n)
    # near-cancellation and same-binade pairs, where rounding decisions are dense
    c = _finite_f16_bits(rng, n)
    d = (c.astype(np.int32) ^ 0x8000) + rng.integers(-40, 41, size=n)
    d = np.clip(d, 0, 0xFFFF).astype(np.uint16)
    d[(d & 0x7C00) == 0x7C00] = 0
    ra = np.concatenate([a, c]).view(np.float16)
    rb = np.concatenate([b, d]).view(np.float16)
    got = bits_of(oracle.residual_sum(ra, rb))
    for x, y, g in zip(ra.tolist(), rb.tolist(), got.tolist()):
        exact = Fraction(x) + Fraction(y)
        v = rne_binary16_exact(exact)
        if exact == 0 and x == 0.0 and y == 0.0 and str(x)[0] == "-" and str(y)[0] == "-":
            v = -0.0
        assert g == int(np.float16(v).view(np.uint16)), (x, y, hex(g), v)


def test_residual_rounds_once_not_in_fp32_normalisation():
    # the LayerNorm reads the rounded residual: add_ln's y equals layer_norm of
    # its own residual output, not of the unrounded sum
    rng = np.random.default_rng(12)
    br = workloads.normal_rows(3, 8, 192)
    res = (rng.normal(size=(8, 192)) * 1e3).astype(np.float16)
    r, y = oracle.add_ln(br, res)
    assert np.array_equal(bits_of(r), bits_of(oracle.residual_sum(res, br)))
    assert np.array_equal(bits_of(y), bits_of(oracle.layer_norm(r)))


# ---------------------------------------------------------------------------
# layer_norm


@pytest.mark.parametrize("C", [192, 384])
def test_ln_plus_minus_one_row(C):
    row = np.array([1.0] * (C // 2) + [-1.0] * (C // 2), dtype=np.float16)[None, :]
    y = oracle.layer_norm(row)
    # mean 0, biased variance 1: y = +-1/sqrt(1 + 1e-5) = +-0.999995 -> +-1.0 in binary16
    assert np.array_equal(bits_of(y)[0, : C // 2], np.full(C // 2, 0x3C00, np.uint16))
    assert np.array_equal(bits_of(y)[0, C // 2:], np.full(C // 2, 0xBC00, np.uint16))


@pytest.mark.parametrize("C", [192, 384])
def test_ln_rounds_once_from_binary64(C):
    # A +-1 row has mean 0 and variance 1, so y = +-1/sqrt(1 + eps). eps is
    # chosen so that y lies 2**-30 below the binary16 midpoint 1 - 2**-12.
    # Rounded once, y goes down to 1 - 2**-11 (0x3BFF). Rounded to binary32
    # first, it lands on the midpoint (binary32 spacing below 1 is 2**-24),
    # and the tie then goes to even, 1.0 (0x3C00).
    getcontext().prec = 60
    target = Decimal(1) - Decimal(2) ** -12 - Decimal(2) ** -30
    eps = float(1 / (target * target) - 1)
    y_exact = 1 / (1 + Decimal(eps)).sqrt()
    mid = Decimal(1) - Decimal(2) ** -12
    assert Decimal(1) - Decimal(2) ** -11 < y_exact < mid and mid - y_exact > Decimal(2) ** -31
    row = np.array([1.0] * (C // 2) + [-1.0] * (C // 2), dtype=np.float16)[None, :]
    y = bits_of(oracle.layer_norm(row, eps))
    assert np.all(y[0, : C // 2] == 0x3BFF) and np.all(y[0, C // 2:] == 0xBBFF), hex(int(y[0, 0]))


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("value", [0.0, 3.5, -100.0, 65504.0])
def test_ln_constant_row_is_plus_zero(C, value):
    row = np.full((1, C), value, dtype=np.float16)
    assert np.array_equal(bits_of(oracle.layer_norm(row)), np.zeros((1, C), np.uint16))


def _two_valued_expected(C, k, a, b, eps=1e-5):
    """Closed form for a row with k entries a and C-k entries b:
    mean = (k a + (C-k) b)/C, biased var = k (C-k) (a-b)^2 / C^2,
    y_a = (C-k)(a-b)/C / sqrt(var+eps), y_b = -k (a-b)/C / sqrt(var+eps)."""
    getcontext().prec = 60
    A, B, D = Decimal(a), Decimal(b), Decimal(a) - Decimal(b)
    var = Decimal(k) * Decimal(C - k) * D * D / Decimal(C * C)
    den = (var + Decimal(eps)).sqrt()
    ya = Decimal(C - k) * D / Decimal(C) / den
    yb = -Decimal(k) * D / Decimal(C) / den
    return np.float16(float(ya)), np.float16(float(yb))


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("k,a,b", [(1, 2.0, 0.0), (5, 1.5, -0.25), (96, 2.0 ** -10, -(2.0 ** -10)),
                                   (37, 100.0, 101.0), (150, -3.0, 7.0), (3, 0.0078125, 0.0)])
def test_ln_two_valued_rows_closed_form(C, k, a, b):
    row = np.array([a] * k + [b] * (C - k), dtype=np.float16)[None, :]
    ya, yb = _two_valued_expected(C, k, float(row[0, 0]), float(row[0, -1]))
    y = oracle.layer_norm(row)
    assert np.all(bits_of(y[0, :k]) == bits_of(ya)), (y[0, 0], ya)
    assert np.all(bits_of(y[0, k:]) == bits_of(yb)), (y[0, -1], yb)


@pytest.mark.parametrize("C", [192, 384])
def test_ln_matches_torch_layer_norm_float64(C):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21 + C)
    x = np.concatenate([
        rng.normal(0, 1, size=(400, C)),
        rng.normal(100, 1, size=(50, C)),
        rng.normal(0.5, 2, size=(50, C)) * 50,
        rng.normal(0, 1, size=(50, 1)) + 1e-3 * rng.normal(0, 1, size=(50, C)),
    ]).astype(np.float16)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (C,), eps=1e-5)
    ref16 = ref.numpy().astype(np.float16)
    assert np.array_equal(bits_of(oracle.layer_norm(x)), bits_of(ref16))


@pytest.mark.parametrize("C", [192, 384])
def test_ln_row_invariants(C):
    rng = np.random.default_rng(31 + C)
    x = np.concatenate([
        rng.normal(0, 1, size=(200, C)),
        rng.normal(100, 1, size=(50, C)),
        rng.normal(0, 1, size=(50, 1)) + 1e-3 * rng.normal(0, 1, size=(50, C)),
    ]).astype(np.float16)
    y = oracle.layer_norm(x).astype(np.float64)
    v = x.astype(np.float64).var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) <= 1e-3
    assert np.max(np.abs(y.var(axis=1) - v / (v + 1e-5))) <= 1e-3


def test_ln_power_of_two_scale_and_shift_invariance():
    # LN(4x + 8) vs LN(x): both transformations are exact in binary16 for these
    # magnitudes; only eps breaks the invariance, by ~eps/var
    x = workloads.normal_rows(41, 64, 192).astype(np.float64)
    x = (np.clip(np.round(x * 64) / 64, -3.9, 3.9)).astype(np.float16)   # multiples of 2**-6
    x2 = (x.astype(np.float64) * 4 + 8).astype(np.float16)
    assert np.array_equal(x2.astype(np.float64), x.astype(np.float64) * 4 + 8)
    d = np.abs(oracle.layer_norm(x2).astype(np.float64) - oracle.layer_norm(x).astype(np.float64))
    assert d.max() <= 2e-3


def test_ln_nonfinite_rows_become_nan_rows():
    x = workloads.normal_rows(42, 4, 192)
    x[1, 7] = np.inf
    x[2, 0] = np.nan
    y = oracle.layer_norm(x)
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all()
    assert np.isfinite(y[0]).all() and np.isfinite(y[3]).all()


def test_ln_rejects_other_widths():
    with pytest.raises(ValueError):
        oracle.layer_norm(np.zeros((2, 256), np.float16))


# ---------------------------------------------------------------------------
# window tables


def brute_force_table(grid, window, shift):
    """Loop form: visit windows and their tokens in order, map each gathered
    position to the padded grid, apply the cyclic shift and test the real grid."""
    Z, H, W = grid
    wz, wh, ww = window
    Zp, Hp, Wp = (-(-Z // wz) * wz, -(-H // wh) * wh, -(-W // ww) * ww)
    out = []
    for bz in range(Zp // wz):
        for bh in range(Hp // wh):
            for bw in range(Wp // ww):
                for dz in range(wz):
                    for dh in range(wh):
                        for dw in range(ww):
                            qz = (bz * wz + dz + shift[0]) % Zp
                            qh = (bh * wh + dh + shift[1]) % Hp
                            qw = (bw * ww + dw + shift[2]) % Wp
                            if qz < Z and qh < H and qw < W:
                                out.append((qz * H + qh) * W + qw)
                            else:
                                out.append(-1)
    return np.array(out, dtype=np.int32)


def test_window_table_golden_points(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "window_table_points.json")))
    for case in spec["cases"]:
        grid, window, shift = tuple(case["grid"]), tuple(case["window"]), tuple(case["shift"])
        t = oracle.window_index_table(grid, window, shift)
        assert t.dtype == np.int32
        assert oracle.window_token_count(grid, window) == case["rows"] == t.shape[0]
        assert int((t == -1).sum()) == case["pads"]
        for j, v in case["points"].items():
            assert int(t[int(j)]) == v, (case["grid"], case["shift"], j)
        if "first_pad" in case:
            assert int(np.argmax(t == -1)) == case["first_pad"]


@pytest.mark.parametrize("grid", [(2, 12, 24), (2, 7, 13), (4, 9, 26), (3, 6, 12), (1, 1, 1), (5, 11, 25)])
@pytest.mark.parametrize("shift", [(0, 0, 0), (1, 3, 6), (0, 5, 11), (3, 13, 30)])
def test_window_table_matches_brute_force(grid, shift):
    window = workloads.WINDOW
    t = oracle.window_index_table(grid, window, shift)
    assert np.array_equal(t, brute_force_table(grid, window, shift))


@pytest.mark.parametrize("level", [workloads.LEVEL1, workloads.LEVEL2])
@pytest.mark.parametrize("shift", [workloads.NO_SHIFT, workloads.SHIFT])
def test_window_table_is_a_bijection_onto_tokens(level, shift):
    t = oracle.window_index_table(level.grid, workloads.WINDOW, shift)
    valid = np.sort(t[t >= 0])
    assert np.array_equal(valid, np.arange(level.tokens, dtype=np.int32))
    assert int((t == -1).sum()) == t.shape[0] - level.tokens
    assert int(t.min()) >= -1


def test_window_table_special_cases():
    # one window covering the whole grid, no shift: identity
    assert np.array_equal(oracle.window_index_table((2, 6, 12), (2, 6, 12)), np.arange(144))
    # unit windows, no shift: identity in grid order
    assert np.array_equal(oracle.window_index_table((3, 5, 7), (1, 1, 1)), np.arange(105))
    # a shift by a whole padded extent is no shift
    a = oracle.window_index_table((8, 20, 30), (2, 6, 12), (0, 0, 0))
    b = oracle.window_index_table((8, 20, 30), (2, 6, 12), (8, 24, 36))
    assert np.array_equal(a, b)
    # unit windows with a shift: a plain cyclic roll of the token ids
    t = oracle.window_index_table((1, 1, 10), (1, 1, 1), (0, 0, 3))
    assert t.tolist() == [3, 4, 5, 6, 7, 8, 9, 0, 1, 2]


# ---------------------------------------------------------------------------
# gathers


def test_window_gather_brute_force_with_pads_and_bad_entries():
    rng = np.random.default_rng(51)
    x = workloads.normal_rows(52, 50, 192)
    table = rng.integers(-1, 50, size=300).astype(np.int32)
    table[::17] = 50          # one past the end: a zero row, not a read
    table[5] = -7             # any other negative entry: a zero row
    out = oracle.window_gather(x, table)
    for j, t in enumerate(table.tolist()):
        if 0 <= t < 50:
            assert np.array_equal(bits_of(out[j]), bits_of(x[t]))
        else:
            assert not bits_of(out[j]).any()   # +0.0 bits


def test_window_gather_id_encoded_rows_decode_to_the_table():
    # each source row carries its own index as exact binary16 integers
    grid = (8, 20, 30)
    n = 8 * 20 * 30
    x = np.zeros((n, 192), np.float16)
    ids = np.arange(n)
    x[:, 0] = ids % 2048
    x[:, 1] = ids // 2048
    x[:, 2] = 1.0
    t = oracle.window_index_table(grid, workloads.WINDOW, workloads.SHIFT)
    g = oracle.window_gather(x, t).astype(np.int64)
    decoded = np.where(g[:, 2] == 1, g[:, 0] + 2048 * g[:, 1], -1)
    assert np.array_equal(decoded, t.astype(np.int64))


def test_norm_gather_rows_agrees_with_full_norm_gather():
    x = workloads.normal_rows(61, 576, 192)
    x[3] = np.float16(2.5)  # a constant row
    t = oracle.window_index_table((2, 12, 24), workloads.WINDOW, workloads.SHIFT)
    full = oracle.norm_gather(x, t)
    rows = np.array([0, 1, 100, 575, int(np.argmax(t == 3))])
    assert np.array_equal(bits_of(oracle.norm_gather_rows(x, t, rows)), bits_of(full[rows]))
    assert not bits_of(full[int(np.argmax(t == 3))]).any()


# ---------------------------------------------------------------------------
# window reverse and the fused rows built on it


def brute_force_inverse(grid, window, shift):
    """Loop form: for each token, find its rolled position, its window and the
    offset inside the window."""
    Z, H, W = grid
    wz, wh, ww = window
    Zp, Hp, Wp = (-(-Z // wz) * wz, -(-H // wh) * wh, -(-W // ww) * ww)
    nbh, nbw = Hp // wh, Wp // ww
    out = []
    for z in range(Z):
        for h in range(H):
            for w in range(W):
                gz, gh, gw = (z - shift[0]) % Zp, (h - shift[1]) % Hp, (w - shift[2]) % Wp
                win = ((gz // wz) * nbh + gh // wh) * nbw + gw // ww
                off = ((gz % wz) * wh + gh % wh) * ww + gw % ww
                out.append(win * wz * wh * ww + off)
    return np.array(out, dtype=np.int32)


def test_window_inverse_golden_points(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "window_inverse_points.json")))
    for case in spec["cases"]:
        inv = oracle.window_inverse_table(tuple(case["grid"]), tuple(case["window"]), tuple(case["shift"]))
        for i, j in case["points"].items():
            assert int(inv[int(i)]) == j, (case["grid"], case["shift"], i)


@pytest.mark.parametrize("grid", [(2, 12, 24), (2, 7, 13), (4, 9, 26), (1, 1, 1), (5, 11, 25)])
@pytest.mark.parametrize("shift", [(0, 0, 0), (1, 3, 6), (3, 13, 30)])
def test_window_inverse_matches_brute_force_and_forward(grid, shift):
    inv = oracle.window_inverse_table(grid, workloads.WINDOW, shift)
    assert np.array_equal(inv, brute_force_inverse(grid, workloads.WINDOW, shift))
    t = oracle.window_index_table(grid, workloads.WINDOW, shift)
    assert np.array_equal(t[inv], np.arange(int(np.prod(grid)), dtype=np.int32))


@pytest.mark.parametrize("grid", [(2, 12, 24), (4, 9, 26), (3, 13, 25)])
@pytest.mark.parametrize("shift", [(0, 0, 0), (1, 3, 6)])
def test_window_reverse_undoes_the_gather(grid, shift):
    n = int(np.prod(grid))
    x = workloads.normal_rows(71, n, 192)
    t = oracle.window_index_table(grid, workloads.WINDOW, shift)
    back = oracle.window_reverse(oracle.window_gather(x, t), grid, workloads.WINDOW, shift)
    assert np.array_equal(bits_of(back), bits_of(x))


def test_window_reverse_drops_padding_rows():
    grid = (2, 7, 13)
    t = oracle.window_index_table(grid, workloads.WINDOW, (1, 3, 6))
    rows = np.where(t[:, None] >= 0, 1.0, 7.0).astype(np.float16).repeat(192, axis=1)
    back = oracle.window_reverse(rows, grid, workloads.WINDOW, (1, 3, 6))
    assert back.shape == (int(np.prod(grid)), 192) and (back == 1.0).all()


def test_window_reverse_add_ln_and_add_norm_gather_compose():
    grid = (2, 7, 13)
    n = int(np.prod(grid))
    t = oracle.window_index_table(grid, workloads.WINDOW, (1, 3, 6))
    attn = workloads.normal_rows(72, t.size, 192)
    res = workloads.normal_rows(73, n, 192)
    r, y = oracle.window_reverse_add_ln(attn, res, grid, workloads.WINDOW, (1, 3, 6))
    inv = oracle.window_inverse_table(grid, workloads.WINDOW, (1, 3, 6))
    for i in (0, 5, n - 1):   # token i adds the attention row that holds it
        exact = res[i].astype(np.float64) + attn[inv[i]].astype(np.float64)
        assert np.array_equal(bits_of(r[i]), bits_of(exact.astype(np.float16)))
    assert np.array_equal(bits_of(y), bits_of(oracle.layer_norm(r)))
    br = workloads.normal_rows(74, n, 192)
    r2, g = oracle.add_norm_gather(br, res, t)
    assert np.array_equal(bits_of(r2), bits_of(oracle.residual_sum(res, br)))
    assert np.array_equal(bits_of(g), bits_of(oracle.window_gather(oracle.layer_norm(r2), t)))


# ---------------------------------------------------------------------------
# the patch-merge width and the affine LayerNorm


def test_ln_width_768_closed_forms():
    C = 768
    row = np.array([1.0] * (C // 2) + [-1.0] * (C // 2), dtype=np.float16)[None, :]
    assert (bits_of(oracle.layer_norm(row))[0, : C // 2] == 0x3C00).all()
    k, a, b = 100, 3.0, -0.5
    row = np.array([a] * k + [b] * (C - k), dtype=np.float16)[None, :]
    ya, yb = _two_valued_expected(C, k, a, b)
    y = oracle.layer_norm(row)
    assert (bits_of(y[0, :k]) == bits_of(ya)).all() and (bits_of(y[0, k:]) == bits_of(yb)).all()


def test_ln_width_768_matches_torch():
    torch = pytest.importorskip("torch")
    x = workloads.normal_rows(95, 300, 768, mean=0.25, std=3.0)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (768,), eps=1e-5)
    assert np.array_equal(bits_of(oracle.layer_norm(x)), bits_of(ref.numpy().astype(np.float16)))


@pytest.mark.parametrize("C", [192, 384, 768])
def test_ln_affine_reduces_and_scales(C):
    x = workloads.normal_rows(96, 200, C, mean=-1.0, std=2.0)
    ones, zeros = np.ones(C, np.float16), np.zeros(C, np.float16)
    # unit scale, zero shift: the plain LayerNorm
    assert np.array_equal(bits_of(oracle.layer_norm_affine(x, ones, zeros)), bits_of(oracle.layer_norm(x)))
    # a scale of 2 doubles every binary16 result exactly in the normal range (in
    # the subnormal range the spacing is fixed at 2**-24, so doubling can round
    # differently there)
    twos = np.full(C, 2.0, np.float16)
    y1 = oracle.layer_norm(x).astype(np.float64)
    y2 = oracle.layer_norm_affine(x, twos, zeros).astype(np.float64)
    normal = np.abs(y1) >= 2.0 ** -14
    assert normal.mean() > 0.99
    assert np.array_equal(y2[normal], 2.0 * y1[normal])
    # zero scale leaves the shift
    beta = workloads.normal_rows(97, 1, C)[0]
    assert np.array_equal(bits_of(oracle.layer_norm_affine(x, zeros, beta)), bits_of(np.tile(beta, (200, 1))))


@pytest.mark.parametrize("C", [192, 384, 768])
def test_ln_affine_matches_torch(C):
    torch = pytest.importorskip("torch")
    x = workloads.normal_rows(98, 300, C)
    g = workloads.normal_rows(99, 1, C, mean=1.0, std=0.2)[0]
    b = workloads.normal_rows(100, 1, C, std=0.1)[0]
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (C,),
                                         weight=torch.from_numpy(g.astype(np.float64)),
                                         bias=torch.from_numpy(b.astype(np.float64)), eps=1e-5)
    assert np.array_equal(bits_of(oracle.layer_norm_affine(x, g, b)), bits_of(ref.numpy().astype(np.float16)))


def test_ln_affine_two_valued_closed_form():
    C, k, a, b = 192, 10, 0.5, -2.0
    row = np.array([a] * k + [b] * (C - k), dtype=np.float16)[None, :]
    g = np.full(C, 1.5, np.float16)
    be = np.full(C, 0.25, np.float16)
    getcontext().prec = 60
    D = Decimal(a) - Decimal(b)
    den = (Decimal(k) * Decimal(C - k) * D * D / Decimal(C * C) + Decimal(1e-5)).sqrt()
    ya = Decimal(C - k) * D / Decimal(C) / den * Decimal(1.5) + Decimal(0.25)
    yb = -Decimal(k) * D / Decimal(C) / den * Decimal(1.5) + Decimal(0.25)
    y = oracle.layer_norm_affine(row, g, be)
    assert (bits_of(y[0, :k]) == bits_of(np.float16(float(ya)))).all()
    assert (bits_of(y[0, k:]) == bits_of(np.float16(float(yb)))).all()
    r, y2 = oracle.add_ln_affine(np.zeros_like(row), row, g, be)
    assert np.array_equal(bits_of(r), bits_of(row)) and np.array_equal(bits_of(y2), bits_of(y))


# ---------------------------------------------------------------------------
# bias + tanh-GELU (float32)


def test_bias_gelu_matches_torch_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(120)
    x = rng.normal(0, 3, size=(257, 96)).astype(np.float32)
    b = rng.normal(0, 1, size=96).astype(np.float32)
    t = torch.from_numpy(x) + torch.from_numpy(b)                # the float32 add of the eager path
    ref = torch.nn.functional.gelu(t.double(), approximate="tanh").numpy()
    got = oracle.bias_gelu(x, b).astype(np.float64)
    # both evaluate the same formula in float64; in the saturated negative tail
    # 1 + tanh(z) cancels and the two differ by ~1e-16 absolute, nowhere else
    assert np.allclose(got, ref.astype(np.float32).astype(np.float64), rtol=1e-7, atol=1e-15)
    big = np.abs(ref) > 1e-6
    assert np.array_equal(got[big], ref[big].astype(np.float32).astype(np.float64))
    # a wrong constant or the exact (erf) GELU is far outside that agreement
    erf = torch.nn.functional.gelu(t.double()).numpy()
    assert np.abs(erf - ref).max() > 1e-4


def test_bias_gelu_closed_forms():
    x = np.array([[0.0, -0.0, 1.0, -1.0, 30.0, -30.0, np.inf, -np.inf, np.nan, 2.5]], np.float32)
    y = oracle.bias_gelu(x, np.zeros(x.shape[1], np.float32))
    assert y[0, 0] == 0.0 and y[0, 1] == 0.0
    # g(t) - g(-t) = t exactly in real arithmetic (tanh is odd)
    assert abs(float(y[0, 2]) - float(y[0, 3]) - 1.0) < 1e-6
    assert y[0, 4] == np.float32(30.0) and y[0, 5] == 0.0        # saturation: t and -0
    assert y[0, 6] == np.inf and np.isnan(y[0, 7]) and np.isnan(y[0, 8])
    # tanh form at 1: 0.5 * (1 + tanh(sqrt(2/pi) * 1.044715)), worked out in high precision
    getcontext().prec = 50
    import math
    z = math.sqrt(2 / math.pi) * 1.044715
    assert abs(float(y[0, 2]) - 0.5 * (1 + math.tanh(z))) < 1e-7


def test_bias_gelu_adds_the_bias_in_float32_first():
    # 1 + 2**-30 rounds to 1 in float32: the activation must see exactly 1.0
    x = np.array([[1.0]], np.float32)
    b = np.array([2.0 ** -30], np.float32)
    assert oracle.bias_gelu(x, b)[0, 0] == oracle.bias_gelu(x, np.zeros(1, np.float32))[0, 0]

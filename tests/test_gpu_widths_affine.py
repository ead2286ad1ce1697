"""Parity of the patch-merge width (C = 768) in every kernel, and of the affine
LayerNorm calls, with the CPU oracle."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import PATCH_MERGE, WINDOW, SHIFT, NO_SHIFT

from parity_helpers import assert_bit_exact, assert_ln_close, bits, host, to_dev

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows", [1, 3, 4, 5, 63, 64, 65, 1000, 4097])
def test_width_768_ln_and_add_ln_ragged(dev, rows):
    x = workloads.normal_rows(300 + rows, rows, 768, mean=0.2, std=1.5)
    res = workloads.normal_rows(400 + rows, rows, 768)
    assert_ln_close(host(lwg.ln_fixed(to_dev(x, dev))), oracle.layer_norm(x), f"ln 768 rows={rows}")
    r, y = lwg.add_ln(to_dev(x, dev), to_dev(res, dev))
    r_ref, y_ref = oracle.add_ln(x, res)
    assert_bit_exact(host(r), r_ref, f"residual 768 rows={rows}")
    assert_ln_close(host(y), y_ref, f"add_ln 768 rows={rows}")


def test_width_768_patch_merge_shape(dev):
    n = PATCH_MERGE.tokens
    nc, off = workloads.stress_row_classes(11, n)
    x = workloads.mixed_rows(12, n, 768, nc, off)
    tx = to_dev(x, dev)
    y = host(lwg.ln_fixed(tx))
    assert_ln_close(y, oracle.layer_norm(x), "patch-merge LayerNorm [32760, 768]")
    y2 = host(lwg.ln_fixed(tx, out=tx))
    assert_bit_exact(y2, y, "in place")


@pytest.mark.parametrize("grid,shift", [((2, 12, 24), SHIFT), ((3, 7, 13), NO_SHIFT), ((4, 9, 26), (3, 13, 30))])
def test_width_768_gathers_and_fusions(dev, grid, shift):
    n = int(np.prod(grid))
    x = workloads.normal_rows(13, n, 768)
    br = workloads.normal_rows(14, n, 768)
    table = oracle.window_index_table(grid, WINDOW, shift)
    t = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    inv = lwg.window_inverse_build(grid, WINDOW, shift, device=dev)
    tx = to_dev(x, dev)
    assert_bit_exact(host(lwg.window_gather(tx, t)), oracle.window_gather(x, table), "gather 768")
    ng = host(lwg.norm_gather(tx, t))
    assert_ln_close(ng, oracle.norm_gather(x, table), "norm_gather 768")
    assert_bit_exact(ng, host(lwg.window_gather(lwg.ln_fixed(tx), t)), "norm_gather == gather(ln) 768")
    rows = workloads.normal_rows(15, table.size, 768)
    r, y = lwg.window_reverse_add_ln(to_dev(rows, dev), inv, tx)
    r_ref, y_ref = oracle.window_reverse_add_ln(rows, x, grid, WINDOW, shift)
    assert_bit_exact(host(r), r_ref, "reverse_add_ln residual 768")
    assert_ln_close(host(y), y_ref, "reverse_add_ln 768")
    r2, g = lwg.add_norm_gather(to_dev(br, dev), tx, t)
    r2_ref, g_ref = oracle.add_norm_gather(br, x, table)
    assert_bit_exact(host(r2), r2_ref, "add_norm_gather residual 768")
    assert_ln_close(host(g), g_ref, "add_norm_gather 768")


def _params(C, seed):
    g = workloads.normal_rows(seed, 1, C, mean=1.0, std=0.3)[0]
    b = workloads.normal_rows(seed + 1, 1, C, std=0.5)[0]
    return g, b


@pytest.mark.parametrize("C", [192, 384, 768])
@pytest.mark.parametrize("rows", [1, 7, 65, 2049])
def test_ln_affine_parity(dev, C, rows):
    x = workloads.normal_rows(500 + rows, rows, C, mean=-0.7, std=2.0)
    g, b = _params(C, 17)
    y = host(lwg.ln_affine(to_dev(x, dev), to_dev(g, dev), to_dev(b, dev)))
    assert_ln_close(y, oracle.layer_norm_affine(x, g, b), f"ln_affine C={C} rows={rows}")


@pytest.mark.parametrize("C", [192, 384, 768])
def test_ln_affine_identity_params_equal_ln_fixed(dev, C):
    x = workloads.normal_rows(21, 3000, C)
    tx = to_dev(x, dev)
    one = torch.ones(C, dtype=torch.float16, device=dev)
    zero = torch.zeros(C, dtype=torch.float16, device=dev)
    assert_bit_exact(host(lwg.ln_affine(tx, one, zero)), host(lwg.ln_fixed(tx)), f"ln_affine(1,0) C={C}")


@pytest.mark.parametrize("C", [192, 384, 768])
def test_add_ln_affine_parity_and_aliasing(dev, C):
    rows = 3001
    nc, off = workloads.stress_row_classes(22, rows)
    res = workloads.mixed_rows(23, rows, C, nc, off)
    br = workloads.mixed_rows(24, rows, C, nc, off, offset_mean=0.0)
    g, b = _params(C, 25)
    tg, tb_ = to_dev(g, dev), to_dev(b, dev)
    r_ref, y_ref = oracle.add_ln_affine(br, res, g, b)
    r, y = lwg.add_ln_affine(to_dev(br, dev), to_dev(res, dev), tg, tb_)
    assert_bit_exact(host(r), r_ref, f"add_ln_affine residual C={C}")
    assert_ln_close(host(y), y_ref, f"add_ln_affine C={C}")
    tbr, tr = to_dev(br, dev), to_dev(res, dev)
    lwg.add_ln_affine(tbr, tr, tg, tb_, residual_out=tr, out=tbr)
    assert_bit_exact(host(tr), r_ref, "in-place residual")
    assert_ln_close(host(tbr), y_ref, "y over the branch")


def test_affine_parameter_checks(dev):
    x = torch.zeros(4, 192, dtype=torch.float16, device=dev)
    with pytest.raises(RuntimeError, match="gamma"):
        lwg.ln_affine(x, torch.ones(191, dtype=torch.float16, device=dev), torch.zeros(192, dtype=torch.float16, device=dev))
    with pytest.raises(RuntimeError, match="beta"):
        lwg.ln_affine(x, torch.ones(192, dtype=torch.float16, device=dev), torch.zeros(192, dtype=torch.float32, device=dev))


@pytest.mark.parametrize("level,seed", [(workloads.LEVEL1, 31), (workloads.LEVEL2, 32)])
def test_affine_full_size(dev, level, seed):
    """Both affine kernels at the workload sizes (at level 2 add_ln_affine runs
    a capped grid whose waves take two row tiles each)."""
    n, c = level.tokens, level.channels
    nc, off = workloads.stress_row_classes(seed, n)
    res = workloads.mixed_rows(seed + 1, n, c, nc, off)
    br = workloads.mixed_rows(seed + 2, n, c, nc, off, offset_mean=0.0)
    g, b = _params(c, seed + 3)
    tg, tb_ = to_dev(g, dev), to_dev(b, dev)
    y = host(lwg.ln_affine(to_dev(res, dev), tg, tb_))
    assert_ln_close(y, oracle.layer_norm_affine(res, g, b), f"ln_affine {level.name}")
    r, y = lwg.add_ln_affine(to_dev(br, dev), to_dev(res, dev), tg, tb_)
    r_ref, y_ref = oracle.add_ln_affine(br, res, g, b)
    assert_bit_exact(host(r), r_ref, f"add_ln_affine residual {level.name}")
    assert_ln_close(host(y), y_ref, f"add_ln_affine {level.name}")


@pytest.mark.parametrize("C", [192, 384, 768])
def test_every_layernorm_rounds_once_next_to_a_midpoint(dev, C):
    """A +-1 row has mean 0 and variance 1, so y = +-1/sqrt(1 + eps). With eps
    chosen so that y lies 2**-30 below the binary16 midpoint 1 - 2**-12, a single
    rounding gives 0x3BFF, while narrowing to binary32 first lands on the
    midpoint and gives 0x3C00 by ties-to-even. Every kernel that normalises a
    row must return 0x3BFF / 0xBBFF there, bit for bit with the oracle, at every
    width (144 rows: one window of the (2, 6, 12) shape, so the reverse uses an
    identity inverse table)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    target = Decimal(1) - Decimal(2) ** -12 - Decimal(2) ** -30
    eps = float(1 / (target * target) - 1)
    n, half = 144, C // 2
    x = workloads.normal_rows(700 + C, n, C, mean=0.1, std=1.3)
    pm = np.array([1.0] * half + [-1.0] * half, dtype=np.float16)
    crafted = [0, 1, 2, 77, n - 1]
    x[0], x[1], x[2], x[77], x[n - 1] = pm, -pm, np.roll(pm, 5), pm[::-1], pm
    ref = oracle.layer_norm(x, eps)
    assert np.all(np.isin(bits(ref[crafted]), (0x3BFF, 0xBBFF)))
    ones = np.ones(C, np.float16)
    zeros = np.zeros(C, np.float16)
    assert np.array_equal(bits(oracle.layer_norm_affine(x, ones, zeros, eps)), bits(ref))

    xd, zd = to_dev(x, dev), torch.zeros(n, C, dtype=torch.float16, device=dev)
    g1, b0 = to_dev(ones, dev), to_dev(zeros, dev)
    ident = torch.arange(n, dtype=torch.int32, device=dev)
    inv = lwg.window_inverse_table((2, 6, 12), WINDOW, NO_SHIFT, device=dev)
    assert np.array_equal(host(inv), np.arange(n, dtype=np.int32))
    outs = {
        "ln_fixed": lwg.ln_fixed(xd, eps),
        "add_ln": lwg.add_ln(xd, zd, eps)[1],
        "norm_gather": lwg.norm_gather(xd, ident, eps),
        "add_norm_gather": lwg.add_norm_gather(xd, zd, ident, eps)[1],
        "window_reverse_add_ln": lwg.window_reverse_add_ln(xd, inv, zd, eps)[1],
        "ln_affine": lwg.ln_affine(xd, g1, b0, eps),
        "add_ln_affine": lwg.add_ln_affine(xd, zd, g1, b0, eps)[1],
    }
    for name, y in outs.items():
        got = host(y)
        assert_bit_exact(got[crafted], ref[crafted], f"{name} C={C} next to the midpoint")
        assert_ln_close(got, ref, f"{name} C={C}")


@pytest.mark.parametrize("C", [192, 384, 768])
def test_subnormal_inputs_and_outputs(dev, C):
    """Rows of binary16 subnormals (|x| < 2**-14, spacing 2**-24) with eps = 0.5:
    the variance is far below eps, so y ~ 1.4 (x - mean) lands in the binary16
    subnormal range too. Every normalising kernel must return the oracle's
    binary16 values bit for bit: subnormal inputs widen exactly, and subnormal
    outputs are produced, not flushed to zero."""
    rng = np.random.default_rng(800 + C)
    n = 333
    x = (rng.integers(-1023, 1024, size=(n, C)) * 2.0 ** -24).astype(np.float16)   # subnormals and zeros
    assert np.all(np.abs(x.astype(np.float64)) < 2.0 ** -14)
    eps = 0.5
    ref = oracle.layer_norm(x, eps)
    sub = (ref != 0) & (np.abs(ref.astype(np.float64)) < 2.0 ** -14)
    assert sub.mean() > 0.5                     # most outputs are subnormal
    xd, zd = to_dev(x, dev), torch.zeros(n, C, dtype=torch.float16, device=dev)
    ones, zeros = np.ones(C, np.float16), np.zeros(C, np.float16)
    ident = torch.arange(n, dtype=torch.int32, device=dev)
    outs = {
        "ln_fixed": lwg.ln_fixed(xd, eps),
        "add_ln": lwg.add_ln(xd, zd, eps)[1],
        "norm_gather": lwg.norm_gather(xd, ident, eps),
        "add_norm_gather": lwg.add_norm_gather(xd, zd, ident, eps)[1],
        "ln_affine": lwg.ln_affine(xd, to_dev(ones, dev), to_dev(zeros, dev), eps),
    }
    for name, y in outs.items():
        assert_bit_exact(host(y), ref, f"{name} C={C} subnormal rows")


@pytest.mark.parametrize("C", [192, 384, 768])
def test_affine_output_at_the_binary16_overflow_threshold(dev, C):
    """gamma = 65504 and a +-1 row with eps = 1e-12 give y = +-(1 - 5e-13), so
    y * gamma + beta lies 3.3e-8 below 65520 (the threshold where binary16
    rounds to +Inf) for beta = 16 and just above it for beta = 17. A single
    rounding gives 65504 and +Inf; a binary32 value first would round the
    beta = 16 case up to 65520 and then to +Inf. The negative side lands
    between binary16 neighbours and goes to -65472."""
    n, half = 6, C // 2
    pm = np.array([1.0] * half + [-1.0] * half, dtype=np.float16)
    x = np.stack([pm, pm[::-1], pm, np.roll(pm, 3), pm, pm]).astype(np.float16)[:n]
    gamma = np.full(C, 65504.0, np.float16)
    beta = np.where(np.arange(C) % 2 == 0, 16.0, 17.0).astype(np.float16)
    eps = 1e-12
    ref = oracle.layer_norm_affine(x, gamma, beta, eps)
    r0 = bits(ref[0])
    assert np.all(r0[:half][0::2] == 0x7BFF) and np.all(r0[:half][1::2] == 0x7C00)   # 65504, +Inf
    assert np.all(r0[half:] == 0xFBFE)                                                 # -65472
    xd, tg, tb = to_dev(x, dev), to_dev(gamma, dev), to_dev(beta, dev)
    assert_bit_exact(host(lwg.ln_affine(xd, tg, tb, eps)), ref, f"ln_affine C={C} at the overflow threshold")
    r, y = lwg.add_ln_affine(xd, torch.zeros_like(xd), tg, tb, eps)
    assert_bit_exact(host(y), ref, f"add_ln_affine C={C} at the overflow threshold")


@pytest.mark.parametrize("eps", [5e-324, 1e-310, 1e-300])
def test_subnormal_and_tiny_eps(dev, eps):
    """eps may be any finite positive binary64, down to the smallest subnormal.
    A constant row then has var + eps = eps, and its rsqrt must not flush to
    infinity (0 * inf would give NaN): the outputs stay +0.0, as in the oracle.
    Rows with a spread are unaffected by so small an eps."""
    C = 384
    rows = np.stack([np.full(C, 3.5), np.array([1.0, -1.0] * (C // 2)), np.zeros(C)] +
                    [workloads.normal_rows(900 + i, 1, C)[0].astype(np.float64) for i in range(5)]).astype(np.float16)
    ref = oracle.layer_norm(rows, eps)
    assert not np.isnan(ref).any() and not bits(ref[[0, 2]]).any()
    xd = to_dev(rows, dev)
    assert_bit_exact(host(lwg.ln_fixed(xd, eps)), ref, f"ln_fixed eps={eps}")
    zeros = torch.zeros_like(xd)
    assert_bit_exact(host(lwg.add_ln(xd, zeros, eps)[1]), ref, f"add_ln eps={eps}")
    ident = torch.arange(rows.shape[0], dtype=torch.int32, device=dev)
    assert_bit_exact(host(lwg.norm_gather(xd, ident, eps)), ref, f"norm_gather eps={eps}")

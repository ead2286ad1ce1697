"""Parity of the window reverse and the two fusions around the window gather
(reverse + add + LayerNorm, add + LayerNorm + gather) with the CPU oracle, at
small ragged sizes and at the level-1 / level-2 shapes."""
import numpy as np
import pytest

import oracle
import workloads
from workloads import LEVEL1, LEVEL2, WINDOW, SHIFT, NO_SHIFT

from parity_helpers import assert_bit_exact, assert_ln_close, bits, host, to_dev

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

GRIDS = [((2, 12, 24), NO_SHIFT), ((2, 12, 24), SHIFT), ((2, 7, 13), SHIFT), ((4, 9, 26), (3, 13, 30)),
         ((1, 1, 1), SHIFT), ((5, 11, 25), (0, 5, 11))]


@pytest.mark.parametrize("grid,shift", GRIDS + [(LEVEL1.grid, SHIFT), (LEVEL2.grid, NO_SHIFT), (LEVEL2.grid, SHIFT)])
def test_window_inverse_build_bit_exact(dev, grid, shift):
    inv = host(lwg.window_inverse_build(grid, WINDOW, shift, device=dev))
    assert inv.dtype == np.int32
    assert np.array_equal(inv, oracle.window_inverse_table(grid, WINDOW, shift))


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("grid,shift", GRIDS[:4])
def test_window_reverse_round_trip(dev, C, grid, shift):
    n = int(np.prod(grid))
    x = workloads.normal_rows(81, n, C)
    t = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    inv = lwg.window_inverse_build(grid, WINDOW, shift, device=dev)
    g = lwg.window_gather(to_dev(x, dev), t)
    back = host(lwg.window_reverse(g, inv))
    assert_bit_exact(back, x, "gather then reverse")
    rows = workloads.normal_rows(82, t.numel(), C)
    assert_bit_exact(host(lwg.window_reverse(to_dev(rows, dev), inv)),
                     oracle.window_reverse(rows, grid, WINDOW, shift), "reverse vs oracle")


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("grid,shift", GRIDS)
def test_window_reverse_add_ln_small(dev, C, grid, shift):
    n = int(np.prod(grid))
    m = oracle.window_token_count(grid, WINDOW)
    rows = workloads.normal_rows(83, m, C, std=2.0)
    res = workloads.normal_rows(84, n, C)
    inv = lwg.window_inverse_build(grid, WINDOW, shift, device=dev)
    r, y = lwg.window_reverse_add_ln(to_dev(rows, dev), inv, to_dev(res, dev))
    r_ref, y_ref = oracle.window_reverse_add_ln(rows, res, grid, WINDOW, shift)
    assert_bit_exact(host(r), r_ref, f"reverse_add_ln residual C={C} grid={grid}")
    assert_ln_close(host(y), y_ref, f"reverse_add_ln C={C} grid={grid}")


@pytest.mark.parametrize("C", [192, 384])
def test_window_reverse_add_ln_in_place_and_composition(dev, C):
    grid, shift = (4, 9, 26), SHIFT
    n, m = int(np.prod(grid)), oracle.window_token_count(grid, WINDOW)
    rows = workloads.normal_rows(85, m, C)
    res = workloads.normal_rows(86, n, C, mean=100.0)
    inv = lwg.window_inverse_build(grid, WINDOW, shift, device=dev)
    tr, trows = to_dev(res, dev), to_dev(rows, dev)
    r_ref, y_ref = oracle.window_reverse_add_ln(rows, res, grid, WINDOW, shift)
    # composition: the fused call equals reverse, then add_ln
    r2, y2 = lwg.add_ln(lwg.window_reverse(trows, inv), tr)
    r1, y1 = lwg.window_reverse_add_ln(trows, inv, tr)
    assert_bit_exact(host(r1), host(r2), "fused residual vs reverse then add_ln")
    assert_bit_exact(host(y1), host(y2), "fused y vs reverse then add_ln")
    # residual stream updated in place
    lwg.window_reverse_add_ln(trows, inv, tr, residual_out=tr)
    assert_bit_exact(host(tr), r_ref, "in-place residual")
    assert_ln_close(host(y1), y_ref, "reverse_add_ln y")


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("grid,shift", GRIDS)
def test_add_norm_gather_small(dev, C, grid, shift):
    n = int(np.prod(grid))
    br = workloads.normal_rows(87, n, C)
    res = workloads.normal_rows(88, n, C, std=3.0)
    t = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    table = oracle.window_index_table(grid, WINDOW, shift)
    r, out = lwg.add_norm_gather(to_dev(br, dev), to_dev(res, dev), t)
    r_ref, out_ref = oracle.add_norm_gather(br, res, table)
    assert_bit_exact(host(r), r_ref, f"add_norm_gather residual C={C} grid={grid}")
    g = host(out)
    assert_ln_close(g, out_ref, f"add_norm_gather C={C} grid={grid}")
    assert not bits(g[table < 0]).any()


@pytest.mark.parametrize("C", [192, 384])
def test_add_norm_gather_aliasing_and_composition(dev, C):
    grid, shift = (4, 9, 26), SHIFT
    n = int(np.prod(grid))
    br = workloads.normal_rows(89, n, C)
    res = workloads.normal_rows(90, n, C)
    t = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    table = oracle.window_index_table(grid, WINDOW, shift)
    r_ref, out_ref = oracle.add_norm_gather(br, res, table)
    tb, tr = to_dev(br, dev), to_dev(res, dev)
    r_sep, _ = lwg.add_ln(tb, tr)
    composed = host(lwg.norm_gather(r_sep, t))
    r1, o1 = lwg.add_norm_gather(tb, tr, t)
    assert_bit_exact(host(o1), composed, "fused vs add_ln then norm_gather")
    lwg.add_norm_gather(tb, tr, t, residual_out=tr)          # in place on the residual
    assert_bit_exact(host(tr), r_ref, "in-place residual")
    tb, tr = to_dev(br, dev), to_dev(res, dev)
    lwg.add_norm_gather(tb, tr, t, residual_out=tb)          # written over the branch
    assert_bit_exact(host(tb), r_ref, "residual over the branch")
    assert_ln_close(host(o1), out_ref, "add_norm_gather out")


@pytest.mark.parametrize("level,seed", [(LEVEL1, 91), (LEVEL2, 92)])
def test_fused_rows_full_size(dev, level, seed):
    n, c = level.tokens, level.channels
    m = oracle.window_token_count(level.grid, WINDOW)
    nc, off = workloads.stress_row_classes(seed, n)
    res = workloads.mixed_rows(seed + 1, n, c, nc, off)
    br = workloads.mixed_rows(seed + 2, n, c, nc, off, offset_mean=0.0)
    attn = workloads.normal_rows(seed + 3, m, c)
    table = oracle.window_index_table(level.grid, WINDOW, SHIFT)
    t = lwg.window_index_build(level.grid, WINDOW, SHIFT, device=dev)
    inv = lwg.window_inverse_build(level.grid, WINDOW, SHIFT, device=dev)
    r, y = lwg.window_reverse_add_ln(to_dev(attn, dev), inv, to_dev(res, dev))
    r_ref, y_ref = oracle.window_reverse_add_ln(attn, res, level.grid, WINDOW, SHIFT)
    assert_bit_exact(host(r), r_ref, f"reverse_add_ln residual {level.name}")
    assert_ln_close(host(y), y_ref, f"reverse_add_ln {level.name}")
    r2, g = lwg.add_norm_gather(to_dev(br, dev), to_dev(res, dev), t)
    r2_ref, g_ref = oracle.add_norm_gather(br, res, table)
    assert_bit_exact(host(r2), r2_ref, f"add_norm_gather residual {level.name}")
    gh = host(g)
    assert_ln_close(gh, g_ref, f"add_norm_gather {level.name}")
    assert not bits(gh[table < 0]).any()


@pytest.mark.parametrize("window", [(1, 1, 1), (3, 5, 7), (8, 7, 7)])
def test_window_inverse_other_windows(dev, window):
    grid = (6, 17, 31)
    for shift in [(0, 0, 0), (1, 2, 3), (5, 40, 100)]:
        inv = host(lwg.window_inverse_build(grid, window, shift, device=dev))
        assert np.array_equal(inv, oracle.window_inverse_table(grid, window, shift)), (window, shift)


def test_in_place_calls_at_level2_size(dev):
    """In-place use at [32760, 384]. There add_ln_affine and add_norm_gather run
    capped, pipelined grids whose waves take more than one row tile (the next
    tile is read before the current one is written); the other kernels run one
    tile per wave. Every in-place result equals the out-of-place one bit for
    bit."""
    lv = workloads.LEVEL2
    n, c = lv.tokens, lv.channels
    x = workloads.normal_rows(81, n, c, mean=0.2, std=1.5)
    res = workloads.normal_rows(82, n, c, std=0.5)
    gamma = workloads.normal_rows(83, 1, c)[0]
    beta = workloads.normal_rows(84, 1, c, std=0.1)[0]
    tg, tbeta = to_dev(gamma, dev), to_dev(beta, dev)

    ref = host(lwg.ln_fixed(to_dev(x, dev)))
    tx = to_dev(x, dev)
    lwg.ln_fixed(tx, out=tx)
    assert_bit_exact(host(tx), ref, "ln_fixed in place at level 2")

    r_ref, y_ref = (host(t) for t in lwg.add_ln(to_dev(x, dev), to_dev(res, dev)))
    assert_bit_exact(r_ref, oracle.residual_sum(res, x), "add_ln residual at level 2")
    tb, tr = to_dev(x, dev), to_dev(res, dev)
    lwg.add_ln(tb, tr, residual_out=tr, out=tb)
    assert_bit_exact(host(tr), r_ref, "add_ln residual in place")
    assert_bit_exact(host(tb), y_ref, "add_ln y over the branch")

    r_ref, y_ref = (host(t) for t in lwg.add_ln_affine(to_dev(x, dev), to_dev(res, dev), tg, tbeta))
    tb, tr = to_dev(x, dev), to_dev(res, dev)
    lwg.add_ln_affine(tb, tr, tg, tbeta, residual_out=tr, out=tb)
    assert_bit_exact(host(tr), r_ref, "add_ln_affine residual in place")
    assert_bit_exact(host(tb), y_ref, "add_ln_affine y over the branch")

    ref = host(lwg.ln_affine(to_dev(x, dev), tg, tbeta))
    tx = to_dev(x, dev)
    lwg.ln_affine(tx, tg, tbeta, out=tx)
    assert_bit_exact(host(tx), ref, "ln_affine in place at level 2")

    table = lwg.window_table(lv.grid, WINDOW, SHIFT, device=dev)
    inv = lwg.window_inverse_table(lv.grid, WINDOW, SHIFT, device=dev)
    win = workloads.normal_rows(85, table.numel(), c)
    r_ref, y_ref = (host(t) for t in lwg.window_reverse_add_ln(to_dev(win, dev), inv, to_dev(res, dev)))
    tr = to_dev(res, dev)
    lwg.window_reverse_add_ln(to_dev(win, dev), inv, tr, residual_out=tr)
    assert_bit_exact(host(tr), r_ref, "window_reverse_add_ln residual in place")

    r_ref, g_ref = (host(t) for t in lwg.add_norm_gather(to_dev(x, dev), to_dev(res, dev), table))
    tb, tr = to_dev(x, dev), to_dev(res, dev)
    _, g = lwg.add_norm_gather(tb, tr, table, residual_out=tr)
    assert_bit_exact(host(tr), r_ref, "add_norm_gather residual in place")
    assert_bit_exact(host(g), g_ref, "add_norm_gather out with the residual in place")


@pytest.mark.parametrize("C", [192, 384, 768])
@pytest.mark.parametrize("eps", [1e-3, 0.5])
def test_eps_reaches_every_layernorm_kernel(dev, C, eps):
    """Every LayerNorm-family call honours its eps. Rows have variance 2.5e-3, so
    eps = 1e-3 or 0.5 moves every output far outside the tolerance of the
    default 1e-5."""
    grid = (2, 7, 13)
    n = int(np.prod(grid))
    x = workloads.normal_rows(91, n, C, mean=0.1, std=0.05)
    res = workloads.normal_rows(92, n, C, std=0.05)
    gamma = workloads.normal_rows(93, 1, C)[0]
    beta = workloads.normal_rows(94, 1, C, std=0.1)[0]
    table = oracle.window_index_table(grid, WINDOW, SHIFT)
    win = workloads.normal_rows(96, table.size, C, std=0.05)
    tx, tr, tg, tb = to_dev(x, dev), to_dev(res, dev), to_dev(gamma, dev), to_dev(beta, dev)
    tt = lwg.window_index_build(grid, WINDOW, SHIFT, device=dev)
    inv = lwg.window_inverse_build(grid, WINDOW, SHIFT, device=dev)
    tag = f"C={C} eps={eps}"
    assert_ln_close(host(lwg.ln_fixed(tx, eps=eps)), oracle.layer_norm(x, eps), f"ln_fixed {tag}")
    _, y = lwg.add_ln(tx, tr, eps=eps)
    assert_ln_close(host(y), oracle.add_ln(x, res, eps)[1], f"add_ln {tag}")
    assert_ln_close(host(lwg.norm_gather(tx, tt, eps=eps)), oracle.norm_gather(x, table, eps), f"norm_gather {tag}")
    _, g = lwg.add_norm_gather(tx, tr, tt, eps=eps)
    assert_ln_close(host(g), oracle.add_norm_gather(x, res, table, eps)[1], f"add_norm_gather {tag}")
    _, y = lwg.window_reverse_add_ln(to_dev(win, dev), inv, tr, eps=eps)
    assert_ln_close(host(y), oracle.window_reverse_add_ln(win, res, grid, WINDOW, SHIFT, eps)[1],
                    f"window_reverse_add_ln {tag}")
    assert_ln_close(host(lwg.ln_affine(tx, tg, tb, eps=eps)), oracle.layer_norm_affine(x, gamma, beta, eps),
                    f"ln_affine {tag}")
    _, y = lwg.add_ln_affine(tx, tr, tg, tb, eps=eps)
    assert_ln_close(host(y), oracle.add_ln_affine(x, res, gamma, beta, eps)[1], f"add_ln_affine {tag}")
    # the default eps would give visibly different rows
    assert np.abs(oracle.layer_norm(x, eps).astype(np.float64) - oracle.layer_norm(x).astype(np.float64)).max() > 0.1

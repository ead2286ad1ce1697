"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: the window tables, the gathers, the FP16 residual and padding rows are
compared bit for bit; normalised outputs must be within max-abs 2e-3 and
mean-abs 1e-4 of the oracle (NaN positions equal). Because the kernels keep
their statistics in binary64, normalised outputs are also expected to be the
same binary16 values as the oracle's almost everywhere; the count of differing
elements is printed and held to a small bound.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import LEVEL1, LEVEL2, TINY, WINDOW, SHIFT, NO_SHIFT

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

from parity_helpers import MAX_ABS, MEAN_ABS, assert_bit_exact, assert_ln_close, bits, host, to_dev  # noqa: E402,F401


RAGGED_ROWS = [1, 3, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 129, 1000, 4097]


# ---------------------------------------------------------------------------
# ln_fixed


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("rows", RAGGED_ROWS)
def test_ln_fixed_ragged(dev, C, rows):
    x = workloads.normal_rows(100 + rows, rows, C, mean=0.3, std=1.7)
    y = host(lwg.ln_fixed(to_dev(x, dev)))
    assert_ln_close(y, oracle.layer_norm(x), f"ln_fixed C={C} rows={rows}")


@pytest.mark.parametrize("C", [192, 384])
def test_ln_fixed_stress_rows(dev, C):
    rows = 3000
    nc, off = workloads.stress_row_classes(7, rows)
    x = workloads.mixed_rows(8, rows, C, nc, off)
    x[5] = np.float16(1.5)                      # constant row -> +0.0
    x[6, :] = np.float16(0.0)
    x[7] = (np.arange(C) % 2 * 2 - 1).astype(np.float16)   # +-1 row -> +-1.0
    x[8] = (workloads.normal_rows(9, 1, C)[0].astype(np.float64) * 50).astype(np.float16)
    x[9] = np.float16(2.0 ** -24) * (np.arange(C) % 3)      # subnormal inputs
    x[10, :] = np.float16(65504.0)
    x[10, ::2] = np.float16(-65504.0)           # extreme two-valued row
    y = host(lwg.ln_fixed(to_dev(x, dev)))
    ref = oracle.layer_norm(x)
    assert_ln_close(y, ref, f"ln_fixed stress C={C}")
    assert not bits(y[5]).any() and not bits(y[6]).any()
    assert_bit_exact(y[7], ref[7], "+-1 row")


@pytest.mark.parametrize("C", [192, 384])
def test_ln_fixed_nonfinite_rows(dev, C):
    x = workloads.normal_rows(10, 40, C)
    x[3, 5] = np.inf
    x[11, 0] = -np.inf
    x[20, C - 1] = np.nan
    y = host(lwg.ln_fixed(to_dev(x, dev)))
    ref = oracle.layer_norm(x)
    for r in (3, 11, 20):
        assert np.isnan(y[r]).all()
    assert_ln_close(y, ref, f"ln_fixed nonfinite C={C}")


@pytest.mark.parametrize("C", [192, 384])
def test_ln_fixed_in_place_and_3d(dev, C):
    x = workloads.normal_rows(11, 2 * 1000, C).reshape(2, 1000, C)
    t = to_dev(x, dev)
    out = lwg.ln_fixed(t, out=t)
    assert out.data_ptr() == t.data_ptr()
    assert_ln_close(host(t).reshape(-1, C), oracle.layer_norm(x.reshape(-1, C)), "in place")


def test_ln_fixed_empty(dev):
    t = torch.empty(0, 192, dtype=torch.float16, device=dev)
    assert lwg.ln_fixed(t).shape == (0, 192)


# ---------------------------------------------------------------------------
# add_ln


def _golden_pairs():
    import json, os
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp16_residual_cases.json")))
    r = np.array([int(c["residual"], 16) for c in spec["cases"]], np.uint16).view(np.float16)
    b = np.array([int(c["branch"], 16) for c in spec["cases"]], np.uint16).view(np.float16)
    return r, b


@pytest.mark.parametrize("C", [192, 384])
def test_add_ln_residual_bit_exact_on_all_kinds_of_pairs(dev, C):
    res, br = workloads.fp16_bit_pattern_pairs(21, 700, C)
    gr, gb = _golden_pairs()
    res[0, : gr.size], br[0, : gb.size] = gr, gb
    r, y = lwg.add_ln(to_dev(br, dev), to_dev(res, dev))
    r_ref = oracle.residual_sum(res, br)
    got_r = host(r)
    g, e = bits(got_r), bits(r_ref)
    nan = np.isnan(r_ref)
    assert np.array_equal(np.isnan(got_r), nan)
    assert np.array_equal(g[~nan], e[~nan])
    assert_ln_close(host(y), oracle.layer_norm(r_ref), f"add_ln y bit-pattern pairs C={C}")


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("rows", [1, 9, 65, 1000, 4097])
def test_add_ln_ragged(dev, C, rows):
    br = workloads.normal_rows(200 + rows, rows, C)
    res = workloads.normal_rows(300 + rows, rows, C, std=4.0)
    r, y = lwg.add_ln(to_dev(br, dev), to_dev(res, dev))
    r_ref, y_ref = oracle.add_ln(br, res)
    assert_bit_exact(host(r), r_ref, f"residual C={C} rows={rows}")
    assert_ln_close(host(y), y_ref, f"add_ln C={C} rows={rows}")


@pytest.mark.parametrize("C", [192, 384])
def test_add_ln_aliasing_modes(dev, C):
    rows = 513
    br = workloads.normal_rows(31, rows, C)
    res = workloads.normal_rows(32, rows, C)
    r_ref, y_ref = oracle.add_ln(br, res)
    # residual updated in place, y separate
    tb, tr = to_dev(br, dev), to_dev(res, dev)
    r, y = lwg.add_ln(tb, tr, residual_out=tr)
    assert r.data_ptr() == tr.data_ptr()
    assert_bit_exact(host(tr), r_ref, "in-place residual")
    assert_ln_close(host(y), y_ref, "y with in-place residual")
    # residual in place, y written over the branch
    tb, tr = to_dev(br, dev), to_dev(res, dev)
    lwg.add_ln(tb, tr, residual_out=tr, out=tb)
    assert_bit_exact(host(tr), r_ref, "residual in place, y over branch")
    assert_ln_close(host(tb), y_ref, "y over branch")
    # residual over the branch, y over the residual
    tb, tr = to_dev(br, dev), to_dev(res, dev)
    lwg.add_ln(tb, tr, residual_out=tb, out=tr)
    assert_bit_exact(host(tb), r_ref, "residual over branch")
    assert_ln_close(host(tr), y_ref, "y over residual")


@pytest.mark.parametrize("C", [192, 384])
def test_add_ln_y_equals_ln_fixed_of_residual(dev, C):
    br = workloads.normal_rows(41, 2000, C)
    res = workloads.normal_rows(42, 2000, C, mean=100.0)
    r, y = lwg.add_ln(to_dev(br, dev), to_dev(res, dev))
    y2 = lwg.ln_fixed(r)
    assert_bit_exact(host(y), host(y2), "add_ln y vs ln_fixed(residual_out)")


# ---------------------------------------------------------------------------
# window tables


TABLE_CASES = [
    ((2, 12, 24), NO_SHIFT), ((2, 12, 24), SHIFT), ((2, 7, 13), SHIFT), ((4, 9, 26), (3, 13, 30)),
    ((1, 1, 1), SHIFT), ((5, 11, 25), (0, 5, 11)), ((8, 20, 30), (8, 24, 36)),
    (LEVEL1.grid, NO_SHIFT), (LEVEL1.grid, SHIFT), (LEVEL2.grid, NO_SHIFT), (LEVEL2.grid, SHIFT),
]


@pytest.mark.parametrize("grid,shift", TABLE_CASES)
def test_window_index_build_bit_exact(dev, grid, shift):
    t = host(lwg.window_index_build(grid, WINDOW, shift, device=dev))
    assert t.dtype == np.int32
    assert np.array_equal(t, oracle.window_index_table(grid, WINDOW, shift))


@pytest.mark.parametrize("window", [(1, 1, 1), (2, 6, 12), (3, 5, 7), (8, 7, 7)])
def test_window_index_build_other_windows(dev, window):
    grid = (6, 17, 31)
    for shift in [(0, 0, 0), (1, 2, 3), (5, 40, 100)]:
        t = host(lwg.window_index_build(grid, window, shift, device=dev))
        assert np.array_equal(t, oracle.window_index_table(grid, window, shift)), (window, shift)


def test_window_table_cache(dev):
    a = lwg.window_table(LEVEL1.grid, WINDOW, SHIFT, device=dev)
    b = lwg.window_table(LEVEL1.grid, WINDOW, SHIFT, device=dev)
    assert a.data_ptr() == b.data_ptr()
    assert lwg.window_index_build((0, 4, 4), WINDOW, NO_SHIFT, device=dev).numel() == 0


# ---------------------------------------------------------------------------
# gathers


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("grid,shift", [((2, 12, 24), SHIFT), ((4, 9, 26), SHIFT), ((3, 13, 25), NO_SHIFT)])
def test_window_gather_bit_exact(dev, C, grid, shift):
    n = int(np.prod(grid))
    x = workloads.normal_rows(51, n, C)
    table = oracle.window_index_table(grid, WINDOW, shift)
    tt = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    out = host(lwg.window_gather(to_dev(x, dev), tt))
    assert_bit_exact(out, oracle.window_gather(x, table), f"gather C={C} grid={grid}")
    assert not bits(out[table < 0]).any()


@pytest.mark.parametrize("C", [192, 384])
def test_gather_out_of_range_entries_are_zero_rows(dev, C):
    x = workloads.normal_rows(53, 300, C)
    table = workloads.table_with_bad_entries(52, 1001, 300)
    tt = to_dev(table, dev)
    out = host(lwg.window_gather(to_dev(x, dev), tt))
    assert_bit_exact(out, oracle.window_gather(x, table), "gather with bad entries")
    ng = host(lwg.norm_gather(to_dev(x, dev), tt))
    assert_ln_close(ng, oracle.norm_gather(x, table), "norm_gather with bad entries")
    bad = (table < 0) | (table >= 300)
    assert not bits(ng[bad]).any()


@pytest.mark.parametrize("C,n_out", [(192, 45061), (384, 45061), (384, 140005), (768, 45061)])
def test_gathers_loop_over_tiles_with_a_ragged_tail(dev, C, n_out):
    # 45,061 output rows end in a part-filled tile at every width; at C = 384
    # the plain gather's waves take two tiles each (all loads first).
    # 140,005 rows at C = 384: past both gathers' large-input thresholds on
    # 256 CUs, so they run their large-input entries.
    n_src = 20000
    x = workloads.normal_rows(71, n_src, C, mean=0.2, std=1.7)
    table = workloads.table_with_bad_entries(72, n_out, n_src)
    tx, tt = to_dev(x, dev), to_dev(table, dev)
    assert_bit_exact(host(lwg.window_gather(tx, tt)), oracle.window_gather(x, table), f"gather C={C} ragged")
    assert_ln_close(host(lwg.norm_gather(tx, tt)), oracle.norm_gather(x, table), f"norm_gather C={C} ragged")


def test_gather_id_encoded_rows(dev):
    grid = LEVEL2.grid
    n = LEVEL2.tokens
    x = np.zeros((n, 384), np.float16)
    ids = np.arange(n)
    x[:, 0] = ids % 2048
    x[:, 1] = ids // 2048
    x[:, 2] = 1.0
    for shift in (NO_SHIFT, SHIFT):
        tt = lwg.window_index_build(grid, WINDOW, shift, device=dev)
        g = host(lwg.window_gather(to_dev(x, dev), tt)).astype(np.int64)
        decoded = np.where(g[:, 2] == 1, g[:, 0] + 2048 * g[:, 1], -1)
        assert np.array_equal(decoded, oracle.window_index_table(grid, WINDOW, shift))


@pytest.mark.parametrize("C", [192, 384])
@pytest.mark.parametrize("grid,shift", [((2, 12, 24), SHIFT), ((4, 9, 26), (3, 13, 30)), ((2, 7, 13), NO_SHIFT)])
def test_norm_gather_parity_and_composition(dev, C, grid, shift):
    n = int(np.prod(grid))
    x = workloads.normal_rows(61, n, C, mean=-0.4, std=3.0)
    table = oracle.window_index_table(grid, WINDOW, shift)
    tx = to_dev(x, dev)
    tt = lwg.window_index_build(grid, WINDOW, shift, device=dev)
    ng = host(lwg.norm_gather(tx, tt))
    assert_ln_close(ng, oracle.norm_gather(x, table), f"norm_gather C={C} grid={grid}")
    assert not bits(ng[table < 0]).any()
    composed = host(lwg.window_gather(lwg.ln_fixed(tx), tt))
    assert_bit_exact(ng, composed, "norm_gather vs window_gather(ln_fixed)")


def test_gather_empty_and_no_source(dev):
    x = torch.zeros(0, 192, dtype=torch.float16, device=dev)
    t = torch.full((37,), -1, dtype=torch.int32, device=dev)
    assert not bits(host(lwg.window_gather(x, t))).any()
    assert not bits(host(lwg.norm_gather(x, t))).any()
    e = torch.empty(0, dtype=torch.int32, device=dev)
    assert lwg.window_gather(to_dev(workloads.normal_rows(1, 4, 192), dev), e).shape == (0, 192)


# ---------------------------------------------------------------------------
# the configurations of the workload at full size, in the benchmark's launch setup


def test_tiny_config(dev):
    x, residual = workloads.tiny_inputs()
    r, y = lwg.add_ln(to_dev(x, dev), to_dev(residual, dev))
    r_ref, y_ref = oracle.add_ln(x, residual)
    assert_bit_exact(host(r), r_ref, "tiny residual")
    assert_ln_close(host(y), y_ref, "tiny y")
    t = lwg.window_index_build(TINY.grid, WINDOW, NO_SHIFT, device=dev)
    table = oracle.window_index_table(TINY.grid, WINDOW, NO_SHIFT)
    assert np.array_equal(host(t), table)
    g = host(lwg.window_gather(y, t))
    assert_bit_exact(g, oracle.window_gather(host(y), table), "tiny gather of the GPU y")
    assert_ln_close(g, oracle.window_gather(y_ref, table), "tiny gather vs oracle chain")


def test_level1_standalone(dev):
    x, residual = workloads.level1_inputs()
    tx = to_dev(x, dev)
    assert_ln_close(host(lwg.ln_fixed(tx)), oracle.layer_norm(x), "level1 ln_fixed")
    r, y = lwg.add_ln(tx, to_dev(residual, dev))
    r_ref, y_ref = oracle.add_ln(x, residual)
    assert_bit_exact(host(r), r_ref, "level1 residual")
    assert_ln_close(host(y), y_ref, "level1 add_ln")


def test_level2_standalone(dev):
    x, residual, scaled = workloads.level2_inputs()
    tx = to_dev(x, dev)
    y = host(lwg.ln_fixed(tx))
    ref = oracle.layer_norm(x)
    assert_ln_close(y, ref, "level2 ln_fixed")
    assert_ln_close(y[scaled], ref[scaled], "level2 ln_fixed x50 rows")
    r, y2 = lwg.add_ln(tx, to_dev(residual, dev))
    r_ref, y2_ref = oracle.add_ln(x, residual)
    assert_bit_exact(host(r), r_ref, "level2 residual")
    assert_ln_close(host(y2), y2_ref, "level2 add_ln")


def test_fused_level1_norm_gather(dev):
    x = workloads.fused_level1_inputs()
    tt = lwg.window_index_build(LEVEL1.grid, WINDOW, SHIFT, device=dev)
    table = oracle.window_index_table(LEVEL1.grid, WINDOW, SHIFT)
    assert tt.numel() == 142848 and int((table == -1).sum()) == 11808
    assert np.array_equal(host(tt), table)
    tx = to_dev(x, dev)
    ng = host(lwg.norm_gather(tx, tt))
    assert_ln_close(ng, oracle.norm_gather(x, table), "fused level1 norm_gather")
    assert not bits(ng[table < 0]).any()
    assert_bit_exact(host(lwg.window_gather(tx, tt)), oracle.window_gather(x, table), "level1 gather")


def test_block_stack_replay(dev):
    """66 calls alternating the two levels, shifted and unshifted windows, with
    the residual stream updated in place. The residual stream is tracked exactly
    by the oracle; normalised outputs are checked on sampled rows (all stress rows
    plus a random sample) at every call."""
    streams = workloads.replay_streams()
    state = {k: (to_dev(v[0], dev), v[0].copy(), v[1], v[2]) for k, v in streams.items()}
    rng = np.random.default_rng(99)
    total_mismatch = 0
    for i, call in enumerate(workloads.replay_schedule()):
        lv = call.level
        t_stream, h_stream, nc, off = state[lv.name]
        label = f"replay call {i} {call.op} {lv.name} shift={call.shift}"
        if call.op == "ln_fixed":
            y = host(lwg.ln_fixed(t_stream))
            total_mismatch += assert_ln_close(y, oracle.layer_norm(h_stream), label)
        elif call.op == "norm_gather":
            tt = lwg.window_table(lv.grid, WINDOW, call.shift, device=dev)
            table = oracle.window_index_table(lv.grid, WINDOW, call.shift)
            out = host(lwg.norm_gather(t_stream, tt))
            inv = np.full(lv.tokens, -1)
            valid = table >= 0
            inv[table[valid]] = np.flatnonzero(valid)
            rows = np.unique(np.concatenate([inv[nc], inv[off], rng.choice(table.size, 2048, replace=False),
                                             np.flatnonzero(~valid)[:64]]))
            total_mismatch += assert_ln_close(out[rows], oracle.norm_gather_rows(h_stream, table, rows), label)
        else:
            br = workloads.replay_branch(call, nc, off)
            _, y = lwg.add_ln(to_dev(br, dev), t_stream, residual_out=t_stream)
            h_stream = oracle.residual_sum(h_stream, br)
            state[lv.name] = (t_stream, h_stream, nc, off)
            assert_bit_exact(host(t_stream), h_stream, label + " residual")
            rows = np.unique(np.concatenate([nc, off, rng.choice(lv.tokens, 2048, replace=False)]))
            total_mismatch += assert_ln_close(host(y)[rows], oracle.layer_norm(h_stream[rows]), label)
    print(f"replay: total normalised mismatches {total_mismatch}")


# ---------------------------------------------------------------------------
# determinism and streams


def test_repeat_runs_are_bitwise_identical(dev):
    x, residual = workloads.level1_inputs()
    tx, tr = to_dev(x, dev), to_dev(residual, dev)
    tt = lwg.window_index_build(LEVEL1.grid, WINDOW, SHIFT, device=dev)
    first = [host(lwg.ln_fixed(tx)), *[host(a) for a in lwg.add_ln(tx, tr)], host(lwg.norm_gather(tx, tt)),
             host(lwg.window_gather(tx, tt))]
    for _ in range(2):
        again = [host(lwg.ln_fixed(tx)), *[host(a) for a in lwg.add_ln(tx, tr)], host(lwg.norm_gather(tx, tt)),
                 host(lwg.window_gather(tx, tt))]
        for a, b in zip(first, again):
            assert np.array_equal(bits(a), bits(b))


def test_runs_on_the_callers_stream(dev):
    x = workloads.normal_rows(71, 50000, 384)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        tx = to_dev(x, dev)
        y = lwg.ln_fixed(tx)
        y2 = lwg.ln_fixed(y)     # ordered after the first call on the same stream
    s.synchronize()
    assert_ln_close(y.cpu().numpy(), oracle.layer_norm(x), "ln on side stream")
    assert_ln_close(y2.cpu().numpy(), oracle.layer_norm(oracle.layer_norm(x)), "chained on side stream")


def test_two_streams_at_once(dev):
    # The kernels keep no state between calls, so work on two streams may run
    # concurrently: each stream chains add_ln -> norm_gather -> ln_fixed on its
    # own buffers (level-1 width on one, level-2 width on the other), issued
    # interleaved, and each result must match the oracle.
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    cases = []
    for k, (grid, C) in enumerate((((4, 30, 40), 192), ((4, 15, 20), 384))):
        n = int(np.prod(grid))
        br = workloads.normal_rows(900 + k, n, C)
        res = workloads.normal_rows(910 + k, n, C, std=0.5)
        cases.append((grid, C, br, res))
    torch.cuda.synchronize(dev)
    outs = []
    for s, (grid, C, br, res) in zip(streams, cases):
        with torch.cuda.stream(s):
            tb, tr = to_dev(br, dev), to_dev(res, dev)
            table = lwg.window_index_build(grid, WINDOW, SHIFT, device=dev)
            outs.append([tb, tr, table])
    for rep in range(3):                 # interleave the two streams' launches
        for s, o in zip(streams, outs):
            with torch.cuda.stream(s):
                tb, tr, table = o[:3]
                r, y = lwg.add_ln(tb, tr, residual_out=tr)
                g = lwg.norm_gather(r, table)
                z = lwg.ln_fixed(y)
                o[3:] = [g, z]
    for s in streams:
        s.synchronize()
    for (grid, C, br, res), o in zip(cases, outs):
        table = oracle.window_index_table(grid, WINDOW, SHIFT)
        r = res
        for _ in range(3):
            r, y = oracle.add_ln(br, r)
        assert_bit_exact(host(o[1]), r, f"two streams: residual C={C}")
        assert_ln_close(host(o[3]), oracle.norm_gather(r, table), f"two streams: norm_gather C={C}")
        assert_ln_close(host(o[4]), oracle.layer_norm(y), f"two streams: ln_fixed C={C}")


def test_cached_tables_built_on_one_stream_serve_another(dev):
    """A cached table first built on a side stream is complete when the call
    returns, and gathers on the default stream read it correctly."""
    grid = (3, 11, 25)
    x = workloads.normal_rows(95, int(np.prod(grid)), 192)
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        t = lwg.window_table(grid, WINDOW, SHIFT, device=dev)
        inv = lwg.window_inverse_table(grid, WINDOW, SHIFT, device=dev)
    out = host(lwg.window_gather(to_dev(x, dev), t))
    assert_bit_exact(out, oracle.window_gather(x, oracle.window_index_table(grid, WINDOW, SHIFT)),
                     "gather with a table built on another stream")
    assert np.array_equal(host(inv), oracle.window_inverse_table(grid, WINDOW, SHIFT))


@pytest.mark.parametrize("shift", [SHIFT, NO_SHIFT])
def test_level2_norm_gather_and_gather_full(dev, shift):
    """norm_gather and window_gather on the whole level-2 tensor [32760, 384]
    (norm_gather one tile per wave, the plain gather two), every row compared."""
    x, _, scaled = workloads.level2_inputs()
    table = oracle.window_index_table(LEVEL2.grid, WINDOW, shift)
    tt = lwg.window_index_build(LEVEL2.grid, WINDOW, shift, device=dev)
    tx = to_dev(x, dev)
    ng = host(lwg.norm_gather(tx, tt))
    assert_ln_close(ng, oracle.norm_gather(x, table), f"level2 norm_gather shift={shift}")
    assert not bits(ng[table < 0]).any()
    assert_bit_exact(host(lwg.window_gather(tx, tt)), oracle.window_gather(x, table), f"level2 gather shift={shift}")

"""Capture of the row operations in a HIP graph (torch.cuda.CUDAGraph).

Every C entry point only enqueues kernels on the caller's stream: no
allocation, no synchronisation, no memset node. So a caller can capture a pass
of the pipeline once and replay it. The test captures one pass of every
operation at each served width (192, 384 and 768) on a ragged, padded, shifted
grid. It replays the
graph several times, copying new inputs in between with eager work and
synchronisations around each replay, and checks every replay bit for bit
against the same calls made eagerly on the same inputs. The eager results of
the first inputs are checked against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import WINDOW, SHIFT

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

from parity_helpers import assert_bit_exact, assert_ln_close, host, to_dev  # noqa: E402

GRID = (4, 13, 25)      # pads to (4, 18, 36) under the (2, 6, 12) window
REPLAYS = 4


def inputs(seed, n, m, C):
    """Host inputs of one replay: fp16 rows for x, branch, residual and the
    window-major attention output, float32 rows and bias for the GELU."""
    xf, bias = workloads.gelu_inputs(seed + 6, 96, C)
    return {
        "x": workloads.normal_rows(seed, n, C, mean=0.3, std=2.0),
        "branch": workloads.normal_rows(seed + 1, n, C),
        "residual": workloads.normal_rows(seed + 2, n, C, std=0.5),
        "win": workloads.normal_rows(seed + 3, m, C),
        "gamma": workloads.normal_rows(seed + 4, 1, C)[0],
        "beta": workloads.normal_rows(seed + 5, 1, C, std=0.1)[0],
        "xf": xf,
        "bias": bias,
    }


def one_pass(t, o):
    """Every row operation once, into the preallocated outputs ``o``."""
    lwg.window_index_build(GRID, WINDOW, SHIFT, out=o["table"])
    lwg.window_inverse_build(GRID, WINDOW, SHIFT, out=o["inverse"])
    lwg.ln_fixed(t["x"], out=o["ln"])
    lwg.add_ln(t["branch"], t["residual"], residual_out=o["add_r"], out=o["add_y"])
    lwg.window_gather(t["x"], o["table"], out=o["gather"])
    lwg.norm_gather(t["x"], o["table"], out=o["norm_gather"])
    lwg.add_norm_gather(t["branch"], t["residual"], o["table"], residual_out=o["ang_r"], out=o["ang"])
    lwg.window_reverse_add_ln(t["win"], o["inverse"], t["residual"], residual_out=o["rev_r"], out=o["rev_y"])
    lwg.ln_affine(t["x"], t["gamma"], t["beta"], out=o["affine"])
    lwg.add_ln_affine(t["branch"], t["residual"], t["gamma"], t["beta"], residual_out=o["aff_r"],
                      out=o["aff_y"])
    lwg.bias_gelu(t["xf"], t["bias"], out=o["gelu"])


def eager(t):
    """The same calls, eagerly, into fresh outputs."""
    table = lwg.window_index_build(GRID, WINDOW, SHIFT, device=t["x"].device)
    inverse = lwg.window_inverse_build(GRID, WINDOW, SHIFT, device=t["x"].device)
    add_r, add_y = lwg.add_ln(t["branch"], t["residual"])
    ang_r, ang = lwg.add_norm_gather(t["branch"], t["residual"], table)
    rev_r, rev_y = lwg.window_reverse_add_ln(t["win"], inverse, t["residual"])
    aff_r, aff_y = lwg.add_ln_affine(t["branch"], t["residual"], t["gamma"], t["beta"])
    return {
        "table": table, "inverse": inverse, "ln": lwg.ln_fixed(t["x"]), "add_r": add_r, "add_y": add_y,
        "gather": lwg.window_gather(t["x"], table), "norm_gather": lwg.norm_gather(t["x"], table),
        "ang_r": ang_r, "ang": ang, "rev_r": rev_r, "rev_y": rev_y,
        "affine": lwg.ln_affine(t["x"], t["gamma"], t["beta"]), "aff_r": aff_r, "aff_y": aff_y,
        "gelu": lwg.bias_gelu(t["xf"], t["bias"]),
    }


def check_against_oracle(h, e, C):
    """Eager results of one input set against the oracle."""
    table = oracle.window_index_table(GRID, WINDOW, SHIFT)
    inverse = oracle.window_inverse_table(GRID, WINDOW, SHIFT)
    assert np.array_equal(host(e["table"]), table)
    assert np.array_equal(host(e["inverse"]), inverse)
    assert_ln_close(host(e["ln"]), oracle.layer_norm(h["x"]), f"graph-case ln_fixed C={C}")
    r, y = oracle.add_ln(h["branch"], h["residual"])
    assert_bit_exact(host(e["add_r"]), r, "graph-case add_ln residual")
    assert_ln_close(host(e["add_y"]), y, f"graph-case add_ln C={C}")
    assert_bit_exact(host(e["gather"]), oracle.window_gather(h["x"], table), "graph-case gather")
    assert_ln_close(host(e["norm_gather"]), oracle.norm_gather(h["x"], table), f"graph-case norm_gather C={C}")
    r, g = oracle.add_norm_gather(h["branch"], h["residual"], table)
    assert_bit_exact(host(e["ang_r"]), r, "graph-case add_norm_gather residual")
    assert_ln_close(host(e["ang"]), g, f"graph-case add_norm_gather C={C}")
    r, y = oracle.window_reverse_add_ln(h["win"], h["residual"], GRID, WINDOW, SHIFT)
    assert_bit_exact(host(e["rev_r"]), r, "graph-case reverse_add_ln residual")
    assert_ln_close(host(e["rev_y"]), y, f"graph-case reverse_add_ln C={C}")
    assert_ln_close(host(e["affine"]), oracle.layer_norm_affine(h["x"], h["gamma"], h["beta"]),
                    f"graph-case ln_affine C={C}")
    r, y = oracle.add_ln_affine(h["branch"], h["residual"], h["gamma"], h["beta"])
    assert_bit_exact(host(e["aff_r"]), r, "graph-case add_ln_affine residual")
    assert_ln_close(host(e["aff_y"]), y, f"graph-case add_ln_affine C={C}")
    ref = oracle.bias_gelu(h["xf"], h["bias"]).astype(np.float64)
    got = host(e["gelu"]).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2e-5 + 2e-5 * np.abs(ref)), "graph-case bias_gelu"


@pytest.mark.parametrize("C", [192, 384, 768])
def test_graph_replays_match_eager_calls(dev, C):
    n = int(np.prod(GRID))
    m = lwg.window_token_count(GRID, WINDOW)
    first = inputs(300 + C, n, m, C)
    t = {k: to_dev(v, dev) for k, v in first.items()}
    e16 = lambda rows: torch.empty(rows, C, dtype=torch.float16, device=dev)  # noqa: E731
    o = {
        "table": torch.empty(m, dtype=torch.int32, device=dev),
        "inverse": torch.empty(n, dtype=torch.int32, device=dev),
        "ln": e16(n), "add_r": e16(n), "add_y": e16(n), "gather": e16(m), "norm_gather": e16(m),
        "ang_r": e16(n), "ang": e16(m), "rev_r": e16(n), "rev_y": e16(n), "affine": e16(n),
        "aff_r": e16(n), "aff_y": e16(n), "gelu": torch.empty_like(t["xf"]),
    }

    # eager warm-up on a side stream (default priority), then capture
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        one_pass(t, o)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass(t, o)
    torch.cuda.synchronize(dev)

    for rep in range(REPLAYS):
        h = first if rep == 0 else inputs(300 + C + 10 * rep, n, m, C)
        for k, v in h.items():
            t[k].copy_(torch.from_numpy(np.ascontiguousarray(v)))
        for v in o.values():       # eager work between replays: poison the outputs
            v.fill_(float("nan")) if v.is_floating_point() else v.fill_(-7)
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        replayed = {k: host(v).copy() for k, v in o.items()}
        ref = eager(t)
        for k, v in ref.items():
            a, b = replayed[k], host(v)
            assert a.dtype == b.dtype and a.shape == b.shape, k
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {rep}: {k} differs from eager"
        if rep == 0:
            check_against_oracle(h, ref, C)


def test_table_first_requested_inside_capture_is_not_cached(dev):
    """A cached window table requested for the first time inside stream capture
    is allocated from the graph's memory and built only when the graph replays,
    so it must not enter the cache: an eager request afterwards builds its own.
    A table cached eagerly beforehand is reused inside capture."""
    grid, shift = (2, 7, 13), (1, 2, 3)                       # a key no other test uses
    key = ((2, 7, 13), tuple(WINDOW), shift, dev.index)
    lwg._tables.pop(key, None)
    C = 192
    n, m = int(np.prod(grid)), lwg.window_token_count(grid, WINDOW)
    x = to_dev(workloads.normal_rows(41, n, C), dev)
    out = torch.empty(m, C, dtype=torch.float16, device=dev)
    cached = lwg.window_table(GRID, WINDOW, SHIFT, device=dev)   # cached eagerly, outside capture

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):                               # warm-up of the gather itself
        lwg.norm_gather(x, lwg.window_index_build(grid, WINDOW, shift, device=dev), out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        t_graph = lwg.window_table(grid, WINDOW, shift, device=dev)
        assert lwg.window_table(GRID, WINDOW, SHIFT, device=dev) is cached
        lwg.norm_gather(x, t_graph, out=out)
    assert key not in lwg._tables
    ref_table = oracle.window_index_table(grid, WINDOW, shift)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        assert np.array_equal(host(t_graph), ref_table)
        assert_ln_close(host(out), oracle.norm_gather(host(x), ref_table), "norm_gather on a captured table")
    eager_table = lwg.window_table(grid, WINDOW, shift, device=dev)
    assert key in lwg._tables and eager_table.data_ptr() != t_graph.data_ptr()
    assert np.array_equal(host(eager_table), ref_table)

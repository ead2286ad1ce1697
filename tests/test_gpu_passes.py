"""Every row kernel at row counts that exercise each launch shape, with every
output element compared against the oracle.

* 45,061 rows at C = 384: 5,633 tiles of 8 rows, 22 per compute unit on
  MI355X's 256: the level-2 entries. ln_fixed, add_ln, window_reverse_add_ln,
  ln_affine and both gathers run one tile per wave; add_ln_affine and
  add_norm_gather run capped grids (2 and 4 workgroups per compute unit) whose
  waves take 1.5-2.8 tiles each. The last tile is part filled
  (45,061 = 8 x 5,632 + 5).
* 140,005 rows at C = 384: 68 tiles per compute unit, past every large-input
  threshold (28 and 48), so ln_fixed, add_ln, window_reverse_add_ln,
  ln_affine, norm_gather and the plain gather take their large-input entries;
  add_ln_affine and add_norm_gather are past their tiles-per-wave limits and
  run one tile per wave. test_large_input_entries_give_the_same_bits checks
  that both entries give the same bits on the same rows.
At C = 192 and 768 the grids at 45,061 rows hold one tile per wave, and the
same counts end in part-filled tiles; at C = 768 that is 44 tiles of 4 rows per
compute unit, past ln_fixed's large-input threshold (40).
"""
import numpy as np
import pytest

import oracle
import workloads

from parity_helpers import assert_bit_exact, assert_ln_close, host, to_dev

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

CASES = [(192, 45061), (384, 45061), (384, 140005), (768, 45061)]


@pytest.fixture(scope="module", params=CASES, ids=lambda c: f"C{c[0]}-rows{c[1]}")
def rows_case(request):
    C, rows = request.param
    nc, off = workloads.stress_row_classes(90 + C, rows)
    res = workloads.mixed_rows(91 + C, rows, C, nc, off)
    br = workloads.mixed_rows(92 + C, rows, C, nc, off, offset_mean=0.0)
    gamma = workloads.normal_rows(93 + C, 1, C)[0]
    beta = workloads.normal_rows(94 + C, 1, C, std=0.1)[0]
    return C, br, res, gamma, beta


def test_ln_and_add_ln(dev, rows_case):
    C, br, res, _, _ = rows_case
    print(f"[passes] ln_fixed / add_ln C={C} rows={len(res)}", flush=True)
    assert_ln_close(host(lwg.ln_fixed(to_dev(res, dev))), oracle.layer_norm(res), f"ln_fixed C={C}")
    r, y = lwg.add_ln(to_dev(br, dev), to_dev(res, dev))
    r_ref, y_ref = oracle.add_ln(br, res)
    assert_bit_exact(host(r), r_ref, f"add_ln residual C={C}")
    assert_ln_close(host(y), y_ref, f"add_ln C={C}")


def test_affine(dev, rows_case):
    C, br, res, gamma, beta = rows_case
    print(f"[passes] ln_affine / add_ln_affine C={C} rows={len(res)}", flush=True)
    tg, tb = to_dev(gamma, dev), to_dev(beta, dev)
    assert_ln_close(host(lwg.ln_affine(to_dev(res, dev), tg, tb)),
                    oracle.layer_norm_affine(res, gamma, beta), f"ln_affine C={C}")
    r, y = lwg.add_ln_affine(to_dev(br, dev), to_dev(res, dev), tg, tb)
    r_ref, y_ref = oracle.add_ln_affine(br, res, gamma, beta)
    assert_bit_exact(host(r), r_ref, f"add_ln_affine residual C={C}")
    assert_ln_close(host(y), y_ref, f"add_ln_affine C={C}")


def test_reverse_add_ln_with_a_permutation(dev, rows_case):
    # the inverse table here is a seeded permutation of more window rows than
    # tokens, so the branch of token i is rows[inverse[i]]
    C, br, res, _, _ = rows_case
    print(f"[passes] window_reverse_add_ln C={C} rows={len(res)}", flush=True)
    n = len(res)
    n_win = n + 1000
    rows = workloads.normal_rows(95 + C, n_win, C)
    inverse = np.random.default_rng(96 + C).permutation(n_win)[:n].astype(np.int32)
    r, y = lwg.window_reverse_add_ln(to_dev(rows, dev), to_dev(inverse, dev), to_dev(res, dev))
    r_ref, y_ref = oracle.add_ln(oracle.window_gather(rows, inverse), res)
    assert_bit_exact(host(r), r_ref, f"window_reverse_add_ln residual C={C}")
    assert_ln_close(host(y), y_ref, f"window_reverse_add_ln C={C}")


def test_add_norm_gather_with_padding(dev, rows_case):
    # every token once, in a seeded order, with -1 padding entries mixed in
    C, br, res, _, _ = rows_case
    print(f"[passes] add_norm_gather C={C} rows={len(res)}", flush=True)
    rng = np.random.default_rng(97 + C)
    table = np.concatenate([np.arange(len(res)), np.full(4099, -1)])
    table = table[rng.permutation(table.size)].astype(np.int32)
    r, g = lwg.add_norm_gather(to_dev(br, dev), to_dev(res, dev), to_dev(table, dev))
    r_ref, g_ref = oracle.add_norm_gather(br, res, table)
    assert_bit_exact(host(r), r_ref, f"add_norm_gather residual C={C}")
    assert_ln_close(host(g), g_ref, f"add_norm_gather C={C}")


def test_gathers_with_padding(dev, rows_case):
    # a seeded order of every token, with -1 padding and out-of-range entries mixed in
    C, _, res, _, _ = rows_case
    print(f"[passes] window_gather / norm_gather C={C} rows={len(res)}", flush=True)
    rng = np.random.default_rng(98 + C)
    table = np.concatenate([np.arange(len(res)), np.full(3001, -1), np.full(7, len(res))])
    table = table[rng.permutation(table.size)].astype(np.int32)
    tx, tt = to_dev(res, dev), to_dev(table, dev)
    assert_bit_exact(host(lwg.window_gather(tx, tt)), oracle.window_gather(res, table), f"window_gather C={C}")
    assert_ln_close(host(lwg.norm_gather(tx, tt)), oracle.norm_gather(res, table), f"norm_gather C={C}")


@pytest.mark.parametrize("C,n,k", [(384, 140005, 40000), (768, 45061, 20000)])
def test_large_input_entries_give_the_same_bits(dev, C, n, k):
    """An input past the large-input thresholds and its first k rows (below
    them) run different launch entries (at C = 768 only ln_fixed has a second
    entry); the shared rows must agree bit for bit, op by op."""
    nc, off = workloads.stress_row_classes(190, n)
    x = to_dev(workloads.mixed_rows(191, n, C, nc, off), dev)
    b = to_dev(workloads.mixed_rows(192, n, C, nc, off, offset_mean=0.0), dev)
    g = to_dev(workloads.normal_rows(193, 1, C)[0], dev)
    bt = to_dev(workloads.normal_rows(194, 1, C, std=0.1)[0], dev)
    table = to_dev(np.random.default_rng(195).permutation(n).astype(np.int32), dev)
    inverse = to_dev(np.random.default_rng(196).permutation(n).astype(np.int32), dev)
    print(f"[passes] large-input entries vs the model-size entries C={C} rows={n}/{k}", flush=True)

    def same(label, full, part):
        full = full if isinstance(full, tuple) else (full,)
        part = part if isinstance(part, tuple) else (part,)
        for f, p in zip(full, part):
            assert_bit_exact(host(f[:k]), host(p), label)

    same("ln_fixed", lwg.ln_fixed(x), lwg.ln_fixed(x[:k]))
    same("add_ln", lwg.add_ln(b, x), lwg.add_ln(b[:k], x[:k]))
    same("ln_affine", lwg.ln_affine(x, g, bt), lwg.ln_affine(x[:k], g, bt))
    same("window_gather", lwg.window_gather(x, table), lwg.window_gather(x, table[:k]))
    same("norm_gather", lwg.norm_gather(x, table), lwg.norm_gather(x, table[:k]))
    same("window_reverse_add_ln", lwg.window_reverse_add_ln(b, inverse, x),
         lwg.window_reverse_add_ln(b, inverse[:k], x[:k]))

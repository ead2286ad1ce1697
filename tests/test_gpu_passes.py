"""Every row kernel at row counts that exercise both launch shapes of the C = 384
kernels, with every output element compared against the oracle.

* 45,061 rows: each wave of the capped C = 384 grids takes 1.5-2.8 row tiles
  (ln_fixed: 3 workgroups per compute unit x 4 waves on 256 CUs = 3,072 waves
  for 5,633 tiles of 8 rows; add_ln: 2,048 waves), within every entry's limit of
  tiles per wave, and the last tile is part filled (45,061 = 8 x 5,632 + 5).
* 140,005 rows (C = 384 only): past every entry's limit, so the same kernels
  run one tile per wave.
At C = 192 and 768 the grids at 45,061 rows hold one tile per wave (C = 768
ln_fixed is past its limit there; it runs capped, with waves looping, at the
32,760-row patch-merge size in tests/test_gpu_widths_affine.py), and the same
counts end in part-filled tiles.
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

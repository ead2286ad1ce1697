"""Parity at the largest sizes: every tensor past 2**31 elements and 2**32 bytes.

Row and byte offsets here overflow 32-bit arithmetic, and the window tables are
built from index values in the tens of millions, so these cases exercise the
64-bit addressing and the multiply-shift divisions that the workload-sized
tests never reach. The grids have ragged extents (1093 and 1297 are not
multiples of the window), so the tables also pad.

What is compared, against the oracle:
* the window index table and its inverse, every entry, bit for bit;
* every gathered row's identity: the inputs carry their row index in three
  exact binary16 digits plus a marker column, so decoding the gathered rows
  must reproduce the oracle's table over all rows;
* sampled rows of each output (the rows around the 2**31-element and
  2**32-byte offsets, the first and last rows, and seeded random rows), bit for
  bit where the result is a copy or the FP16 residual, within the LayerNorm
  tolerance where it is normalised.
"""
import numpy as np
import pytest

import oracle
import workloads
from workloads import LARGE_192, LARGE_384, WINDOW, SHIFT

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

from parity_helpers import assert_bit_exact, assert_ln_close, host, to_dev  # noqa: E402


def boundary_rows(n: int, C: int, seed: int, extra: int = 3000) -> np.ndarray:
    """Row indices to check: the rows whose elements cross 2**31 elements and
    2**32 bytes, the first and last rows, and ``extra`` seeded random rows."""
    picks = [0, 1, 2, n - 3, n - 2, n - 1]
    for cross in ((1 << 31) // C, (1 << 32) // (2 * C)):
        picks += list(range(cross - 3, cross + 4))
    rng = np.random.default_rng(seed)
    picks += list(rng.choice(n, size=extra, replace=False))
    picks = np.unique(np.asarray(picks, dtype=np.int64))
    return picks[(picks >= 0) & (picks < n)]


def output_rows(table: np.ndarray, src_rows: np.ndarray, seed: int, extra: int = 3000) -> np.ndarray:
    """Gathered rows to check: those reading the sampled source rows, the first
    and last rows, the first padding rows, and seeded random rows."""
    m = table.shape[0]
    reads = np.flatnonzero(np.isin(table, src_rows))
    pads = np.flatnonzero(table < 0)[:8]
    rng = np.random.default_rng(seed)
    picks = np.concatenate([reads, pads, [0, 1, m - 2, m - 1], rng.choice(m, size=extra, replace=False)])
    return np.unique(picks.astype(np.int64))


def take(t, rows: np.ndarray) -> np.ndarray:
    """Selected rows of a device tensor, on the host."""
    idx = torch.from_numpy(rows).to(t.device)
    return host(t.index_select(0, idx))


def decode_ids(t) -> np.ndarray:
    """Row index carried by each row of an id-tagged tensor (see
    workloads.id_tagged_rows), or -1 for a row without the marker."""
    d = host(t[:, :4].to(torch.int64))
    ids = d[:, 0] + (d[:, 1] << 10) + (d[:, 2] << 20)
    return np.where(d[:, 3] == 1, ids, -1)


@pytest.fixture(scope="module", params=[LARGE_192, LARGE_384], ids=lambda lv: lv.name)
def big(request, dev):
    """Host and device copies of one large id-tagged input, with its tables."""
    lv = request.param
    n, C = lv.tokens, lv.channels
    print(f"[large] {lv.name}: grid {lv.grid}, {n} rows x {C}", flush=True)
    x = workloads.id_tagged_rows(70 + C, n, C)
    data = {
        "level": lv, "x": x, "tx": to_dev(x, dev),
        "table": oracle.window_index_table(lv.grid, WINDOW, SHIFT),
        "tt": lwg.window_index_build(lv.grid, WINDOW, SHIFT, device=dev),
        "src_rows": boundary_rows(n, C, 80 + C),
    }
    data["out_rows"] = output_rows(data["table"], data["src_rows"], 90 + C)
    yield data
    data.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_large_sizes_pass_32_bit_offsets(big):
    lv = big["level"]
    assert lv.tokens * lv.channels > (1 << 31)
    assert big["table"].shape[0] > lv.tokens  # the grid pads


def test_large_index_and_inverse_tables(dev, big):
    lv = big["level"]
    assert np.array_equal(host(big["tt"]), big["table"])
    inv = host(lwg.window_inverse_build(lv.grid, WINDOW, SHIFT, device=dev))
    assert np.array_equal(inv, oracle.window_inverse_table(lv.grid, WINDOW, SHIFT))


def test_large_window_gather(dev, big):
    x, table, js = big["x"], big["table"], big["out_rows"]
    out = lwg.window_gather(big["tx"], big["tt"])
    assert np.array_equal(decode_ids(out), table), "gathered rows carry the wrong source index"
    assert_bit_exact(take(out, js), oracle.window_gather(x, table[js]), "large gather, sampled rows")


def test_large_norm_gather(dev, big):
    x, table, js = big["x"], big["table"], big["out_rows"]
    ng = lwg.norm_gather(big["tx"], big["tt"])
    assert_ln_close(take(ng, js), oracle.norm_gather_rows(x, table, js), "large norm_gather, sampled rows")
    composed = lwg.window_gather(lwg.ln_fixed(big["tx"]), big["tt"])
    assert torch.equal(ng.view(torch.int16), composed.view(torch.int16)), \
        "norm_gather differs from window_gather(ln_fixed) at large size"


def test_large_ln_fixed(dev, big):
    x, rows = big["x"], big["src_rows"]
    y = lwg.ln_fixed(big["tx"])
    assert_ln_close(take(y, rows), oracle.layer_norm(x[rows]), "large ln_fixed, sampled rows")


def test_large_add_ln(dev, big):
    lv, x, rows = big["level"], big["x"], big["src_rows"]
    residual = workloads.id_tagged_rows(100 + lv.channels, lv.tokens, lv.channels)
    r, y = lwg.add_ln(big["tx"], to_dev(residual, dev))
    ref_r, ref_y = oracle.add_ln(x[rows], residual[rows])
    assert_bit_exact(take(r, rows), ref_r, "large add_ln residual, sampled rows")
    assert_ln_close(take(y, rows), ref_y, "large add_ln y, sampled rows")


def test_large_window_reverse_add_ln(dev, big):
    lv, x, rows = big["level"], big["x"], big["src_rows"]
    m = big["table"].shape[0]
    win = workloads.id_tagged_rows(110 + lv.channels, m, lv.channels)
    inv = oracle.window_inverse_table(lv.grid, WINDOW, SHIFT)
    tinv = lwg.window_inverse_build(lv.grid, WINDOW, SHIFT, device=dev)
    r, y = lwg.window_reverse_add_ln(to_dev(win, dev), tinv, big["tx"])
    ref_r, ref_y = oracle.add_ln(win[inv[rows]], x[rows])
    assert_bit_exact(take(r, rows), ref_r, "large reverse_add_ln residual, sampled rows")
    assert_ln_close(take(y, rows), ref_y, "large reverse_add_ln y, sampled rows")


def test_large_add_norm_gather(dev, big):
    lv, x, table = big["level"], big["x"], big["table"]
    rows, js = big["src_rows"], big["out_rows"]
    branch = workloads.id_tagged_rows(120 + lv.channels, lv.tokens, lv.channels)
    r, out = lwg.add_norm_gather(to_dev(branch, dev), big["tx"], big["tt"])
    assert_bit_exact(take(r, rows), oracle.residual_sum(x[rows], branch[rows]),
                     "large add_norm_gather residual, sampled rows")
    t = table[js]
    ok = t >= 0
    ref = np.zeros((js.size, lv.channels), np.float16)
    ref[ok] = oracle.layer_norm(oracle.residual_sum(x[t[ok]], branch[t[ok]]))
    assert_ln_close(take(out, js), ref, "large add_norm_gather out, sampled rows")


def test_grid_past_2_to_32_work_items(dev):
    """In-place ln_fixed at C = 192 on 2**29 + 1000 rows (192 GiB). One tile per
    wave would take more than 2**32 work-items, which one dispatch cannot count,
    so the launch clamps the grid and the waves loop over the rest. The input
    repeats a seeded block of rows; the rows just below and above 2**29 (the
    last ones the clamped grid's first pass reaches, and the ones only the loop
    reaches), the first and last rows and seeded random rows must all be
    normalised."""
    C, B = 192, 4096
    n = (1 << 29) + 1000
    need = n * C * 2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(dev)
    if free < need + (4 << 30):
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory; {free / 2**30:.0f} GiB free")
    print(f"[large] in-place ln_fixed, {n} rows x {C}", flush=True)
    block = workloads.normal_rows(110, B, C)
    tb = to_dev(block, dev)
    x = torch.empty(n, C, dtype=torch.float16, device=dev)
    q = n // B
    x[: q * B].view(q, B, C).copy_(tb.unsqueeze(0).expand(q, B, C))
    x[q * B:].copy_(tb[: n - q * B])
    lwg.ln_fixed(x, out=x)
    rows = np.unique(np.concatenate([
        np.arange(0, 4), np.arange((1 << 29) - 2048, (1 << 29) + 8), np.arange(n - 1100, n),
        np.random.default_rng(111).choice(n, size=3000, replace=False)]).astype(np.int64))
    got = take(x, rows)
    del x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    assert_ln_close(got, oracle.layer_norm(block[rows % B]), "in-place ln_fixed past 2**32 work-items")

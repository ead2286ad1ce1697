"""The boundary used from plain C: tests/c_client/lwg_c_client.c (C99, only
include/lwg.h and the HIP runtime's C API, built by build()) allocates its own
device buffers and stream, runs ln_fixed, add_ln, window_index_build,
window_gather and norm_gather, and checks that malformed calls are refused with
a message. Its outputs are compared here with the oracle, at the level-1 size
and on ragged padded grids at the other widths."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from workloads import LEVEL1, WINDOW, SHIFT, NO_SHIFT

from parity_helpers import assert_bit_exact, assert_ln_close

pytestmark = pytest.mark.gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "lwg_c_client")
REFUSED = {"width_100": "LWG_ERR_UNSUPPORTED_WIDTH", "misaligned": "LWG_ERR_MISALIGNED",
           "eps_negative": "LWG_ERR_INVALID_ARGUMENT", "table_len": "LWG_ERR_SIZE_MISMATCH",
           "partial_overlap": "LWG_ERR_ALIASING", "null_x": "LWG_ERR_INVALID_ARGUMENT", "empty": "LWG_OK"}


@pytest.mark.parametrize("grid,C,shift", [(LEVEL1.grid, 192, SHIFT), ((4, 13, 25), 384, SHIFT),
                                          ((2, 12, 24), 768, NO_SHIFT)])
def test_c_client_matches_oracle(dev, tmp_path, grid, C, shift):
    assert os.access(BINARY, os.X_OK), "the C client is built by __graft_entry__.build()"
    n = int(np.prod(grid))
    x = workloads.normal_rows(400 + C, n, C, mean=0.2, std=1.5)
    residual = workloads.normal_rows(401 + C, n, C, std=0.5)
    (tmp_path / "meta.txt").write_text(" ".join(map(str, (*grid, C, *WINDOW, *shift))))
    x.tofile(tmp_path / "x.bin")
    residual.tofile(tmp_path / "residual.bin")
    print(f"[c client] grid={grid} C={C} shift={shift}", flush=True)
    res = subprocess.run([BINARY, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr

    def out(name, dtype, cols):
        a = np.fromfile(tmp_path / name, dtype=dtype)
        return a.reshape(-1, cols) if cols else a

    table = oracle.window_index_table(grid, WINDOW, shift)
    assert np.array_equal(out("table.bin", np.int32, 0), table)
    assert_ln_close(out("ln.bin", np.float16, C), oracle.layer_norm(x), f"C client ln_fixed C={C}")
    r, y = oracle.add_ln(x, residual)
    assert_bit_exact(out("add_r.bin", np.float16, C), r, "C client add_ln residual")
    assert_ln_close(out("add_y.bin", np.float16, C), y, f"C client add_ln C={C}")
    assert_bit_exact(out("gather.bin", np.float16, C), oracle.window_gather(x, table), "C client gather")
    assert_ln_close(out("norm_gather.bin", np.float16, C), oracle.norm_gather(x, table),
                    f"C client norm_gather C={C}")
    status = dict(line.split(" ", 2)[:2] for line in (tmp_path / "status.txt").read_text().splitlines())
    assert status == REFUSED

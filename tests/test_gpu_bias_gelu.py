"""Parity of the float32 bias + tanh-GELU kernel with the CPU oracle, at the
shapes of the HIP extension tutorial page ((1024, 768), (4096, 1024),
(8192, 2048)) and on edge values. The gate is the page's own:
allclose(rtol=2e-5, atol=2e-5)."""
import numpy as np
import pytest

import oracle
import workloads

from parity_helpers import host, to_dev

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

RTOL = ATOL = 2e-5


def _close(got, ref, label):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), label
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), label
    ok = ~nan & ~inf
    d = np.abs(got[ok] - ref[ok])
    print(f"[{label}] max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
    assert np.all(d <= ATOL + RTOL * np.abs(ref[ok])), label


@pytest.mark.parametrize("rows,cols", [(1024, 768), (4096, 1024), (8192, 2048), (1, 4), (3, 12), (257, 96)])
def test_bias_gelu_matches_oracle(dev, rows, cols):
    x, b = workloads.gelu_inputs(rows * 7 + cols, rows, cols)
    y = host(lwg.bias_gelu(to_dev(x, dev), to_dev(b, dev)))
    _close(y, oracle.bias_gelu(x, b), f"bias_gelu {rows}x{cols}")


def test_bias_gelu_edge_values_and_in_place(dev):
    vals = np.array([0.0, -0.0, 1e-30, -1e-30, 1e-3, -1e-3, 1.0, -1.0, 3.0, -3.0, 9.0, -9.0, 30.0, -30.0,
                     1e4, -1e4, 3e38, -3e38, np.inf, -np.inf, np.nan, 5.5], np.float32)
    x = np.tile(vals, (8, 1))
    x = np.concatenate([x, np.zeros((8, 2), np.float32)], axis=1)     # 24 columns
    b = np.zeros(24, np.float32)
    b[1::3] = np.float32(0.5)
    tx = to_dev(x, dev)
    y = host(lwg.bias_gelu(tx, to_dev(b, dev)))
    _close(y, oracle.bias_gelu(x, b), "edge values")
    lwg.bias_gelu(tx, to_dev(b, dev), out=tx)
    assert np.array_equal(host(tx).view(np.uint32), y.view(np.uint32))


def test_bias_gelu_matches_the_pages_eager_reference(dev):
    # the page's reference: torch's float32 gelu(input + bias, approximate="tanh")
    xh, bh = workloads.gelu_inputs(20260716, 4096, 1024)
    x, b = to_dev(xh, dev), to_dev(bh, dev)
    ref = torch.nn.functional.gelu(x + b, approximate="tanh")
    assert torch.allclose(lwg.bias_gelu(x, b), ref, rtol=RTOL, atol=ATOL)


def test_bias_gelu_argument_checks(dev):
    x = torch.zeros(4, 8, device=dev)
    with pytest.raises(RuntimeError, match="bias"):
        lwg.bias_gelu(x, torch.zeros(7, device=dev))
    with pytest.raises(RuntimeError, match="float32"):
        lwg.bias_gelu(x.half(), torch.zeros(8, device=dev))
    with pytest.raises(lwg.LwgError, match="multiple of 4"):
        lwg.bias_gelu(torch.zeros(4, 6, device=dev), torch.zeros(6, device=dev))
    assert lwg.bias_gelu(torch.zeros(0, 8, device=dev), torch.zeros(8, device=dev)).shape == (0, 8)

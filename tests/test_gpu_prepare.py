"""prepare() applies the plain functions' argument checks (the input contract of
section 6 of "PyTorch + HIP custom fused operator": device, same device, dtype,
contiguity, rank, parameter length). The C ABI takes no buffer lengths, so a
shape it cannot see would become an out-of-bounds access: every such case must
raise RuntimeError from prepare() itself, before a callable exists and before
anything is enqueued. The outputs of each refused call keep their sentinel.
Well-formed prepared calls give the plain functions' results bit for bit."""
import numpy as np
import pytest

import workloads
from workloads import WINDOW, SHIFT

torch = pytest.importorskip("torch")
lwg = pytest.importorskip("layernorm_window_gather_amd")

pytestmark = pytest.mark.gpu

from parity_helpers import host, to_dev  # noqa: E402

GRID = (2, 12, 24)


def h16(dev, rows, C, seed=0):
    return to_dev(workloads.normal_rows(seed, rows, C), dev)


def sentinel(*ts):
    for t in ts:
        t.fill_(-3.0) if t.is_floating_point() else t.fill_(-5)
    torch.cuda.synchronize()
    return [host(t).copy() for t in ts]


def refused(op, *tensors, untouched=(), **kw):
    """prepare(op, ...) must raise RuntimeError, and the tensors in `untouched`
    must still hold their sentinel afterwards."""
    before = sentinel(*untouched)
    with pytest.raises(RuntimeError):
        lwg.prepare(op, *tensors, **kw)
    torch.cuda.synchronize()
    for t, b in zip(untouched, before):
        assert np.array_equal(host(t).view(np.uint8), b.view(np.uint8)), f"{op}: an output changed"


@pytest.mark.parametrize("C", [192, 384])
def test_prepared_calls_equal_plain_calls(dev, C):
    n = int(np.prod(GRID))
    m = lwg.window_token_count(GRID, WINDOW)
    x, b, r = h16(dev, n, C, 1), h16(dev, n, C, 2), h16(dev, n, C, 3)
    e = lambda rows: torch.empty(rows, C, dtype=torch.float16, device=dev)  # noqa: E731
    table = torch.empty(m, dtype=torch.int32, device=dev)
    inv = torch.empty(n, dtype=torch.int32, device=dev)
    lwg.prepare("window_index_build", table, grid=GRID, window=WINDOW, shift=SHIFT)()
    lwg.prepare("window_inverse_build", inv, grid=GRID, window=WINDOW, shift=SHIFT)()
    assert torch.equal(table, lwg.window_index_build(GRID, WINDOW, SHIFT, device=dev))
    assert torch.equal(inv, lwg.window_inverse_build(GRID, WINDOW, SHIFT, device=dev))
    gamma, beta = h16(dev, 1, C, 4)[0], h16(dev, 1, C, 5)[0]
    win = h16(dev, m, C, 6)
    outs = {k: e(m if k in ("gather", "ng", "ang") else n) for k in
            ("ln", "ar", "ay", "gather", "ng", "rr", "ry", "angr", "ang", "aff", "afr", "afy")}
    lwg.prepare("ln_fixed", x, outs["ln"])()
    lwg.prepare("add_ln", b, r, outs["ar"], outs["ay"])()
    lwg.prepare("window_gather", x, table, outs["gather"])()
    lwg.prepare("norm_gather", x, table, outs["ng"])()
    lwg.prepare("window_reverse_add_ln", win, inv, r, outs["rr"], outs["ry"])()
    lwg.prepare("add_norm_gather", b, r, outs["angr"], table, outs["ang"])()
    lwg.prepare("ln_affine", x, gamma, beta, outs["aff"])()
    lwg.prepare("add_ln_affine", b, r, gamma, beta, outs["afr"], outs["afy"])()
    xf, bias = (to_dev(a, dev) for a in workloads.gelu_inputs(7, 64, 256))
    gelu = torch.empty_like(xf)
    lwg.prepare("bias_gelu", xf, bias, gelu)()
    ar, ay = lwg.add_ln(b, r)
    rr, ry = lwg.window_reverse_add_ln(win, inv, r)
    angr, ang = lwg.add_norm_gather(b, r, table)
    afr, afy = lwg.add_ln_affine(b, r, gamma, beta)
    ref = {"ln": lwg.ln_fixed(x), "ar": ar, "ay": ay, "gather": lwg.window_gather(x, table),
           "ng": lwg.norm_gather(x, table), "rr": rr, "ry": ry, "angr": angr, "ang": ang,
           "aff": lwg.ln_affine(x, gamma, beta), "afr": afr, "afy": afy}
    for k, v in ref.items():
        assert torch.equal(outs[k].view(torch.int16), v.view(torch.int16)), k
    assert torch.equal(gelu.view(torch.int32), lwg.bias_gelu(xf, bias).view(torch.int32))


def test_prepare_refuses_bad_bias_gelu(dev):
    xf, bias = (to_dev(a, dev) for a in workloads.gelu_inputs(8, 64, 256))
    y = torch.empty_like(xf)
    refused("bias_gelu", xf, bias[:128].contiguous(), y, untouched=(y,))          # short bias
    refused("bias_gelu", xf, bias.half(), y, untouched=(y,))                       # bias dtype
    refused("bias_gelu", xf, bias, y[:32], untouched=(y,))                         # short output
    wide = torch.empty(64, 512, dtype=torch.float32, device=dev)
    refused("bias_gelu", xf, bias, wide[:, ::2], untouched=(wide,))               # non-contiguous output
    refused("bias_gelu", xf, bias, torch.empty(64, 256), untouched=(y,))          # output on the host
    refused("bias_gelu", xf, bias.cpu(), y, untouched=(y,))                       # bias on the host


@pytest.mark.parametrize("C", [192, 384])
def test_prepare_refuses_mismatched_branch(dev, C):
    n = int(np.prod(GRID))
    m = lwg.window_token_count(GRID, WINDOW)
    table = lwg.window_table(GRID, WINDOW, SHIFT, device=dev)
    b, r = h16(dev, n, C, 1), h16(dev, n, C, 2)
    ro, out, y = h16(dev, n, C, 3), h16(dev, m, C, 4), h16(dev, n, C, 5)
    short_b = h16(dev, n - 8, C, 6)
    other_w = h16(dev, n, 768 if C == 384 else 384, 7)
    gamma, beta = h16(dev, 1, C, 8)[0], h16(dev, 1, C, 9)[0]
    # add_norm_gather: branch shape != residual shape, branch width, branch on the host
    refused("add_norm_gather", short_b, r, ro, table, out, untouched=(ro, out))
    refused("add_norm_gather", other_w, r, ro, table, out, untouched=(ro, out))
    refused("add_norm_gather", b.cpu(), r, ro, table, out, untouched=(ro, out))
    # add_ln_affine: branch shape != residual shape, short gamma
    refused("add_ln_affine", short_b, r, gamma, beta, ro, y, untouched=(ro, y))
    refused("add_ln_affine", b, r, gamma[:C // 2].contiguous(), beta, ro, y, untouched=(ro, y))
    # add_ln: branch shape, output shape
    refused("add_ln", short_b, r, ro, y, untouched=(ro, y))
    refused("add_ln", b, r, ro, y[: n - 8], untouched=(ro, y))


@pytest.mark.parametrize("C", [192, 384])
def test_prepare_refuses_bad_window_reverse(dev, C):
    n = int(np.prod(GRID))
    m = lwg.window_token_count(GRID, WINDOW)
    inv = lwg.window_inverse_table(GRID, WINDOW, SHIFT, device=dev)
    r, ro, y = h16(dev, n, C, 1), h16(dev, n, C, 2), h16(dev, n, C, 3)
    narrow = h16(dev, m, 192 if C == 384 else 384, 4)          # rows of another width
    win = h16(dev, m, C, 5)
    refused("window_reverse_add_ln", narrow, inv, r, ro, y, untouched=(ro, y))
    refused("window_reverse_add_ln", win.cpu(), inv, r, ro, y, untouched=(ro, y))
    refused("window_reverse_add_ln", win, inv[:-1].contiguous(), r, ro, y, untouched=(ro, y))
    refused("window_reverse_add_ln", win, inv.long(), r, ro, y, untouched=(ro, y))
    refused("window_reverse_add_ln", win, inv, r, ro, y[:-1], untouched=(ro, y))


@pytest.mark.parametrize("C", [192, 384])
def test_prepare_refuses_bad_gathers_and_rows(dev, C):
    n = int(np.prod(GRID))
    m = lwg.window_token_count(GRID, WINDOW)
    table = lwg.window_table(GRID, WINDOW, SHIFT, device=dev)
    x, out, y = h16(dev, n, C, 1), h16(dev, m, C, 2), h16(dev, n, C, 3)
    for op in ("window_gather", "norm_gather"):
        refused(op, x, table, out[:-1], untouched=(out,))                             # short output
        refused(op, x, table.long(), out, untouched=(out,))                           # int64 table
        wide_t = torch.empty(2 * m, dtype=torch.int32, device=dev)
        refused(op, x, wide_t[::2], out, untouched=(out,))                            # strided table
        refused(op, x, table.cpu(), out, untouched=(out,))                            # table on the host
    refused("ln_fixed", x, y[:-1], untouched=(y,))
    wide = torch.empty(n, 2 * C, dtype=torch.float16, device=dev)
    refused("ln_fixed", x, wide[:, :C], untouched=(wide,))                            # non-contiguous
    refused("ln_affine", x, h16(dev, 1, C, 4)[0][: C - 8].contiguous(), h16(dev, 1, C, 5)[0], y, untouched=(y,))
    t_short = torch.empty(m - 1, dtype=torch.int32, device=dev)
    refused("window_index_build", t_short, grid=GRID, window=WINDOW, shift=SHIFT, untouched=(t_short,))
    i_short = torch.empty(n - 1, dtype=torch.int32, device=dev)
    refused("window_inverse_build", i_short, grid=GRID, window=WINDOW, shift=SHIFT, untouched=(i_short,))

"""MI355X (gfx950) row pipeline of a Pangu-Weather-style shifted-window transformer.

Thin PyTorch binding over liblwg.so (include/lwg.h). PyTorch provides device
memory and the current stream; every computation runs in the library's HIP
kernels. Each function checks its tensors, allocates outputs that were not
given, and calls the matching ``lwg_*`` entry point on
``torch.cuda.current_stream(device)``. There is no CPU path: CPU tensors are
refused.

Operations (page "Pangu-Weather inference optimisation on Hygon BW1000
(gfx936)", sections 3-5):
  ln_fixed(x)                        LayerNorm of rows of width 192/384/768, no affine
  add_ln(branch, residual)           (FP16(residual + branch), LayerNorm of it)
  window_token_count(grid, window)   rows of the padded, windowed tensor
  window_index_build(grid, window, shift)   INT32 table built on the device
  window_table(grid, window, shift)  the same, cached per key and device
  window_gather(x, table)            out[j] = x[table[j]], or zeros for -1
  norm_gather(x, table)              out[j] = LayerNorm(x[table[j]]), or zeros

and the window reverse that follows attention, plus the two fusions around it:
  window_inverse_build(grid, window, shift)  token -> gathered row, on the device
  window_inverse_table(grid, window, shift)  the same, cached
  window_reverse(rows, inverse)      rows back to token order (a gather by inverse)
  window_reverse_add_ln(rows, inverse, residual)  reverse + add + LayerNorm
  add_norm_gather(branch, residual, table)        add + LayerNorm + gather

and, for callers that keep the LayerNorm scale and shift:
  ln_affine(x, gamma, beta), add_ln_affine(branch, residual, gamma, beta)

and the float32 bias + tanh-GELU of the HIP extension tutorial:
  bias_gelu(x, bias)                 gelu_tanh(x + bias), float32

Row widths: 192 and 384 (the model's) and 768 (its patch-merge width).
prepare(op, ...) checks the arguments once and returns a callable that only
crosses the C ABI (for timing loops).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LwgError

__all__ = [
    "ln_fixed", "add_ln", "window_token_count", "window_index_build", "window_table", "window_gather",
    "norm_gather", "window_inverse_build", "window_inverse_table", "window_reverse", "window_reverse_add_ln",
    "add_norm_gather", "ln_affine", "add_ln_affine", "bias_gelu", "prepare", "library", "LwgError", "WIDTHS",
    "EPS",
]

WIDTHS = (192, 384, 768)
EPS = 1e-5


def library():
    """The loaded ctypes handle of liblwg.so (raises if it is not built)."""
    return _lib.load()


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _rows(t: torch.Tensor, name: str) -> int:
    """Check a [..., C] binary16 device tensor; return its row count."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float16:
        raise RuntimeError(f"{name} must be float16, got {t.dtype}")
    if t.dim() < 1 or t.shape[-1] not in WIDTHS:
        raise RuntimeError(f"{name} must have last dimension 192, 384 or 768, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise RuntimeError(f"{name} must be on a GPU device, got {t.device}")
    return t.numel() // t.shape[-1]


def _same_device(ref: torch.Tensor, *others):
    for name, t in others:
        if t.device != ref.device:
            raise RuntimeError(f"{name} is on {t.device}, expected {ref.device}")


def _out_like(out, shape, device, name):
    if out is None:
        return torch.empty(shape, dtype=torch.float16, device=device)
    _rows(out, name)
    if tuple(out.shape) != tuple(shape):
        raise RuntimeError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.device != device:
        raise RuntimeError(f"{name} is on {out.device}, expected {device}")
    return out


# Argument checks shared by the plain functions and prepare(): the C ABI takes
# no buffer lengths, so every size, shape, dtype, layout and device relation it
# relies on is checked here before any call crosses it (section 6 of "PyTorch +
# HIP custom fused operator": device, same device, dtype, contiguity, rank,
# parameter length).

def _check_ln(x, y) -> int:
    rows = _rows(x, "x")
    _out_like(y, x.shape, x.device, "out")
    return rows


def _check_add_ln(branch, residual, residual_out, y) -> int:
    rows = _rows(residual, "residual")
    _rows(branch, "branch")
    if tuple(branch.shape) != tuple(residual.shape):
        raise RuntimeError(f"branch shape {tuple(branch.shape)} != residual shape {tuple(residual.shape)}")
    _same_device(residual, ("branch", branch))
    _out_like(residual_out, residual.shape, residual.device, "residual_out")
    _out_like(y, residual.shape, residual.device, "out")
    return rows


def _check_gather(x, table, out, name) -> int:
    n_src, shape = _gather_args(x, table, name)
    _out_like(out, shape, x.device, "out")
    return n_src


def _check_reverse_add_ln(rows, inverse, residual, residual_out, y):
    n_win = _rows(rows, "rows")
    n = _rows(residual, "residual")
    if rows.shape[-1] != residual.shape[-1]:
        raise RuntimeError(f"rows width {rows.shape[-1]} != residual width {residual.shape[-1]}")
    if not isinstance(inverse, torch.Tensor) or inverse.dtype != torch.int32 or inverse.dim() != 1 \
            or not inverse.is_contiguous() or inverse.numel() != n:
        raise RuntimeError("inverse must be a contiguous 1-D int32 tensor with one entry per residual row")
    _same_device(residual, ("rows", rows), ("inverse", inverse))
    _out_like(residual_out, residual.shape, residual.device, "residual_out")
    _out_like(y, residual.shape, residual.device, "out")
    return n_win, n


def _check_add_norm_gather(branch, residual, residual_out, table, out) -> int:
    n_src, shape = _gather_args(residual, table, "add_norm_gather")
    _rows(branch, "branch")
    if tuple(branch.shape) != tuple(residual.shape):
        raise RuntimeError(f"branch shape {tuple(branch.shape)} != residual shape {tuple(residual.shape)}")
    _same_device(residual, ("branch", branch))
    _out_like(residual_out, residual.shape, residual.device, "residual_out")
    _out_like(out, shape, residual.device, "out")
    return n_src


def _affine_params(gamma, beta, C, device):
    for name, t in (("gamma", gamma), ("beta", beta)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or t.dim() != 1 or t.numel() != C:
            raise RuntimeError(f"{name} must be a 1-D float16 tensor of length {C}")
        if not t.is_contiguous() or t.device != device:
            raise RuntimeError(f"{name} must be contiguous and on {device}")


def _check_ln_affine(x, gamma, beta, y) -> int:
    rows = _rows(x, "x")
    _affine_params(gamma, beta, x.shape[-1], x.device)
    _out_like(y, x.shape, x.device, "out")
    return rows


def _check_add_ln_affine(branch, residual, gamma, beta, residual_out, y) -> int:
    rows = _check_add_ln(branch, residual, residual_out, y)
    _affine_params(gamma, beta, residual.shape[-1], residual.device)
    return rows


def _check_bias_gelu(x, bias, out):
    for name, t in (("x", x), ("bias", bias), ("out", out)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
            raise RuntimeError(f"{name} must be a float32 tensor")
        if not t.is_contiguous():
            raise RuntimeError(f"{name} must be contiguous")
        if t.device.type != "cuda":
            raise RuntimeError(f"{name} must be on a GPU device, got {t.device}")
    if x.dim() < 1 or bias.dim() != 1 or bias.numel() != x.shape[-1]:
        raise RuntimeError("bias must be 1-D with one entry per column of x")
    if tuple(out.shape) != tuple(x.shape):
        raise RuntimeError(f"out has shape {tuple(out.shape)}, expected {tuple(x.shape)}")
    _same_device(x, ("bias", bias), ("out", out))
    cols = x.shape[-1]
    return (x.numel() // cols if cols else 0), cols


def _check_table_out(t, n, name):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device.type != "cuda" \
            or not t.is_contiguous() or t.dim() != 1:
        raise RuntimeError(f"{name} must be a contiguous 1-D int32 GPU tensor")
    if t.numel() != n:
        raise RuntimeError(f"{name} has {t.numel()} entries, expected {n}")


def ln_fixed(x: torch.Tensor, eps: float = EPS, out: torch.Tensor = None) -> torch.Tensor:
    """LayerNorm over the last dimension (192, 384 or 768) without affine; ``out`` may be ``x``."""
    _rows(x, "x")
    y = torch.empty(x.shape, dtype=torch.float16, device=x.device) if out is None else out
    rows = _check_ln(x, y)
    lib = _lib.load()
    with torch.cuda.device(x.device):
        _lib.check(lib.lwg_ln_fixed(_ptr(x), _ptr(y), rows, x.shape[-1], float(eps), _stream(x.device)))
    return y


def add_ln(branch: torch.Tensor, residual: torch.Tensor, eps: float = EPS,
           residual_out: torch.Tensor = None, out: torch.Tensor = None):
    """Returns (FP16(residual + branch), LayerNorm of it). ``residual_out`` may be
    ``residual`` or ``branch`` (in-place update); ``out`` may be either input."""
    _rows(residual, "residual")
    r = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if residual_out is None \
        else residual_out
    y = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if out is None else out
    rows = _check_add_ln(branch, residual, r, y)
    lib = _lib.load()
    with torch.cuda.device(residual.device):
        _lib.check(lib.lwg_add_ln(_ptr(branch), _ptr(residual), _ptr(r), _ptr(y), rows,
                                  residual.shape[-1], float(eps), _stream(residual.device)))
    return r, y


def ln_affine(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = EPS,
              out: torch.Tensor = None) -> torch.Tensor:
    """LayerNorm over the last dimension with a per-channel scale and shift."""
    _rows(x, "x")
    y = torch.empty(x.shape, dtype=torch.float16, device=x.device) if out is None else out
    rows = _check_ln_affine(x, gamma, beta, y)
    lib = _lib.load()
    with torch.cuda.device(x.device):
        _lib.check(lib.lwg_ln_affine(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, x.shape[-1], float(eps),
                                     _stream(x.device)))
    return y


def add_ln_affine(branch: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
                  eps: float = EPS, residual_out: torch.Tensor = None, out: torch.Tensor = None):
    """Returns (FP16(residual + branch), affine LayerNorm of it)."""
    _rows(residual, "residual")
    r = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if residual_out is None \
        else residual_out
    y = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if out is None else out
    rows = _check_add_ln_affine(branch, residual, gamma, beta, r, y)
    lib = _lib.load()
    with torch.cuda.device(residual.device):
        _lib.check(lib.lwg_add_ln_affine(_ptr(branch), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(r), _ptr(y),
                                         rows, residual.shape[-1], float(eps), _stream(residual.device)))
    return r, y


def bias_gelu(x: torch.Tensor, bias: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """float32 gelu(x + bias, tanh form) over the last dimension; ``out`` may be ``x``."""
    if out is None and isinstance(x, torch.Tensor):
        out = torch.empty_like(x)
    rows, cols = _check_bias_gelu(x, bias, out)
    lib = _lib.load()
    with torch.cuda.device(x.device):
        _lib.check(lib.lwg_bias_gelu(_ptr(x), _ptr(bias), _ptr(out), rows, cols, _stream(x.device)))
    return out


def _triple(v, name):
    v = tuple(int(a) for a in v)
    if len(v) != 3:
        raise ValueError(f"{name} must have three entries (z, h, w)")
    return v


def window_token_count(grid, window) -> int:
    """Rows of the gathered tensor: product of the extents padded up to the window."""
    g, w = _triple(grid, "grid"), _triple(window, "window")
    n = _lib.load().lwg_window_token_count(*g, *w)
    if n < 0:
        raise RuntimeError(f"invalid grid {g} / window {w}")
    return int(n)


def window_index_build(grid, window, shift=(0, 0, 0), device=None, out: torch.Tensor = None) -> torch.Tensor:
    """Build the INT32 shifted-window index table on the device (one kernel)."""
    g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
    m = window_token_count(g, w)
    if out is None:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        if dev.type != "cuda":
            raise RuntimeError(f"window tables live on a GPU device, got {dev}")
        out = torch.empty(m, dtype=torch.int32, device=dev)
    _check_table_out(out, m, "out")
    lib = _lib.load()
    with torch.cuda.device(out.device):
        _lib.check(lib.lwg_window_index_build(*g, *w, *s, ctypes.c_void_p(out.data_ptr()), out.numel(),
                                              _stream(out.device)))
    return out


_tables = {}


def _cached_build(cache, key, build, dev):
    """A table from ``cache``, or built now. A table built outside stream capture
    is waited for and cached, so that any stream may read it later. One first
    requested inside stream capture is returned uncached: it is allocated from the
    graph's memory and only built when the graph replays, so an eager call later
    builds (and caches) its own."""
    t = cache.get(key)
    if t is not None:
        return t
    t = build()
    with torch.cuda.device(dev):
        if torch.cuda.is_current_stream_capturing():
            return t
        torch.cuda.current_stream(dev).synchronize()
    cache[key] = t
    return t


def _table_device(device) -> torch.device:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if dev.type != "cuda":
        raise RuntimeError(f"window tables live on a GPU device, got {dev}")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    return dev


def window_table(grid, window, shift=(0, 0, 0), device=None) -> torch.Tensor:
    """Cached ``window_index_build``: one table per (grid, window, shift, device).
    The table is built on the device's current stream at first use, and that
    first call waits for it, so later calls may use it on any stream (a first
    call inside stream capture returns a table of that graph, uncached)."""
    g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
    dev = _table_device(device)
    return _cached_build(_tables, (g, w, s, dev.index), lambda: window_index_build(g, w, s, device=dev), dev)


def _gather_args(x, table, name):
    n_src = _rows(x, "x")
    if not isinstance(table, torch.Tensor) or table.dtype != torch.int32 or table.dim() != 1:
        raise RuntimeError("table must be a 1-D int32 tensor")
    if not table.is_contiguous():
        raise RuntimeError("table must be contiguous")
    _same_device(x, ("table", table))
    if x.dim() == 3 and x.shape[0] != 1:
        raise RuntimeError(f"{name} gathers one [N, C] slab; got shape {tuple(x.shape)}")
    if x.dim() not in (2, 3):
        raise RuntimeError(f"x must be [N, C] or [1, N, C], got {tuple(x.shape)}")
    shape = (table.numel(), x.shape[-1]) if x.dim() == 2 else (1, table.numel(), x.shape[-1])
    return n_src, shape


def window_gather(x: torch.Tensor, table: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """out[j] = x[table[j]] for 0 <= table[j] < N, else a +0.0 row."""
    _, shape = _gather_args(x, table, "window_gather")
    o = torch.empty(shape, dtype=torch.float16, device=x.device) if out is None else out
    n_src = _check_gather(x, table, o, "window_gather")
    lib = _lib.load()
    with torch.cuda.device(x.device):
        _lib.check(lib.lwg_window_gather(_ptr(x), n_src, x.shape[-1], _ptr(table), table.numel(),
                                         _ptr(o), _stream(x.device)))
    return o


def norm_gather(x: torch.Tensor, table: torch.Tensor, eps: float = EPS,
                out: torch.Tensor = None) -> torch.Tensor:
    """out[j] = LayerNorm(x[table[j]]) for 0 <= table[j] < N, else a +0.0 row;
    the normalised tensor itself is never written."""
    _, shape = _gather_args(x, table, "norm_gather")
    o = torch.empty(shape, dtype=torch.float16, device=x.device) if out is None else out
    n_src = _check_gather(x, table, o, "norm_gather")
    lib = _lib.load()
    with torch.cuda.device(x.device):
        _lib.check(lib.lwg_norm_gather(_ptr(x), n_src, x.shape[-1], _ptr(table), table.numel(),
                                       float(eps), _ptr(o), _stream(x.device)))
    return o


def _token_count(grid) -> int:
    g = _triple(grid, "grid")
    if min(g) < 0:
        raise RuntimeError(f"invalid grid {g}")
    return g[0] * g[1] * g[2]


def window_inverse_build(grid, window, shift=(0, 0, 0), device=None, out: torch.Tensor = None) -> torch.Tensor:
    """Build the INT32 inverse table (token -> gathered row) on the device."""
    g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
    n = _token_count(g)
    if out is None:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        if dev.type != "cuda":
            raise RuntimeError(f"window tables live on a GPU device, got {dev}")
        out = torch.empty(n, dtype=torch.int32, device=dev)
    _check_table_out(out, n, "out")
    lib = _lib.load()
    with torch.cuda.device(out.device):
        _lib.check(lib.lwg_window_inverse_build(*g, *w, *s, ctypes.c_void_p(out.data_ptr()), out.numel(),
                                                _stream(out.device)))
    return out


_inverses = {}


def window_inverse_table(grid, window, shift=(0, 0, 0), device=None) -> torch.Tensor:
    """Cached ``window_inverse_build``: one table per (grid, window, shift, device),
    waited for at first use like ``window_table``."""
    g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
    dev = _table_device(device)
    return _cached_build(_inverses, (g, w, s, dev.index), lambda: window_inverse_build(g, w, s, device=dev), dev)


def window_reverse(rows: torch.Tensor, inverse: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """Window-ordered rows back to token order: out[i] = rows[inverse[i]]. This is
    the window gather driven by the inverse table (the same kernel)."""
    return window_gather(rows, inverse, out=out)


def window_reverse_add_ln(rows: torch.Tensor, inverse: torch.Tensor, residual: torch.Tensor,
                          eps: float = EPS, residual_out: torch.Tensor = None, out: torch.Tensor = None):
    """Returns (FP16(residual + rows[inverse]), LayerNorm of it): the window reverse
    of an attention output fused with the residual add + LayerNorm."""
    _rows(residual, "residual")
    r = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if residual_out is None \
        else residual_out
    y = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if out is None else out
    n_win, n = _check_reverse_add_ln(rows, inverse, residual, r, y)
    lib = _lib.load()
    with torch.cuda.device(residual.device):
        _lib.check(lib.lwg_window_reverse_add_ln(_ptr(rows), n_win, _ptr(inverse), _ptr(residual), _ptr(r),
                                                 _ptr(y), n, residual.shape[-1], float(eps),
                                                 _stream(residual.device)))
    return r, y


def add_norm_gather(branch: torch.Tensor, residual: torch.Tensor, table: torch.Tensor, eps: float = EPS,
                    residual_out: torch.Tensor = None, out: torch.Tensor = None):
    """Returns (FP16(residual + branch), gathered LayerNorm of it): out[j] is the
    LayerNorm of residual_out[table[j]], or zeros for padding. The table's valid
    entries must be distinct and cover every token (window_index_build's are)."""
    _, shape = _gather_args(residual, table, "add_norm_gather")
    r = torch.empty(residual.shape, dtype=torch.float16, device=residual.device) if residual_out is None \
        else residual_out
    o = torch.empty(shape, dtype=torch.float16, device=residual.device) if out is None else out
    n_src = _check_add_norm_gather(branch, residual, r, table, o)
    lib = _lib.load()
    with torch.cuda.device(residual.device):
        _lib.check(lib.lwg_add_norm_gather(_ptr(branch), _ptr(residual), _ptr(r), n_src, residual.shape[-1],
                                           _ptr(table), table.numel(), float(eps), _ptr(o),
                                           _stream(residual.device)))
    return r, o


class Prepared:
    """A checked, pre-marshalled call of one C entry point on fixed tensors and a
    fixed stream (the device's current stream when prepared). Calling it only
    crosses the C ABI, which repeats its own argument checks; use it where the
    per-call Python checks would cost more than the kernel (timed loops).
    The tensors must stay alive and unchanged in shape while it is used."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        _lib.check(self._fn(*self._args))


def prepare(op: str, *tensors, eps: float = EPS, grid=None, window=None, shift=(0, 0, 0)) -> Prepared:
    """Prepare ``op`` on the given tensors, checked as the plain functions check them:
      prepare("ln_fixed", x, y)
      prepare("add_ln", branch, residual, residual_out, y)
      prepare("window_index_build", table, grid=..., window=..., shift=...)
      prepare("window_gather", x, table, out)
      prepare("norm_gather", x, table, out)
      prepare("window_inverse_build", inverse, grid=..., window=..., shift=...)
      prepare("window_reverse_add_ln", rows, inverse, residual, residual_out, y)
      prepare("add_norm_gather", branch, residual, residual_out, table, out)
      prepare("ln_affine", x, gamma, beta, y)
      prepare("add_ln_affine", branch, residual, gamma, beta, residual_out, y)
      prepare("bias_gelu", x, bias, y)
    Every argument error raises RuntimeError here, before anything is enqueued."""
    lib = _lib.load()
    if op == "ln_fixed":
        x, y = tensors
        rows = _check_ln(x, y)
        dev = x.device
        fn, args = lib.lwg_ln_fixed, (_ptr(x), _ptr(y), rows, x.shape[-1], float(eps), _stream(dev))
    elif op == "add_ln":
        b, r, ro, y = tensors
        rows = _check_add_ln(b, r, ro, y)
        dev = r.device
        fn, args = lib.lwg_add_ln, (_ptr(b), _ptr(r), _ptr(ro), _ptr(y), rows, r.shape[-1], float(eps),
                                    _stream(dev))
    elif op == "window_index_build":
        (table,) = tensors
        g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
        _check_table_out(table, window_token_count(g, w), "table")
        dev = table.device
        fn, args = lib.lwg_window_index_build, (*g, *w, *s, _ptr(table), table.numel(), _stream(dev))
    elif op in ("window_gather", "norm_gather"):
        x, table, out = tensors
        n_src = _check_gather(x, table, out, op)
        dev = x.device
        if op == "window_gather":
            fn, args = lib.lwg_window_gather, (_ptr(x), n_src, x.shape[-1], _ptr(table), table.numel(),
                                               _ptr(out), _stream(dev))
        else:
            fn, args = lib.lwg_norm_gather, (_ptr(x), n_src, x.shape[-1], _ptr(table), table.numel(),
                                             float(eps), _ptr(out), _stream(dev))
    elif op == "window_inverse_build":
        (inv,) = tensors
        g, w, s = _triple(grid, "grid"), _triple(window, "window"), _triple(shift, "shift")
        _check_table_out(inv, _token_count(g), "inverse")
        dev = inv.device
        fn, args = lib.lwg_window_inverse_build, (*g, *w, *s, _ptr(inv), inv.numel(), _stream(dev))
    elif op == "window_reverse_add_ln":
        rows, inv, r, ro, y = tensors
        n_win, n = _check_reverse_add_ln(rows, inv, r, ro, y)
        dev = r.device
        fn, args = lib.lwg_window_reverse_add_ln, (_ptr(rows), n_win, _ptr(inv), _ptr(r), _ptr(ro), _ptr(y), n,
                                                   r.shape[-1], float(eps), _stream(dev))
    elif op == "add_norm_gather":
        b, r, ro, table, out = tensors
        n_src = _check_add_norm_gather(b, r, ro, table, out)
        dev = r.device
        fn, args = lib.lwg_add_norm_gather, (_ptr(b), _ptr(r), _ptr(ro), n_src, r.shape[-1], _ptr(table),
                                             table.numel(), float(eps), _ptr(out), _stream(dev))
    elif op == "ln_affine":
        x, g, b, y = tensors
        rows = _check_ln_affine(x, g, b, y)
        dev = x.device
        fn, args = lib.lwg_ln_affine, (_ptr(x), _ptr(g), _ptr(b), _ptr(y), rows, x.shape[-1], float(eps),
                                       _stream(dev))
    elif op == "add_ln_affine":
        br, r, g, b, ro, y = tensors
        rows = _check_add_ln_affine(br, r, g, b, ro, y)
        dev = r.device
        fn, args = lib.lwg_add_ln_affine, (_ptr(br), _ptr(r), _ptr(g), _ptr(b), _ptr(ro), _ptr(y), rows,
                                           r.shape[-1], float(eps), _stream(dev))
    elif op == "bias_gelu":
        x, b, y = tensors
        rows, cols = _check_bias_gelu(x, b, y)
        dev = x.device
        fn, args = lib.lwg_bias_gelu, (_ptr(x), _ptr(b), _ptr(y), rows, cols, _stream(dev))
    else:
        raise ValueError(f"unknown op {op!r}")
    return Prepared(fn, args, tensors)


__all__ += ["Prepared", "prepare"]

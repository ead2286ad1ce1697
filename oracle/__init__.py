"""CPU oracle for the fixed-width LayerNorm / shifted-window gather row pipeline.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and two legs
of ``bench.py`` (the sampled parity gate that runs before any timing, and the
``cpu_baseline`` timing) import this package. The product path (the HIP
library under ``include/lwg.h`` and its Python binding) never imports, calls
or links anything here, and this package imports nothing from it.

Everything is plain numpy in float64, written from the definitions on the page
"Pangu-Weather inference optimisation on Hygon BW1000 (gfx936)"
(l189.com/news/2144533):

* ``residual_sum`` -- section 4 (fused residual add + norm: the residual is
  rounded to FP16 once, before the normalisation reads it);
* ``layer_norm`` -- section 3 (fixed-width LayerNorm, no affine, widths 192/384,
  plus the patch-merge width 768);
* ``layer_norm_affine`` / ``add_ln_affine`` -- the same with a per-channel scale
  and shift, for callers that do not fold them into the next Linear;
* ``window_token_count`` / ``window_index_table`` -- section 5 (INT32 index
  table per window shape, padding folded into the index protocol);
* ``window_gather`` -- section 5 (index >= 0 copies the source token, -1 writes
  a zero row);
* ``norm_gather`` -- section 5 (norm1's output feeds only the window gather);
* ``window_reverse`` / ``window_inverse_table`` -- the inverse of the window
  partition (windows back to the grid, roll back, crop), which the pages imply
  but do not describe;
* ``window_reverse_add_ln`` / ``add_norm_gather`` -- the residual add + norm of
  section 4 fused with the reverse, or with the forward gather of section 5;
* ``bias_gelu`` -- the float32 bias + tanh-GELU of the page "PyTorch + HIP custom
  fused operator" (Hygon DCU practice series), sections 3-6.

Each function is pinned by ``tests/test_oracle_pins.py`` to closed forms,
brute force on tiny inputs, a library routine, or values derived by hand and
stored under ``tests/golden/``.
"""
from .rowops import (EPS, WIDTHS, fp16_round, residual_sum, layer_norm, add_ln, layer_norm_affine,
                     add_ln_affine)
from .activation import bias_gelu
from .window import (padded_extent, window_token_count, window_index_table,
                     window_gather, norm_gather, norm_gather_rows, window_reverse,
                     window_inverse_table, window_reverse_add_ln, add_norm_gather)

__all__ = [
    "EPS", "WIDTHS", "fp16_round", "residual_sum", "layer_norm", "add_ln", "layer_norm_affine",
    "add_ln_affine",
    "padded_extent", "window_token_count", "window_index_table", "window_gather",
    "norm_gather", "norm_gather_rows", "window_reverse", "window_inverse_table",
    "window_reverse_add_ln", "add_norm_gather", "bias_gelu",
]

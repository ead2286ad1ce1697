"""Planted mistakes in a copy of the oracle must fail the pins (CPU).

Each case edits one line of a temporary copy of ``oracle/`` -- the kind of
slip a reader could make when writing the definitions from the pages -- and
runs ``tests/test_oracle_pins.py`` against that copy. The pins must fail for
every real mistake. One edit is kept on purpose as an equivalent change: adding
the two binary16 residual operands in binary32 before the binary16 rounding.
It must *pass*, because when such a sum is inexact in binary32 the smaller
operand is below an eighth of a binary16 ulp of the larger, so both routes
round to the same binary16 value (the reading of the FP16 residual in the
design notes). A second equivalent edit normalises after the gather instead of
before: a padding row is all +0.0, and the LayerNorm of a zero row is
0 / sqrt(0 + eps) = +0.0, so the two orders agree.
"""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

# name -> (file, original text, planted text)
MISTAKES = {
    "padding rounds down": ("oracle/window.py", "return -(-extent // window) * window",
                            "return (extent // window) * window"),
    "a whole window of padding on exact extents": ("oracle/window.py", "return -(-extent // window) * window",
                                                   "return (extent // window + 1) * window"),
    "inverse numbers the gathered rows backwards": ("oracle/window.py",
                                                    "ids = np.arange(m, dtype=np.int64)[:, None]",
                                                    "ids = np.arange(m, dtype=np.int64)[::-1, None]"),
    "unbiased variance": ("oracle/rowops.py", "var = (dev * dev).mean(axis=1, keepdims=True)",
                          "var = (dev * dev).sum(axis=1, keepdims=True) / (v.shape[1] - 1)"),
    "eps outside the root": ("oracle/rowops.py", "y = dev / np.sqrt(var + eps)", "y = dev / (np.sqrt(var) + eps)"),
    "no eps": ("oracle/rowops.py", "y = dev / np.sqrt(var + eps)", "y = dev / np.sqrt(var)"),
    "roll sign": ("oracle/window.py", "shift=tuple(-s for s in shift)", "shift=tuple(s for s in shift)"),
    "window order": ("oracle/window.py", "windows.transpose(0, 2, 4, 1, 3, 5)", "windows.transpose(4, 2, 0, 5, 3, 1)"),
    "padding at the low end": ("oracle/window.py", "pad = [(0, padded_extent(g, w) - g)",
                               "pad = [(padded_extent(g, w) - g, 0)"),
    "out-of-range entries clamped": ("oracle/window.py", "valid = (table >= 0) & (table < x.shape[0])",
                                     "valid = (table >= 0)\n    table = np.minimum(table, x.shape[0] - 1)"),
    "affine: beta subtracted": ("oracle/rowops.py", "y = dev / np.sqrt(var + eps) * g + b",
                                "y = dev / np.sqrt(var + eps) * g - b"),
    "affine: gamma ignored": ("oracle/rowops.py", "y = dev / np.sqrt(var + eps) * g + b",
                              "y = dev / np.sqrt(var + eps) + b"),
    "affine: no eps": ("oracle/rowops.py", "y = dev / np.sqrt(var + eps) * g + b", "y = dev / np.sqrt(var) * g + b"),
    "gelu: cubic coefficient": ("oracle/activation.py", "GELU_K1 * t ** 3", "0.04 * t ** 3"),
    "gelu: half dropped": ("oracle/activation.py", "y = 0.5 * t * (1.0 + np.tanh(", "y = t * (1.0 + np.tanh("),
    "gelu: bias added in float64": ("oracle/activation.py", "t = (a + b[None, :]).astype(np.float64)",
                                    "t = a.astype(np.float64) + b[None, :].astype(np.float64)"),
    "reverse: roll sign": ("oracle/window.py", "g = np.roll(g, shift=tuple(shift), axis=(0, 1, 2))",
                           "g = np.roll(g, shift=tuple(-s for s in shift), axis=(0, 1, 2))"),
    "reverse: axes swapped": ("oracle/window.py", "g = g.transpose(0, 3, 1, 4, 2, 5, 6)",
                              "g = g.transpose(0, 3, 2, 4, 1, 5, 6)"),
    "add_norm_gather normalises the old residual": ("oracle/window.py", "    return r, norm_gather(r, table, eps)",
                                                    "    return r, norm_gather(residual, table, eps)"),
    "binary16 rounding through binary32": ("oracle/rowops.py",
                                           "return np.asarray(values, dtype=np.float64).astype(np.float16)",
                                           "return np.asarray(values, dtype=np.float64).astype(np.float32)"
                                           ".astype(np.float16)"),
    "mean over the wrong axis": ("oracle/rowops.py", "mean = v.mean(axis=1, keepdims=True)",
                                 "mean = v.mean(axis=0, keepdims=True)"),
    "deviations not centred": ("oracle/rowops.py", "dev = v - mean", "dev = v"),
    "padding as token 0": ("oracle/window.py", "constant_values=-1", "constant_values=0"),
    "shift before padding": ("oracle/window.py",
                             "    padded = np.pad(ids, pad, mode=\"constant\", constant_values=-1)\n"
                             "    rolled = np.roll(padded, shift=tuple(-s for s in shift), axis=(0, 1, 2))",
                             "    ids = np.roll(ids, shift=tuple(-s for s in shift), axis=(0, 1, 2))\n"
                             "    padded = np.pad(ids, pad, mode=\"constant\", constant_values=-1)\n"
                             "    rolled = padded"),
    "tokens with w slowest": ("oracle/window.py", "ids = np.arange(Z * H * W, dtype=np.int64).reshape(Z, H, W)",
                              "ids = np.arange(Z * H * W, dtype=np.int64).reshape(W, H, Z).transpose(2, 1, 0)"),
    "reverse: crop at the low end": ("oracle/window.py", "g[:Z, :H, :W]", "g[Zp - Z:, Hp - H:, Wp - W:]"),
    "gelu: sqrt(2/pi) dropped": ("oracle/activation.py", "np.tanh(GELU_K0 * (t + GELU_K1 * t ** 3))",
                                 "np.tanh(t + GELU_K1 * t ** 3)"),
}
EQUIVALENT = {
    "residual added in binary32": ("oracle/rowops.py", "return fp16_round(r + b)",
                                   "return fp16_round(np.float32(r) + np.float32(b))"),
    "norm_gather normalises after the gather": ("oracle/window.py",
                                                "return window_gather(layer_norm(x, eps), table)",
                                                "return layer_norm(window_gather(x, table), eps)"),
}


def run_pins_with(tmp_path, edit):
    """Copy the oracle and its pins into tmp_path, apply one edit, run the pins."""
    for sub in ("oracle", os.path.join("tests", "golden")):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub)
    for f in ("workloads.py", os.path.join("tests", "conftest.py"), os.path.join("tests", "test_oracle_pins.py")):
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    path, old, new = edit
    target = tmp_path / path
    text = target.read_text()
    assert old in text, f"the line to edit is gone from {path}: {old!r}"
    target.write_text(text.replace(old, new))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           os.path.join("tests", "test_oracle_pins.py")],
                          cwd=tmp_path, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_fails_the_pins(tmp_path, name):
    res = run_pins_with(tmp_path, MISTAKES[name])
    assert res.returncode != 0, f"pins did not catch: {name}\n{res.stdout[-500:]}"


@pytest.mark.parametrize("name", sorted(EQUIVALENT))
def test_equivalent_edit_passes_the_pins(tmp_path, name):
    res = run_pins_with(tmp_path, EQUIVALENT[name])
    assert res.returncode == 0, f"an equivalent edit failed the pins: {name}\n{res.stdout[-1500:]}"

"""Planted mistakes in a copy of the oracle must fail the pins (CPU).

Each case edits one line of a temporary copy of ``oracle/`` -- the kind of
slip a reader could make when writing the definitions from the pages -- and
runs ``tests/test_oracle_pins.py`` against that copy. The pins must fail for
every real mistake. One edit is kept on purpose as an equivalent change: adding
the two binary16 residual operands in binary32 before the binary16 rounding.
It must *pass*, because when such a sum is inexact in binary32 the smaller
operand is below an eighth of a binary16 ulp of the larger, so both routes
round to the same binary16 value (the reading of the FP16 residual in the
design notes).
"""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

# name -> (file, original text, planted text)
MISTAKES = {
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
}
EQUIVALENT = {
    "residual added in binary32": ("oracle/rowops.py", "return fp16_round(r + b)",
                                   "return fp16_round(np.float32(r) + np.float32(b))"),
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

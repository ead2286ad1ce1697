"""The bench's command-line contract on the CPU: more than one GPU is refused
with a message (only the one-GPU shard is built), and the algorithmic byte
counts it reports per op are the formulas of the row pipeline."""
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from workloads import LEVEL1, LEVEL2  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 4" in res.stderr


def test_algorithmic_bytes_of_the_step():
    n1, n2, c1, c2 = LEVEL1.tokens, LEVEL2.tokens, LEVEL1.channels, LEVEL2.channels
    m1, m2 = 142848, 36864
    assert bench.algorithmic_bytes("add_ln", n1, m1, c1) == 201_277_440
    assert bench.algorithmic_bytes("ln_fixed", n2, m2, c2) == 50_319_360
    assert bench.algorithmic_bytes("norm_gather", n1, m1, c1) == 105_744_384
    assert bench.algorithmic_bytes("window_gather", n2, m2, c2) == 53_618_688
    assert bench.algorithmic_bytes("window_index_build", n1, m1, c1) == 4 * m1
    step = sum(bench.algorithmic_bytes(op, lv.tokens, m, lv.channels)
               for lv, m in ((LEVEL1, m1), (LEVEL2, m2)) for op in bench.OPS)
    assert step == 201_277_440 + 100_638_720 + 105_744_384 * 2 + 4 * m1 + \
        100_638_720 + 50_319_360 + 53_618_688 * 2 + 4 * m2

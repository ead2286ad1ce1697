"""Build the plain C client of liblwg (tests/c_client/lwg_c_client.c) with gcc.

It is compiled as C99 against include/lwg.h and the HIP runtime's C API, linked
to the in-tree liblwg.so and libamdhip64, and found at run time through an rpath
relative to the binary. Run after the library is built.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "lwg_c_client.c")
BINARY = os.path.join(HERE, "lwg_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BINARY) -> list:
    return [
        shutil.which("gcc") or "gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
        SOURCE, "-o", out,
        "-L", os.path.join(ROOT, "layernorm_window_gather_amd"), "-llwg",
        "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
        "-Wl,-rpath,$ORIGIN/../../layernorm_window_gather_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
    ]


def build(verbose: bool = False) -> str:
    cmd = command(BINARY + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed with status {res.returncode}:\n{res.stdout}{res.stderr}")
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    print(build(verbose=True))

"""The C ABI on the host: the library loads, exports every function that
include/lwg.h declares, and refuses bad arguments before any HIP call.

No test here launches a kernel: every call below fails validation (or is a
host-only function), so these run without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

lwg = pytest.importorskip("layernorm_window_gather_amd")
from layernorm_window_gather_amd import _lib  # noqa: E402

HEADER = os.path.join(ROOT, "include", "lwg.h")
P = ctypes.c_void_p
A16 = P(0x10000)          # 16-byte aligned stand-ins; never dereferenced
B16 = P(0x20000)
MIS = P(0x10008)          # 8-byte aligned only
ST = P(0)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lwg_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_list_the_same_functions():
    assert header_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.lwg_abi_version() == 1


def test_status_strings(lib):
    names = [lib.lwg_status_string(i).decode() for i in range(7)]
    assert names == ["LWG_OK", "LWG_ERR_INVALID_ARGUMENT", "LWG_ERR_UNSUPPORTED_WIDTH",
                     "LWG_ERR_MISALIGNED", "LWG_ERR_ALIASING", "LWG_ERR_SIZE_MISMATCH", "LWG_ERR_HIP"]
    assert lib.lwg_status_string(99).decode() == "LWG_ERR_UNKNOWN"


def test_window_token_count_host(lib):
    assert lib.lwg_window_token_count(8, 182, 90, 2, 6, 12) == 142848
    assert lib.lwg_window_token_count(8, 91, 45, 2, 6, 12) == 36864
    assert lib.lwg_window_token_count(2, 12, 24, 2, 6, 12) == 576
    assert lib.lwg_window_token_count(0, 5, 5, 2, 6, 12) == 0
    assert lib.lwg_window_token_count(1, 1, 1, 0, 1, 1) == -1
    assert lib.lwg_window_token_count(-1, 1, 1, 1, 1, 1) == -1
    assert lib.lwg_window_token_count(2**20, 2**20, 2, 1, 1, 1) == -1   # above INT32_MAX


def test_window_token_count_matches_oracle(lib):
    import oracle
    rng = np.random.default_rng(5)
    for _ in range(200):
        g = tuple(int(v) for v in rng.integers(1, 40, 3))
        w = tuple(int(v) for v in rng.integers(1, 13, 3))
        assert lib.lwg_window_token_count(*g, *w) == oracle.window_token_count(g, w)


def _err(lib, status):
    return status, lib.lwg_last_error().decode()


def test_ln_fixed_validation(lib):
    S = _lib
    assert _err(lib, lib.lwg_ln_fixed(A16, B16, 10, 256, 1e-5, ST))[0] == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert _err(lib, lib.lwg_ln_fixed(A16, B16, 10, 192, 0.0, ST))[0] == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(A16, B16, 10, 192, float("nan"), ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(A16, B16, 10, 192, float("inf"), ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(A16, B16, -1, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(A16, B16, 2**31, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(None, B16, 10, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(A16, None, 10, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_ln_fixed(MIS, B16, 10, 192, 1e-5, ST) == S.LWG_ERR_MISALIGNED
    assert lib.lwg_ln_fixed(A16, MIS, 10, 192, 1e-5, ST) == S.LWG_ERR_MISALIGNED
    # partial overlap: y starts one row into x
    st, msg = _err(lib, lib.lwg_ln_fixed(A16, P(0x10000 + 384), 10, 192, 1e-5, ST))
    assert st == S.LWG_ERR_ALIASING and "overlap" in msg
    # empty input: OK with no launch, pointers not inspected
    assert lib.lwg_ln_fixed(None, None, 0, 192, 1e-5, ST) == S.LWG_OK
    assert lib.lwg_last_error().decode() == ""


def test_add_ln_validation(lib):
    S = _lib
    f = lib.lwg_add_ln
    C3, C4 = P(0x30000), P(0x40000)
    assert f(A16, B16, C3, C4, 10, 128, 1e-5, ST) == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert f(A16, B16, C3, C4, 10, 384, -1.0, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(A16, None, C3, C4, 10, 384, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(A16, B16, C3, MIS, 10, 384, 1e-5, ST) == S.LWG_ERR_MISALIGNED
    # y and residual_out may not be the same buffer
    assert f(A16, B16, C3, C3, 10, 384, 1e-5, ST) == S.LWG_ERR_ALIASING
    # partial overlap of an output with an input
    assert f(A16, B16, P(0x20000 + 768), C4, 10, 384, 1e-5, ST) == S.LWG_ERR_ALIASING
    assert f(A16, B16, C3, P(0x10000 + 16), 10, 384, 1e-5, ST) == S.LWG_ERR_ALIASING
    assert f(None, None, None, None, 0, 384, 1e-5, ST) == S.LWG_OK


def test_index_build_validation(lib):
    S = _lib
    f = lib.lwg_window_index_build
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, A16, 142847, ST) == S.LWG_ERR_SIZE_MISMATCH
    assert f(8, 182, 90, 0, 6, 12, 1, 3, 6, A16, 142848, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, -1, 3, 6, A16, 142848, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(-8, 182, 90, 2, 6, 12, 1, 3, 6, A16, 142848, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, None, 142848, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, P(0x10002), 142848, ST) == S.LWG_ERR_MISALIGNED
    assert f(0, 182, 90, 2, 6, 12, 1, 3, 6, None, 0, ST) == S.LWG_OK


def test_gather_validation(lib):
    S = _lib
    for name, extra in (("lwg_window_gather", ()), ("lwg_norm_gather", (1e-5,))):
        f = getattr(lib, name)

        def call(x, n_src, C, table, n_out, out):
            return f(x, n_src, C, table, n_out, *extra, out, ST)

        T = P(0x80000)
        assert call(A16, 100, 200, T, 50, B16) == S.LWG_ERR_UNSUPPORTED_WIDTH
        assert call(A16, -1, 192, T, 50, B16) == S.LWG_ERR_INVALID_ARGUMENT
        assert call(A16, 100, 192, T, 2**31, B16) == S.LWG_ERR_INVALID_ARGUMENT
        assert call(A16, 100, 192, None, 50, B16) == S.LWG_ERR_INVALID_ARGUMENT
        assert call(None, 100, 192, T, 50, B16) == S.LWG_ERR_INVALID_ARGUMENT
        assert call(A16, 100, 192, P(0x80002), 50, B16) == S.LWG_ERR_MISALIGNED
        assert call(A16, 100, 192, T, 50, MIS) == S.LWG_ERR_MISALIGNED
        # out overlapping x or the table
        assert call(A16, 100, 192, T, 50, P(0x10000 + 384 * 10)) == S.LWG_ERR_ALIASING
        assert call(A16, 100, 192, T, 50, P(0x80000 - 16)) == S.LWG_ERR_ALIASING
        assert call(None, 0, 192, None, 0, None) == S.LWG_OK
    assert lib.lwg_norm_gather(A16, 100, 192, P(0x80000), 50, 0.0, B16, ST) == S.LWG_ERR_INVALID_ARGUMENT


def test_python_binding_refuses_cpu_and_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 192, dtype=torch.float16)
    with pytest.raises(RuntimeError, match="GPU"):
        lwg.ln_fixed(x)
    with pytest.raises(RuntimeError, match="GPU"):
        lwg.add_ln(x, x)
    with pytest.raises(RuntimeError, match="GPU"):
        lwg.window_gather(x, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(RuntimeError, match="float16"):
        lwg.ln_fixed(torch.zeros(4, 192))
    with pytest.raises(RuntimeError, match="192, 384 or 768"):
        lwg.ln_fixed(torch.zeros(4, 256, dtype=torch.float16))
    with pytest.raises(RuntimeError, match="contiguous"):
        lwg.ln_fixed(torch.zeros(192, 8, dtype=torch.float16).t())
    with pytest.raises(RuntimeError):
        lwg.window_index_build((8, 182, 90), (2, 6, 12), (1, 3, 6), device="cpu")


def test_python_window_token_count():
    assert lwg.window_token_count((8, 182, 90), (2, 6, 12)) == 142848
    with pytest.raises(RuntimeError):
        lwg.window_token_count((8, 182, 90), (0, 6, 12))


def test_error_carries_status_and_message():
    with pytest.raises(lwg.LwgError) as e:
        _lib.check(_lib.load().lwg_ln_fixed(A16, B16, 10, 100, 1e-5, ST))
    assert e.value.status == _lib.LWG_ERR_UNSUPPORTED_WIDTH
    assert "C=100" in str(e.value)


def test_inverse_build_validation(lib):
    S = _lib
    f = lib.lwg_window_inverse_build
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, A16, 131039, ST) == S.LWG_ERR_SIZE_MISMATCH
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, A16, 142848, ST) == S.LWG_ERR_SIZE_MISMATCH
    assert f(8, 182, 90, 2, 0, 12, 1, 3, 6, A16, 131040, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, 1, -3, 6, A16, 131040, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, None, 131040, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(8, 182, 90, 2, 6, 12, 1, 3, 6, P(0x10001), 131040, ST) == S.LWG_ERR_MISALIGNED
    assert f(0, 182, 90, 2, 6, 12, 1, 3, 6, None, 0, ST) == S.LWG_OK


def test_reverse_add_ln_validation(lib):
    S = _lib
    f = lib.lwg_window_reverse_add_ln
    W, I, R, RO, Y = P(0x100000), P(0x200000), P(0x300000), P(0x400000), P(0x500000)
    assert f(W, 200, I, R, RO, Y, 100, 128, 1e-5, ST) == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert f(W, 200, I, R, RO, Y, 100, 192, 0.0, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(W, -1, I, R, RO, Y, 100, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(W, 200, None, R, RO, Y, 100, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(W, 200, P(0x200002), R, RO, Y, 100, 192, 1e-5, ST) == S.LWG_ERR_MISALIGNED
    assert f(None, 200, I, R, RO, Y, 100, 192, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(W, 200, I, R, RO, RO, 100, 192, 1e-5, ST) == S.LWG_ERR_ALIASING        # y == residual_out
    assert f(W, 200, I, R, P(0x300000 + 384), Y, 100, 192, 1e-5, ST) == S.LWG_ERR_ALIASING
    assert f(W, 200, I, R, P(0x100000 + 384), Y, 100, 192, 1e-5, ST) == S.LWG_ERR_ALIASING  # into win
    assert f(W, 200, I, R, RO, P(0x200000 - 16), 100, 192, 1e-5, ST) == S.LWG_ERR_ALIASING  # onto inverse
    assert f(None, 0, None, None, None, None, 0, 192, 1e-5, ST) == S.LWG_OK


def test_add_norm_gather_validation(lib):
    S = _lib
    f = lib.lwg_add_norm_gather
    B, R, RO, T, O = P(0x100000), P(0x200000), P(0x300000), P(0x400000), P(0x500000)
    assert f(B, R, RO, 100, 200, T, 150, 1e-5, O, ST) == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert f(B, R, RO, 100, 192, T, 150, float("nan"), O, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(B, R, RO, -5, 192, T, 150, 1e-5, O, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(B, R, RO, 100, 192, None, 150, 1e-5, O, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(B, None, RO, 100, 192, T, 150, 1e-5, O, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(B, R, RO, 100, 192, T, 150, 1e-5, MIS, ST) == S.LWG_ERR_MISALIGNED
    assert f(B, R, RO, 100, 192, T, 150, 1e-5, P(0x100000 + 384), ST) == S.LWG_ERR_ALIASING   # out on branch
    assert f(B, R, RO, 100, 192, T, 150, 1e-5, P(0x400000 - 16), ST) == S.LWG_ERR_ALIASING    # out on table
    assert f(B, R, P(0x200000 + 768), 100, 192, T, 150, 1e-5, O, ST) == S.LWG_ERR_ALIASING    # partial
    assert f(None, None, None, 0, 192, None, 0, 1e-5, None, ST) == S.LWG_OK


def test_affine_validation(lib):
    S = _lib
    X, G, B, Y = P(0x100000), P(0x200000), P(0x210000), P(0x300000)
    f = lib.lwg_ln_affine
    assert f(X, G, B, Y, 10, 256, 1e-5, ST) == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert f(X, None, B, Y, 10, 768, 1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(X, G, P(0x210008), Y, 10, 768, 1e-5, ST) == S.LWG_ERR_MISALIGNED
    assert f(X, G, B, P(0x200000 - 16), 10, 192, 1e-5, ST) == S.LWG_ERR_ALIASING      # y over gamma
    assert f(X, G, B, P(0x100000 + 384), 10, 192, 1e-5, ST) == S.LWG_ERR_ALIASING     # y partly on x
    assert f(None, None, None, None, 0, 384, 1e-5, ST) == S.LWG_OK
    g = lib.lwg_add_ln_affine
    R, RO = P(0x400000), P(0x500000)
    assert g(X, R, G, B, RO, Y, 10, 100, 1e-5, ST) == S.LWG_ERR_UNSUPPORTED_WIDTH
    assert g(X, R, G, B, RO, RO, 10, 192, 1e-5, ST) == S.LWG_ERR_ALIASING
    assert g(X, R, G, B, P(0x210000 - 32), Y, 10, 192, 1e-5, ST) == S.LWG_ERR_ALIASING  # residual_out over beta region
    assert g(X, R, G, B, RO, Y, 10, 192, -1e-5, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert g(None, None, None, None, None, None, 0, 768, 1e-5, ST) == S.LWG_OK


def test_width_768_accepted_by_every_row_call(lib):
    # a 768-wide call that fails later validation proves the width itself passed
    assert lib.lwg_ln_fixed(None, B16, 10, 768, 1e-5, ST) == _lib.LWG_ERR_INVALID_ARGUMENT
    assert lib.lwg_window_gather(A16, 10, 768, None, 5, B16, ST) == _lib.LWG_ERR_INVALID_ARGUMENT


def test_bias_gelu_validation(lib):
    S = _lib
    f = lib.lwg_bias_gelu
    X, Bi, Y = P(0x100000), P(0x200000), P(0x300000)
    assert f(X, Bi, Y, 10, 6, ST) == S.LWG_ERR_INVALID_ARGUMENT        # cols not a multiple of 4
    assert f(X, Bi, Y, 10, 0, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(X, Bi, Y, -1, 8, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(X, Bi, Y, 2**30, 16, ST) == S.LWG_ERR_INVALID_ARGUMENT    # more than 2^31-1 float4 groups
    assert f(X, None, Y, 10, 8, ST) == S.LWG_ERR_INVALID_ARGUMENT
    assert f(X, P(0x200004), Y, 10, 8, ST) == S.LWG_ERR_MISALIGNED
    assert f(X, Bi, P(0x100000 + 32), 10, 8, ST) == S.LWG_ERR_ALIASING  # partial overlap with x
    assert f(X, Bi, P(0x200000 - 16), 10, 8, ST) == S.LWG_ERR_ALIASING  # y over the bias
    assert f(None, None, None, 0, 8, ST) == S.LWG_OK


def test_header_is_strict_c99(tmp_path):
    """include/lwg.h compiles as C99 with -pedantic -Werror (no C++ in the ABI)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use_header.c"
    src.write_text('#include "lwg.h"\nint main(void) { return lwg_abi_version() == LWG_ABI_VERSION ? 0 : 1; }\n')
    res = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                          "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_huge_grids_are_refused_without_overflow():
    """Grid products past 2^63 (a padded extent can reach 2^32 - 2) are refused,
    not wrapped: the token count is -1 and both table builders refuse."""
    lib = _lib.load()
    big = 2**31 - 1
    assert lib.lwg_window_token_count(big, big, big, 1, 1, 1) == -1
    assert lib.lwg_window_token_count(big, big, 1, big - 1, big - 1, 1) == -1
    assert lib.lwg_window_token_count(0, big, big, 1, 1, 1) == 0
    st = lib.lwg_window_index_build(big, big, big, 1, 1, 1, 0, 0, 0, ctypes.c_void_p(0x1000), 1, None)
    assert st == _lib.LWG_ERR_INVALID_ARGUMENT
    st = lib.lwg_window_inverse_build(big, big, big, 2, 6, 12, 0, 0, 0, ctypes.c_void_p(0x1000), 1, None)
    assert st == _lib.LWG_ERR_INVALID_ARGUMENT


def test_missing_library_fails_loudly(tmp_path):
    # With no liblwg.so there is no fallback: loading the library raises and
    # names the build command. Run in a fresh process so the already-loaded
    # library of this one is not reused.
    import subprocess
    import sys
    code = ("import layernorm_window_gather_amd as lwg\n"
            "try:\n"
            "    lwg.library()\n"
            "except RuntimeError as e:\n"
            "    print('RAISED', e)\n")
    env = dict(os.environ, LWG_LIBRARY=str(tmp_path / "absent" / "liblwg.so"))
    run = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert run.returncode == 0, run.stderr
    assert "RAISED" in run.stdout and "no fallback" in run.stdout, run.stdout + run.stderr

// extern "C" entry points declared in include/lwg.h: host-side argument checks,
// then one launch on the caller's stream. Nothing here allocates, frees or
// synchronises. The checks follow the contract style of the page "PyTorch + HIP
// custom fused operator" (Hygon DCU practice series), section 6: refuse bad
// input before launching, return early on empty input, use the caller's
// stream, and turn a launch error into an error result.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include <hip/hip_runtime.h>

#include "lwg.h"
#include "lwg_launch.h"

#define LWG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int32_t fail(lwg_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

int32_t ok() {
    g_last_error.clear();
    return LWG_OK;
}

int32_t hip_result(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(LWG_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) share a byte.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// Same buffer (exact alias) or disjoint; a partial overlap is an error.
bool same_or_disjoint(const void* a, const void* b, uint64_t n) {
    return a == b || !overlap(a, n, b, n);
}

int32_t check_width(const char* fn, int32_t C) {
    if (C != 192 && C != 384 && C != 768)
        return fail(LWG_ERR_UNSUPPORTED_WIDTH, "%s: C=%d is not served (only 192, 384 and 768)", fn, C);
    return LWG_OK;
}

int32_t check_eps(const char* fn, double eps) {
    if (!(std::isfinite(eps) && eps > 0.0))
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: eps must be finite and > 0 (got %g)", fn, eps);
    return LWG_OK;
}

int32_t check_rows(const char* fn, const char* name, int64_t rows) {
    if (rows < 0 || rows > INT32_MAX)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: %s=%lld must be in [0, 2^31-1]", fn, name,
                    static_cast<long long>(rows));
    return LWG_OK;
}

int32_t check_tensor(const char* fn, const char* name, const void* p) {
    if (p == nullptr) return fail(LWG_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, name);
    if (!aligned16(p)) return fail(LWG_ERR_MISALIGNED, "%s: %s is not 16-byte aligned", fn, name);
    return LWG_OK;
}

// Padded extent of one axis, or -1 when the inputs are out of range.
int64_t padded(int64_t extent, int64_t window) {
    if (extent < 0 || window < 1) return -1;
    return (extent + window - 1) / window * window;
}

}  // namespace

LWG_EXPORT int32_t lwg_abi_version(void) { return LWG_ABI_VERSION; }

LWG_EXPORT const char* lwg_last_error(void) { return g_last_error.c_str(); }

LWG_EXPORT const char* lwg_status_string(int32_t status) {
    switch (status) {
        case LWG_OK: return "LWG_OK";
        case LWG_ERR_INVALID_ARGUMENT: return "LWG_ERR_INVALID_ARGUMENT";
        case LWG_ERR_UNSUPPORTED_WIDTH: return "LWG_ERR_UNSUPPORTED_WIDTH";
        case LWG_ERR_MISALIGNED: return "LWG_ERR_MISALIGNED";
        case LWG_ERR_ALIASING: return "LWG_ERR_ALIASING";
        case LWG_ERR_SIZE_MISMATCH: return "LWG_ERR_SIZE_MISMATCH";
        case LWG_ERR_HIP: return "LWG_ERR_HIP";
        default: return "LWG_ERR_UNKNOWN";
    }
}

LWG_EXPORT int32_t lwg_ln_fixed(const void* x, void* y, int64_t rows, int32_t C, double eps,
                                void* stream) {
    static const char* fn = "lwg_ln_fixed";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "rows", rows)))
        return st;
    if (rows == 0) return ok();
    if ((st = check_tensor(fn, "x", x)) || (st = check_tensor(fn, "y", y))) return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * C * 2;
    if (!same_or_disjoint(x, y, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y partially overlaps x (only y == x is allowed)", fn);
    return hip_result(lwg::launch_ln_fixed(x, y, rows, C, eps, static_cast<hipStream_t>(stream)), fn);
}

LWG_EXPORT int32_t lwg_add_ln(const void* branch, const void* residual, void* residual_out,
                              void* y, int64_t rows, int32_t C, double eps, void* stream) {
    static const char* fn = "lwg_add_ln";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "rows", rows)))
        return st;
    if (rows == 0) return ok();
    if ((st = check_tensor(fn, "branch", branch)) || (st = check_tensor(fn, "residual", residual)) ||
        (st = check_tensor(fn, "residual_out", residual_out)) || (st = check_tensor(fn, "y", y)))
        return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * C * 2;
    if (overlap(y, bytes, residual_out, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y and residual_out overlap", fn);
    if (!same_or_disjoint(residual_out, residual, bytes) || !same_or_disjoint(residual_out, branch, bytes) ||
        !same_or_disjoint(y, residual, bytes) || !same_or_disjoint(y, branch, bytes))
        return fail(LWG_ERR_ALIASING,
                    "%s: an output partially overlaps an input (only exact in-place aliasing is allowed)", fn);
    return hip_result(lwg::launch_add_ln(branch, residual, residual_out, y, rows, C, eps,
                                         static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int64_t lwg_window_token_count(int32_t Z, int32_t H, int32_t W, int32_t wz, int32_t wh,
                                          int32_t ww) {
    const int64_t zp = padded(Z, wz), hp = padded(H, wh), wp = padded(W, ww);
    if (zp < 0 || hp < 0 || wp < 0) return -1;
    if (zp == 0 || hp == 0 || wp == 0) return 0;
    // a padded extent can reach 2^32 - 2; bound every factor and partial product
    // by 2^31 - 1 before the next multiply, so no product leaves int64
    if (zp > INT32_MAX || hp > INT32_MAX || wp > INT32_MAX) return -1;
    const int64_t zh = zp * hp;
    if (zh > INT32_MAX) return -1;
    const int64_t n = zh * wp;
    return n > INT32_MAX ? -1 : n;
}

namespace {

// Checks the window geometry shared by both table builders and fills g; `len`
// must equal `expect` (the table length the geometry implies).
int32_t window_geometry(const char* fn, int32_t Z, int32_t H, int32_t W, int32_t wz, int32_t wh,
                        int32_t ww, int32_t sz, int32_t sh, int32_t sw, lwg::WindowGeometry& g,
                        int64_t* rows_out, int64_t* tokens_out) {
    if (Z < 0 || H < 0 || W < 0)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: grid extents must be >= 0 (got %d,%d,%d)", fn, Z, H, W);
    if (wz < 1 || wh < 1 || ww < 1)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: window extents must be >= 1 (got %d,%d,%d)", fn, wz, wh, ww);
    if (sz < 0 || sh < 0 || sw < 0)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: shifts must be >= 0 (got %d,%d,%d)", fn, sz, sh, sw);
    // Z*H < 2^62; bound it before multiplying by W so the product stays in int64
    const int64_t zh = static_cast<int64_t>(Z) * H;
    if (W != 0 && (zh > INT32_MAX || zh * W > INT32_MAX))
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: grid holds more than 2^31-1 tokens", fn);
    const int64_t tokens = zh * W;
    const int64_t m = lwg_window_token_count(Z, H, W, wz, wh, ww);
    if (m < 0)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: padded grid holds more than 2^31-1 rows", fn);
    *rows_out = m;
    *tokens_out = tokens;
    if (m == 0) return LWG_OK;
    g.Z = Z; g.H = H; g.W = W;
    g.wz = wz; g.wh = wh; g.ww = ww;
    g.Zp = static_cast<int32_t>(padded(Z, wz));
    g.Hp = static_cast<int32_t>(padded(H, wh));
    g.Wp = static_cast<int32_t>(padded(W, ww));
    g.sz = sz % g.Zp; g.sh = sh % g.Hp; g.sw = sw % g.Wp;
    g.nbh = g.Hp / wh; g.nbw = g.Wp / ww;
    g.win_tokens = wz * wh * ww;
    g.rows = static_cast<int32_t>(m);
    g.div_win = lwg::make_fastdiv(static_cast<uint32_t>(g.win_tokens));
    g.div_nbw = lwg::make_fastdiv(static_cast<uint32_t>(g.nbw));
    g.div_nbh = lwg::make_fastdiv(static_cast<uint32_t>(g.nbh));
    g.div_ww = lwg::make_fastdiv(static_cast<uint32_t>(ww));
    g.div_wh = lwg::make_fastdiv(static_cast<uint32_t>(wh));
    g.div_wz = lwg::make_fastdiv(static_cast<uint32_t>(wz));
    g.div_W = lwg::make_fastdiv(static_cast<uint32_t>(W > 0 ? W : 1));
    g.div_H = lwg::make_fastdiv(static_cast<uint32_t>(H > 0 ? H : 1));
    return LWG_OK;
}

int32_t check_table_ptr(const char* fn, const char* name, const int32_t* t) {
    if (t == nullptr) return fail(LWG_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, name);
    if ((reinterpret_cast<uintptr_t>(t) & 3u) != 0)
        return fail(LWG_ERR_MISALIGNED, "%s: %s is not 4-byte aligned", fn, name);
    return LWG_OK;
}

}  // namespace

LWG_EXPORT int32_t lwg_window_index_build(int32_t Z, int32_t H, int32_t W, int32_t wz, int32_t wh,
                                          int32_t ww, int32_t sz, int32_t sh, int32_t sw,
                                          int32_t* table, int64_t table_len, void* stream) {
    static const char* fn = "lwg_window_index_build";
    lwg::WindowGeometry g;
    int64_t m = 0, tokens = 0;
    int32_t st = window_geometry(fn, Z, H, W, wz, wh, ww, sz, sh, sw, g, &m, &tokens);
    if (st) return st;
    if (table_len != m)
        return fail(LWG_ERR_SIZE_MISMATCH, "%s: table_len=%lld but the window token count is %lld", fn,
                    static_cast<long long>(table_len), static_cast<long long>(m));
    if (m == 0) return ok();
    if ((st = check_table_ptr(fn, "table", table))) return st;
    return hip_result(lwg::launch_window_index(g, table, static_cast<hipStream_t>(stream)), fn);
}

LWG_EXPORT int32_t lwg_window_inverse_build(int32_t Z, int32_t H, int32_t W, int32_t wz, int32_t wh,
                                            int32_t ww, int32_t sz, int32_t sh, int32_t sw,
                                            int32_t* inverse, int64_t inverse_len, void* stream) {
    static const char* fn = "lwg_window_inverse_build";
    lwg::WindowGeometry g;
    int64_t m = 0, tokens = 0;
    int32_t st = window_geometry(fn, Z, H, W, wz, wh, ww, sz, sh, sw, g, &m, &tokens);
    if (st) return st;
    if (inverse_len != tokens)
        return fail(LWG_ERR_SIZE_MISMATCH, "%s: inverse_len=%lld but the grid holds %lld tokens", fn,
                    static_cast<long long>(inverse_len), static_cast<long long>(tokens));
    if (tokens == 0) return ok();
    if ((st = check_table_ptr(fn, "inverse", inverse))) return st;
    return hip_result(lwg::launch_window_inverse(g, inverse, static_cast<hipStream_t>(stream)), fn);
}

namespace {

int32_t check_gather(const char* fn, const void* x, int64_t n_src, int32_t C, const int32_t* table,
                     int64_t n_out, const void* out) {
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_rows(fn, "n_src", n_src)) ||
        (st = check_rows(fn, "n_out", n_out)))
        return st;
    if (n_out == 0) return LWG_OK;
    if (n_src > 0 && (st = check_tensor(fn, "x", x))) return st;
    if ((st = check_tensor(fn, "out", out))) return st;
    if (table == nullptr) return fail(LWG_ERR_INVALID_ARGUMENT, "%s: table is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(table) & 3u) != 0)
        return fail(LWG_ERR_MISALIGNED, "%s: table is not 4-byte aligned", fn);
    const uint64_t out_bytes = static_cast<uint64_t>(n_out) * C * 2;
    if (n_src > 0 && overlap(out, out_bytes, x, static_cast<uint64_t>(n_src) * C * 2))
        return fail(LWG_ERR_ALIASING, "%s: out overlaps x", fn);
    if (overlap(out, out_bytes, table, static_cast<uint64_t>(n_out) * 4))
        return fail(LWG_ERR_ALIASING, "%s: out overlaps table", fn);
    return LWG_OK;
}

}  // namespace

LWG_EXPORT int32_t lwg_window_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                                     int64_t n_out, void* out, void* stream) {
    static const char* fn = "lwg_window_gather";
    int32_t st = check_gather(fn, x, n_src, C, table, n_out, out);
    if (st) return st;
    if (n_out == 0) return ok();
    return hip_result(lwg::launch_window_gather(x, n_src, C, table, n_out, out,
                                                static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int32_t lwg_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                                   int64_t n_out, double eps, void* out, void* stream) {
    static const char* fn = "lwg_norm_gather";
    int32_t st = check_eps(fn, eps);
    if (st) return st;
    if ((st = check_gather(fn, x, n_src, C, table, n_out, out))) return st;
    if (n_out == 0) return ok();
    return hip_result(lwg::launch_norm_gather(x, n_src, C, table, n_out, eps, out,
                                              static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int32_t lwg_window_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse,
                                             const void* residual, void* residual_out, void* y,
                                             int64_t rows, int32_t C, double eps, void* stream) {
    static const char* fn = "lwg_window_reverse_add_ln";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "rows", rows)) ||
        (st = check_rows(fn, "n_win", n_win)))
        return st;
    if (rows == 0) return ok();
    if ((n_win > 0 && (st = check_tensor(fn, "win", win))) || (st = check_table_ptr(fn, "inverse", inverse)) ||
        (st = check_tensor(fn, "residual", residual)) || (st = check_tensor(fn, "residual_out", residual_out)) ||
        (st = check_tensor(fn, "y", y)))
        return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * C * 2;
    const uint64_t win_bytes = static_cast<uint64_t>(n_win) * C * 2;
    if (overlap(y, bytes, residual_out, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y and residual_out overlap", fn);
    if (!same_or_disjoint(residual_out, residual, bytes) || !same_or_disjoint(y, residual, bytes))
        return fail(LWG_ERR_ALIASING, "%s: an output partially overlaps residual", fn);
    if ((n_win > 0 && (overlap(residual_out, bytes, win, win_bytes) || overlap(y, bytes, win, win_bytes))) ||
        overlap(residual_out, bytes, inverse, static_cast<uint64_t>(rows) * 4) ||
        overlap(y, bytes, inverse, static_cast<uint64_t>(rows) * 4))
        return fail(LWG_ERR_ALIASING, "%s: an output overlaps win or inverse", fn);
    return hip_result(lwg::launch_reverse_add_ln(win, n_win, inverse, residual, residual_out, y, rows, C, eps,
                                                 static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int32_t lwg_add_norm_gather(const void* branch, const void* residual, void* residual_out,
                                       int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                                       double eps, void* out, void* stream) {
    static const char* fn = "lwg_add_norm_gather";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "n_src", n_src)) ||
        (st = check_rows(fn, "n_out", n_out)))
        return st;
    if (n_out == 0) return ok();
    if ((st = check_table_ptr(fn, "table", table)) || (st = check_tensor(fn, "out", out))) return st;
    if (n_src > 0 && ((st = check_tensor(fn, "branch", branch)) || (st = check_tensor(fn, "residual", residual)) ||
                      (st = check_tensor(fn, "residual_out", residual_out))))
        return st;
    const uint64_t src_bytes = static_cast<uint64_t>(n_src) * C * 2;
    const uint64_t out_bytes = static_cast<uint64_t>(n_out) * C * 2;
    const uint64_t table_bytes = static_cast<uint64_t>(n_out) * 4;
    if (overlap(out, out_bytes, table, table_bytes))
        return fail(LWG_ERR_ALIASING, "%s: out overlaps table", fn);
    if (n_src > 0) {
        if (overlap(out, out_bytes, branch, src_bytes) || overlap(out, out_bytes, residual, src_bytes) ||
            overlap(out, out_bytes, residual_out, src_bytes))
            return fail(LWG_ERR_ALIASING, "%s: out overlaps a token tensor", fn);
        if (!same_or_disjoint(residual_out, residual, src_bytes) ||
            !same_or_disjoint(residual_out, branch, src_bytes) ||
            overlap(residual_out, src_bytes, table, table_bytes))
            return fail(LWG_ERR_ALIASING, "%s: residual_out partially overlaps an input", fn);
    }
    return hip_result(lwg::launch_add_norm_gather(branch, residual, residual_out, n_src, C, table, n_out, eps,
                                                  out, static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int32_t lwg_ln_affine(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                                 int32_t C, double eps, void* stream) {
    static const char* fn = "lwg_ln_affine";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "rows", rows)))
        return st;
    if (rows == 0) return ok();
    if ((st = check_tensor(fn, "x", x)) || (st = check_tensor(fn, "gamma", gamma)) ||
        (st = check_tensor(fn, "beta", beta)) || (st = check_tensor(fn, "y", y)))
        return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * C * 2;
    if (!same_or_disjoint(x, y, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y partially overlaps x (only y == x is allowed)", fn);
    if (overlap(y, bytes, gamma, static_cast<uint64_t>(C) * 2) || overlap(y, bytes, beta, static_cast<uint64_t>(C) * 2))
        return fail(LWG_ERR_ALIASING, "%s: y overlaps gamma or beta", fn);
    return hip_result(lwg::launch_ln_affine(x, gamma, beta, y, rows, C, eps, static_cast<hipStream_t>(stream)), fn);
}

LWG_EXPORT int32_t lwg_add_ln_affine(const void* branch, const void* residual, const void* gamma,
                                     const void* beta, void* residual_out, void* y, int64_t rows, int32_t C,
                                     double eps, void* stream) {
    static const char* fn = "lwg_add_ln_affine";
    int32_t st;
    if ((st = check_width(fn, C)) || (st = check_eps(fn, eps)) || (st = check_rows(fn, "rows", rows)))
        return st;
    if (rows == 0) return ok();
    if ((st = check_tensor(fn, "branch", branch)) || (st = check_tensor(fn, "residual", residual)) ||
        (st = check_tensor(fn, "gamma", gamma)) || (st = check_tensor(fn, "beta", beta)) ||
        (st = check_tensor(fn, "residual_out", residual_out)) || (st = check_tensor(fn, "y", y)))
        return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * C * 2;
    const uint64_t pbytes = static_cast<uint64_t>(C) * 2;
    if (overlap(y, bytes, residual_out, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y and residual_out overlap", fn);
    if (!same_or_disjoint(residual_out, residual, bytes) || !same_or_disjoint(residual_out, branch, bytes) ||
        !same_or_disjoint(y, residual, bytes) || !same_or_disjoint(y, branch, bytes))
        return fail(LWG_ERR_ALIASING,
                    "%s: an output partially overlaps an input (only exact in-place aliasing is allowed)", fn);
    if (overlap(y, bytes, gamma, pbytes) || overlap(y, bytes, beta, pbytes) ||
        overlap(residual_out, bytes, gamma, pbytes) || overlap(residual_out, bytes, beta, pbytes))
        return fail(LWG_ERR_ALIASING, "%s: an output overlaps gamma or beta", fn);
    return hip_result(lwg::launch_add_ln_affine(branch, residual, gamma, beta, residual_out, y, rows, C, eps,
                                                static_cast<hipStream_t>(stream)),
                      fn);
}

LWG_EXPORT int32_t lwg_bias_gelu(const void* x, const void* bias, void* y, int64_t rows, int32_t cols,
                                 void* stream) {
    static const char* fn = "lwg_bias_gelu";
    int32_t st;
    if (cols < 4 || cols % 4 != 0)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: cols=%d must be a positive multiple of 4", fn, cols);
    if (rows < 0 || rows > INT32_MAX || rows * static_cast<int64_t>(cols) / 4 > INT32_MAX)
        return fail(LWG_ERR_INVALID_ARGUMENT, "%s: rows=%lld with cols=%d exceeds 2^31-1 float4 groups", fn,
                    static_cast<long long>(rows), cols);
    if (rows == 0) return ok();
    if ((st = check_tensor(fn, "x", x)) || (st = check_tensor(fn, "bias", bias)) || (st = check_tensor(fn, "y", y)))
        return st;
    const uint64_t bytes = static_cast<uint64_t>(rows) * cols * 4;
    if (!same_or_disjoint(x, y, bytes))
        return fail(LWG_ERR_ALIASING, "%s: y partially overlaps x (only y == x is allowed)", fn);
    if (overlap(y, bytes, bias, static_cast<uint64_t>(cols) * 4))
        return fail(LWG_ERR_ALIASING, "%s: y overlaps bias", fn);
    return hip_result(lwg::launch_bias_gelu(x, bias, y, rows, cols, static_cast<hipStream_t>(stream)), fn);
}

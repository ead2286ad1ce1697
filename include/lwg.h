/*
 * lwg.h -- C ABI of the fixed-width LayerNorm / shifted-window gather library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are the memory-bound row pipeline of a Pangu-Weather-style 3D
 * shifted-window transformer, as described on the page "Pangu-Weather inference
 * optimisation on Hygon BW1000 (gfx936)" (l189.com/news/2144533), sections 3-5.
 * The calling conventions (validate before launching, no launch on empty
 * input, enqueue on the caller's stream, report launch errors) follow the page
 * "PyTorch + HIP custom fused operator" (Hygon DCU practice series), section 6.
 *
 * Conventions shared by every call:
 *  - Tensors are contiguous row-major [rows, C] arrays of IEEE 754 binary16
 *    (lwg_bias_gelu alone takes float32). Token rows of a (Z,H,W) grid are
 *    stored in (z,h,w) order, z slowest.
 *  - Every tensor pointer is a device pointer, 16-byte aligned, allocated and
 *    freed by the caller. The library never allocates, frees, synchronises or
 *    changes the current device.
 *  - `stream` is a hipStream_t passed as void*; NULL means the legacy default
 *    stream. Work is enqueued asynchronously; a call returns before it runs.
 *  - Arguments are checked on the host before any HIP call. A non-OK status
 *    means nothing was enqueued; lwg_last_error() then describes the problem.
 *    Calls return an lwg_status value as int32_t, a type of fixed width for
 *    callers through a foreign-function interface.
 *  - eps is a double and enters the binary64 statistics as given (1e-5 is not
 *    exactly representable, and a float eps would differ from it).
 *  - rows == 0 (or n_out == 0) returns LWG_OK without launching anything; the
 *    pointers are not inspected in that case.
 *  - C = 192 and C = 384 (the model's hidden widths, section 3 of the BW1000
 *    page) and C = 768 (its patch-merge width: four 192-channel tokens
 *    concatenated) are served, each with its own tests. The page refuses widths
 *    without tests rather than serving them by an untested path; any other
 *    width returns LWG_ERR_UNSUPPORTED_WIDTH.
 *  - Statistics (row mean and biased variance) are accumulated in binary64 from
 *    the binary16 inputs and each output is rounded once to binary16, to
 *    nearest-even. The plain LayerNorm calls have no scale or shift (the
 *    BW1000 page folds the affine parameters into the following Linear at load
 *    time); lwg_ln_affine and lwg_add_ln_affine apply them for callers that
 *    do not fold.
 *  - Calls only enqueue kernels on `stream`, so they may be recorded by HIP
 *    stream capture into a graph and replayed. Calls on different threads
 *    are independent; lwg_last_error() is per thread. Calls that overlap on
 *    the device must not write the same memory.
 *  - Faults inside a kernel surface at the caller's next synchronisation.
 */
#ifndef LWG_H
#define LWG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LWG_ABI_VERSION 1

typedef enum lwg_status {
    LWG_OK = 0,
    LWG_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, bad eps, bad window */
    LWG_ERR_UNSUPPORTED_WIDTH = 2, /* C not in {192, 384, 768} */
    LWG_ERR_MISALIGNED = 3,        /* a tensor pointer not 16-byte aligned */
    LWG_ERR_ALIASING = 4,          /* an output overlaps an input in a way the call forbids */
    LWG_ERR_SIZE_MISMATCH = 5,     /* table length differs from the window token count */
    LWG_ERR_HIP = 6                /* the HIP runtime reported an error at launch */
} lwg_status;

/*
 * Fixed-width LayerNorm (BW1000 page, section 3).
 *   y[r, :] = (x[r, :] - mean_r) / sqrt(var_r + eps), var_r biased (divide by C).
 * x, y : [rows, C] binary16. y may equal x (in place); any other overlap is
 *        LWG_ERR_ALIASING.
 * eps  : finite and > 0 (1e-5 in the model).
 * A row holding Inf or NaN yields a NaN row; a constant row yields +0.0.
 */
int32_t lwg_ln_fixed(const void* x, void* y, int64_t rows, int32_t C, double eps,
                     void* stream);

/*
 * Residual add + LayerNorm (BW1000 page, section 4).
 *   residual_out = FP16(residual + branch)      (exact sum rounded once, nearest-even)
 *   y            = LayerNorm(residual_out)      (reads the rounded residual)
 * All four tensors are [rows, C] binary16. residual_out may equal residual or
 * branch (in-place update of the residual stream); y may equal residual or
 * branch. y and residual_out must not overlap each other, and no output may
 * partially overlap anything (LWG_ERR_ALIASING).
 */
int32_t lwg_add_ln(const void* branch, const void* residual, void* residual_out, void* y,
                   int64_t rows, int32_t C, double eps, void* stream);

/*
 * Number of rows of the gathered tensor for a (Z,H,W) grid cut into
 * (wz,wh,ww) windows: each extent is padded at its high end to a multiple of
 * the window extent and the padded extents are multiplied. Host only (no HIP
 * call). Returns -1 for a negative grid extent, a window extent < 1, or a
 * count above INT32_MAX.
 */
int64_t lwg_window_token_count(int32_t Z, int32_t H, int32_t W,
                               int32_t wz, int32_t wh, int32_t ww);

/*
 * INT32 shifted-window index table (BW1000 page, section 5: one INT32 index per
 * gathered token, padding folded into the index protocol).
 * Entry j (window-major: windows row-major over their (z,h,w) coordinates,
 * tokens row-major inside a window) is the source token index of gathered row j,
 * or -1 where that row is padding. The padded grid is rolled so that gathered
 * position p reads padded position (p + shift) mod padded_extent on each axis.
 * Shifts must be >= 0 and are taken modulo the padded extent.
 * table     : device int32 [table_len], written by one kernel on `stream`.
 * table_len : must equal lwg_window_token_count(Z,H,W,wz,wh,ww), else
 *             LWG_ERR_SIZE_MISMATCH. The grid must hold at most INT32_MAX tokens.
 */
int32_t lwg_window_index_build(int32_t Z, int32_t H, int32_t W,
                               int32_t wz, int32_t wh, int32_t ww,
                               int32_t sz, int32_t sh, int32_t sw,
                               int32_t* table, int64_t table_len, void* stream);

/*
 * Window token gather (BW1000 page, section 5).
 *   out[j, :] = x[table[j], :]   if 0 <= table[j] < n_src
 *             = +0.0             otherwise (-1 marks padding; any other
 *                                out-of-range entry is treated the same way and
 *                                never read)
 * x     : [n_src, C] binary16 (may be NULL when n_src == 0).
 * table : device int32 [n_out], 4-byte aligned.
 * out   : [n_out, C] binary16; must not overlap x or table.
 * n_src and n_out must not exceed INT32_MAX.
 */
int32_t lwg_window_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                          int64_t n_out, void* out, void* stream);

/*
 * Fused norm-gather (BW1000 page, section 5: norm1's output is consumed only by
 * the window gather, so the normalised tensor is never written).
 *   out[j, :] = LayerNorm(x[table[j], :])  if 0 <= table[j] < n_src, else +0.0
 * Same argument rules as lwg_window_gather, eps as in lwg_ln_fixed. Bitwise
 * equal to lwg_ln_fixed followed by lwg_window_gather.
 */
int32_t lwg_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                        int64_t n_out, double eps, void* out, void* stream);

/*
 * Inverse window table: one INT32 entry per source token (Z*H*W of them), the
 * gathered row that lwg_window_index_build's table sends that token to. Same
 * geometry arguments and rules as lwg_window_index_build. It drives the window
 * reverse that follows attention in a shifted-window block: the BW1000 page,
 * section 5, describes the forward gather; the reverse undoes it (windows back
 * onto the padded grid, roll back by +shift, crop the padding).
 * inverse     : device int32 [inverse_len], written by one kernel on `stream`.
 * inverse_len : must equal Z*H*W, else LWG_ERR_SIZE_MISMATCH.
 * The plain window reverse is lwg_window_gather(window_rows, M, C, inverse, Z*H*W, out).
 */
int32_t lwg_window_inverse_build(int32_t Z, int32_t H, int32_t W,
                                 int32_t wz, int32_t wh, int32_t ww,
                                 int32_t sz, int32_t sh, int32_t sw,
                                 int32_t* inverse, int64_t inverse_len, void* stream);

/*
 * Window reverse fused with residual add + LayerNorm (BW1000 page, section 4,
 * applied to the attention output that comes back in window order):
 *   branch[i]       = win[inverse[i]] if 0 <= inverse[i] < n_win, else +0.0
 *   residual_out[i] = FP16(residual[i] + branch[i])
 *   y[i]            = LayerNorm(residual_out[i])
 * win             : [n_win, C] binary16 rows in window order (padding rows are
 *                   never read).
 * inverse         : device int32 [rows], 4-byte aligned (lwg_window_inverse_build).
 * residual, residual_out, y : [rows, C] binary16. residual_out and y may each
 *                   equal residual; y and residual_out must not overlap; no output
 *                   may overlap win or inverse (LWG_ERR_ALIASING).
 * rows and n_win must not exceed INT32_MAX.
 */
int32_t lwg_window_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse,
                                  const void* residual, void* residual_out, void* y,
                                  int64_t rows, int32_t C, double eps, void* stream);

/*
 * Residual add + LayerNorm + window gather (BW1000 page, sections 4 and 5: the
 * residual sum is rounded to FP16 once and written; its LayerNorm feeds only the
 * window gather, so the normalised tensor is never written):
 *   residual_out[t] = FP16(residual[t] + branch[t])            for every token t
 *   out[j]          = LayerNorm(residual_out[table[j]])  if 0 <= table[j] < n_src,
 *                     else +0.0
 * branch, residual, residual_out : [n_src, C] binary16; out : [n_out, C].
 * The valid entries of table must be distinct and cover every token (the tables
 * of lwg_window_index_build are); a token no entry names keeps its residual_out
 * row unwritten. residual_out may equal residual or branch. out must not
 * overlap any other argument, and residual_out must not overlap table.
 */
int32_t lwg_add_norm_gather(const void* branch, const void* residual, void* residual_out,
                            int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                            double eps, void* out, void* stream);

/*
 * Affine LayerNorm, for callers that do not fold the scale and shift into the
 * next Linear (the BW1000 page, section 3, folds them at load time):
 *   y[r, c] = (x[r, c] - mean_r) / sqrt(var_r + eps) * gamma[c] + beta[c]
 * evaluated in binary64 and rounded once to binary16.
 * gamma, beta : device binary16 [C], 16-byte aligned, read by every wave.
 * x, y        : as in lwg_ln_fixed (y may equal x); y must not overlap gamma or beta.
 */
int32_t lwg_ln_affine(const void* x, const void* gamma, const void* beta, void* y,
                      int64_t rows, int32_t C, double eps, void* stream);

/*
 * Residual add + affine LayerNorm: residual_out = FP16(residual + branch) as in
 * lwg_add_ln (section 4), y = affine LayerNorm of residual_out as in
 * lwg_ln_affine. Aliasing rules of lwg_add_ln; outputs must not overlap gamma
 * or beta.
 */
int32_t lwg_add_ln_affine(const void* branch, const void* residual, const void* gamma,
                          const void* beta, void* residual_out, void* y, int64_t rows,
                          int32_t C, double eps, void* stream);

/*
 * Bias + tanh-approximated GELU in float32 (the fused operator of the page
 * "PyTorch + HIP custom fused operator", sections 3-6):
 *   t = x[r, c] + bias[c]  (float32 add)
 *   y[r, c] = 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3)))
 * evaluated as t / (1 + exp(-2z)) with the hardware exponential and
 * reciprocal (within a few float32 ulp of the exact value; the page's gate is
 * rtol = atol = 2e-5).
 * x, y : device float32 [rows, cols], 16-byte aligned; y may equal x.
 * bias : device float32 [cols], 16-byte aligned; must not overlap y.
 * cols : a positive multiple of 4, and rows*cols/4 at most INT32_MAX.
 * This operation is not part of the LayerNorm/gather path and takes float32,
 * not binary16.
 */
int32_t lwg_bias_gelu(const void* x, const void* bias, void* y, int64_t rows, int32_t cols,
                      void* stream);

/* Static, human-readable name of a status code. */
const char* lwg_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next lwg_* call on that thread. */
const char* lwg_last_error(void);

/* LWG_ABI_VERSION of the loaded library. */
int32_t lwg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LWG_H */

// Internal launchers between the C ABI (argument checks) and the kernels.
// Every launcher assumes its arguments were validated by the caller: sizes in
// range, C in {192, 384, 768}, pointers non-null and 16-byte aligned.
#ifndef LWG_LAUNCH_H
#define LWG_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwg {

// Division of a dividend below 2^31 by a fixed divisor d >= 1 with one 64-bit
// multiply and a shift: q = (n * m) >> s with s = 31 + ceil(log2 d) and
// m = ceil(2^s / d) < 2^32. The rounding error of m times n stays below 1/d for
// every n < 2^31, so q is exactly floor(n / d) (the round-up reciprocal method
// of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint32_t s = 31 + l;
    const uint64_t num = uint64_t{1} << s;
    return FastDiv{d, static_cast<uint32_t>((num + d - 1) / d), s};
}

// Geometry of one shifted-window table, reduced on the host: shifts already
// taken modulo the padded extents, all products known to fit in int32.
struct WindowGeometry {
    int32_t Z, H, W;        // token grid
    int32_t wz, wh, ww;     // window extents
    int32_t Zp, Hp, Wp;     // padded extents
    int32_t sz, sh, sw;     // shifts, 0 <= s < padded extent
    int32_t nbh, nbw;       // windows along h and w
    int32_t win_tokens;     // wz * wh * ww
    int32_t rows;           // Zp * Hp * Wp
    FastDiv div_win, div_nbw, div_nbh, div_ww, div_wh;  // forward table
    FastDiv div_W, div_H, div_wz;                        // inverse table
};

hipError_t launch_ln_fixed(const void* x, void* y, int64_t rows, int32_t C, double eps,
                           hipStream_t stream);
hipError_t launch_add_ln(const void* branch, const void* residual, void* residual_out,
                         void* y, int64_t rows, int32_t C, double eps, hipStream_t stream);
hipError_t launch_window_index(const WindowGeometry& g, int32_t* table, hipStream_t stream);
hipError_t launch_window_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                                int64_t n_out, void* out, hipStream_t stream);
hipError_t launch_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                              int64_t n_out, double eps, void* out, hipStream_t stream);
hipError_t launch_window_inverse(const WindowGeometry& g, int32_t* inverse, hipStream_t stream);
hipError_t launch_bias_gelu(const void* x, const void* bias, void* y, int64_t rows, int32_t cols,
                            hipStream_t stream);
hipError_t launch_ln_affine(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                            int32_t C, double eps, hipStream_t stream);
hipError_t launch_add_ln_affine(const void* branch, const void* residual, const void* gamma, const void* beta,
                                void* residual_out, void* y, int64_t rows, int32_t C, double eps,
                                hipStream_t stream);
hipError_t launch_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse,
                                 const void* residual, void* residual_out, void* y, int64_t rows,
                                 int32_t C, double eps, hipStream_t stream);
hipError_t launch_add_norm_gather(const void* branch, const void* residual, void* residual_out,
                                  int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                                  double eps, void* out, hipStream_t stream);

}  // namespace lwg

#endif

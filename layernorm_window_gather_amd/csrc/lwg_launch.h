// Internal launchers between the C ABI (argument checks) and the kernels.
// Every launcher assumes its arguments were validated by the caller: sizes in
// range, C in {192, 384}, pointers non-null and 16-byte aligned.
#ifndef LWG_LAUNCH_H
#define LWG_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwg {

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

}  // namespace lwg

#endif

// Stand-ins for the kernel launchers (lwg_launch.h) used by the host-only
// sanitizer build of the C ABI. They launch nothing. Each records that it was
// reached and checks the preconditions lwg_launch.h states for its arguments
// (sizes in range, C served, pointers non-null and aligned, window geometry
// consistent), so that the argument checks in front of them are tested for
// letting through only what the launchers accept.
#include <cstdint>
#include <cstdio>

#include "lwg_launch.h"
#include "abi_stubs.h"

namespace stubs {
std::atomic<long> g_launches{0};
std::atomic<long> g_violations{0};
}  // namespace stubs

namespace {

void expect(bool ok, const char* what) {
    if (!ok) {
        ++stubs::g_violations;
        std::fprintf(stderr, "launcher precondition violated: %s\n", what);
    }
}

bool served(int32_t C) { return C == 192 || C == 384 || C == 768; }
bool a16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool a4(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool rows_ok(int64_t r) { return r > 0 && r <= INT32_MAX; }

hipError_t reached() {
    ++stubs::g_launches;
    return hipSuccess;
}

bool fastdiv_ok(const lwg::FastDiv& f) {
    if (f.d == 0) return false;
    // spot-check the reciprocal on the divisor's neighbourhood and at the top of the range
    const uint32_t probes[] = {0u, 1u, f.d - 1u, f.d, f.d + 1u, 2u * f.d - 1u, 0x7FFFFFFFu, 0x7FFFFFFEu};
    for (uint32_t n : probes) {
        if (n > 0x7FFFFFFFu) continue;
        const uint32_t q = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.s);
        if (q != n / f.d) return false;
    }
    return true;
}

void geometry_ok(const lwg::WindowGeometry& g) {
    expect(g.Z >= 0 && g.H >= 0 && g.W >= 0, "grid extents >= 0");
    expect(g.wz >= 1 && g.wh >= 1 && g.ww >= 1, "window extents >= 1");
    expect(g.Zp >= g.Z && g.Hp >= g.H && g.Wp >= g.W, "padded extents cover the grid");
    expect(g.Zp % g.wz == 0 && g.Hp % g.wh == 0 && g.Wp % g.ww == 0, "padded extents are window multiples");
    expect(g.sz >= 0 && g.sz < g.Zp && g.sh >= 0 && g.sh < g.Hp && g.sw >= 0 && g.sw < g.Wp,
           "shifts reduced modulo the padded extents");
    expect(static_cast<int64_t>(g.Zp) * g.Hp * g.Wp == g.rows, "rows is the padded volume");
    expect(g.rows > 0 && g.rows <= INT32_MAX, "rows in (0, 2^31)");
    expect(static_cast<int64_t>(g.wz) * g.wh * g.ww == g.win_tokens, "window volume");
    expect(g.nbh == g.Hp / g.wh && g.nbw == g.Wp / g.ww, "window counts");
    expect(fastdiv_ok(g.div_win) && fastdiv_ok(g.div_nbw) && fastdiv_ok(g.div_nbh) && fastdiv_ok(g.div_ww) &&
               fastdiv_ok(g.div_wh),
           "forward reciprocals exact");
}

}  // namespace

namespace lwg {

hipError_t launch_ln_fixed(const void* x, void* y, int64_t rows, int32_t C, double eps, hipStream_t) {
    expect(a16(x) && a16(y) && rows_ok(rows) && served(C) && eps > 0, "ln_fixed");
    return reached();
}

hipError_t launch_add_ln(const void* b, const void* r, void* ro, void* y, int64_t rows, int32_t C, double eps,
                         hipStream_t) {
    expect(a16(b) && a16(r) && a16(ro) && a16(y) && rows_ok(rows) && served(C) && eps > 0, "add_ln");
    return reached();
}

hipError_t launch_window_index(const WindowGeometry& g, int32_t* table, hipStream_t) {
    expect(a4(table), "window_index table");
    geometry_ok(g);
    return reached();
}

hipError_t launch_window_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                                void* out, hipStream_t) {
    expect((n_src == 0 || a16(x)) && n_src >= 0 && n_src <= INT32_MAX && a4(table) && rows_ok(n_out) &&
               a16(out) && served(C),
           "window_gather");
    return reached();
}

hipError_t launch_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                              double eps, void* out, hipStream_t) {
    expect((n_src == 0 || a16(x)) && n_src >= 0 && n_src <= INT32_MAX && a4(table) && rows_ok(n_out) &&
               a16(out) && served(C) && eps > 0,
           "norm_gather");
    return reached();
}

hipError_t launch_window_inverse(const WindowGeometry& g, int32_t* inverse, hipStream_t) {
    expect(a4(inverse), "window_inverse table");
    geometry_ok(g);
    expect(static_cast<int64_t>(g.Z) * g.H * g.W > 0 && static_cast<int64_t>(g.Z) * g.H * g.W <= INT32_MAX,
           "token count in (0, 2^31)");
    expect(fastdiv_ok(g.div_W) && fastdiv_ok(g.div_H) && fastdiv_ok(g.div_wz), "inverse reciprocals exact");
    return reached();
}

hipError_t launch_bias_gelu(const void* x, const void* bias, void* y, int64_t rows, int32_t cols, hipStream_t) {
    expect(a16(x) && a16(bias) && a16(y) && rows_ok(rows) && cols > 0 && cols % 4 == 0 &&
               rows * static_cast<int64_t>(cols) / 4 <= INT32_MAX,
           "bias_gelu");
    return reached();
}

hipError_t launch_ln_affine(const void* x, const void* g, const void* b, void* y, int64_t rows, int32_t C,
                            double eps, hipStream_t) {
    expect(a16(x) && a16(g) && a16(b) && a16(y) && rows_ok(rows) && served(C) && eps > 0, "ln_affine");
    return reached();
}

hipError_t launch_add_ln_affine(const void* br, const void* r, const void* g, const void* b, void* ro, void* y,
                                int64_t rows, int32_t C, double eps, hipStream_t) {
    expect(a16(br) && a16(r) && a16(g) && a16(b) && a16(ro) && a16(y) && rows_ok(rows) && served(C) && eps > 0,
           "add_ln_affine");
    return reached();
}

hipError_t launch_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse, const void* r, void* ro,
                                 void* y, int64_t rows, int32_t C, double eps, hipStream_t) {
    expect((n_win == 0 || a16(win)) && n_win >= 0 && n_win <= INT32_MAX && a4(inverse) && a16(r) && a16(ro) &&
               a16(y) && rows_ok(rows) && served(C) && eps > 0,
           "reverse_add_ln");
    return reached();
}

hipError_t launch_add_norm_gather(const void* b, const void* r, void* ro, int64_t n_src, int32_t C,
                                  const int32_t* table, int64_t n_out, double eps, void* out, hipStream_t) {
    // with no source rows every gathered row is padding and the token tensors are not touched
    expect((n_src == 0 || (a16(b) && a16(r) && a16(ro))) && n_src >= 0 && n_src <= INT32_MAX && a4(table) &&
               rows_ok(n_out) && a16(out) && served(C) && eps > 0,
           "add_norm_gather");
    return reached();
}

}  // namespace lwg

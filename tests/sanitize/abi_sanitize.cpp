// Host-only exercise of every C entry point of include/lwg.h, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against lwg_abi.hip and the
// stand-in launchers of abi_stubs.cpp (no GPU, no kernel code).
//
// Pointers here are addresses that are never dereferenced: the argument checks
// compare and align them, nothing more. Each call must
//   * return a status of the lwg_status enum,
//   * leave a message in lwg_last_error() when it refuses,
//   * reach its launcher exactly once when it accepts non-empty work, never
//     when it refuses or the work is empty,
// and every accepted call must satisfy the launcher's preconditions (checked by
// the stubs). A fixed list of cases names the expected status of each refusal;
// a seeded sweep then draws arguments from extreme sets (sizes at and past the
// 2^31 limits, widths, misaligned and overlapping pointers, non-finite eps,
// huge grids, zero and negative windows) and checks the same properties.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>

#include "lwg.h"
#include "abi_stubs.h"

namespace {

int g_failures = 0;

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
int32_t* T(uintptr_t a) { return reinterpret_cast<int32_t*>(a); }

// Check one call: status in range, message on refusal, launch count as expected.
void check(const char* what, int32_t st, long launches_before, bool empty, int32_t want = -1) {
    const long launched = stubs::g_launches - launches_before;
    bool ok = st >= LWG_OK && st <= LWG_ERR_HIP;
    if (want >= 0 && st != want) ok = false;
    if (st != LWG_OK && (lwg_last_error() == nullptr || lwg_last_error()[0] == '\0')) ok = false;
    if (st != LWG_OK && launched != 0) ok = false;
    if (st == LWG_OK && launched != (empty ? 0 : 1)) ok = false;
    if (!ok) {
        ++g_failures;
        std::fprintf(stderr, "FAIL %s: status %d (%s), want %d, launches %ld, empty %d, msg '%s'\n", what, st,
                     lwg_status_string(st), want, launched, empty, lwg_last_error());
    }
}

constexpr uintptr_t A = 0x10000000, B = 0x20000000, Cc = 0x30000000, D = 0x40000000, E = 0x50000000,
                    F = 0x60000000, G = 0x70000000;
constexpr double kEps = 1e-5;

void fixed_cases() {
    long n;
    // ln_fixed
    n = stubs::g_launches; check("ln ok", lwg_ln_fixed(P(A), P(B), 10, 192, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("ln in place", lwg_ln_fixed(P(A), P(A), 10, 384, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("ln empty", lwg_ln_fixed(nullptr, nullptr, 0, 192, kEps, nullptr), n, true, LWG_OK);
    n = stubs::g_launches; check("ln width", lwg_ln_fixed(P(A), P(B), 10, 256, kEps, nullptr), n, false, LWG_ERR_UNSUPPORTED_WIDTH);
    n = stubs::g_launches; check("ln null", lwg_ln_fixed(nullptr, P(B), 10, 192, kEps, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("ln misaligned", lwg_ln_fixed(P(A + 8), P(B), 10, 192, kEps, nullptr), n, false, LWG_ERR_MISALIGNED);
    n = stubs::g_launches; check("ln partial", lwg_ln_fixed(P(A), P(A + 384), 10, 192, kEps, nullptr), n, false, LWG_ERR_ALIASING);
    n = stubs::g_launches; check("ln rows<0", lwg_ln_fixed(P(A), P(B), -1, 192, kEps, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("ln rows>2^31", lwg_ln_fixed(P(A), P(B), int64_t{1} << 31, 192, kEps, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("ln rows max", lwg_ln_fixed(P(A), P(B), INT64_MAX, 768, kEps, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("ln eps nan", lwg_ln_fixed(P(A), P(B), 10, 192, std::nan(""), nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("ln eps 0", lwg_ln_fixed(P(A), P(B), 10, 192, 0.0, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    // add_ln
    n = stubs::g_launches; check("add ok", lwg_add_ln(P(A), P(B), P(Cc), P(D), 7, 192, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("add in place", lwg_add_ln(P(A), P(B), P(B), P(A), 7, 768, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("add y=ro", lwg_add_ln(P(A), P(B), P(Cc), P(Cc), 7, 192, kEps, nullptr), n, false, LWG_ERR_ALIASING);
    n = stubs::g_launches; check("add partial", lwg_add_ln(P(A), P(B), P(B + 16), P(D), 7, 192, kEps, nullptr), n, false, LWG_ERR_ALIASING);
    // tables
    const int64_t m = lwg_window_token_count(8, 182, 90, 2, 6, 12);
    n = stubs::g_launches; check("index ok", lwg_window_index_build(8, 182, 90, 2, 6, 12, 1, 3, 6, T(A), m, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("index len", lwg_window_index_build(8, 182, 90, 2, 6, 12, 1, 3, 6, T(A), m - 1, nullptr), n, false, LWG_ERR_SIZE_MISMATCH);
    n = stubs::g_launches; check("index window 0", lwg_window_index_build(8, 182, 90, 0, 6, 12, 0, 0, 0, T(A), m, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("index shift<0", lwg_window_index_build(8, 182, 90, 2, 6, 12, -1, 0, 0, T(A), m, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("index huge grid", lwg_window_index_build(INT32_MAX, INT32_MAX, INT32_MAX, 1, 1, 1, 0, 0, 0, T(A), 1, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("index table misaligned", lwg_window_index_build(8, 182, 90, 2, 6, 12, 1, 3, 6, T(A + 2), m, nullptr), n, false, LWG_ERR_MISALIGNED);
    n = stubs::g_launches; check("index empty", lwg_window_index_build(0, 182, 90, 2, 6, 12, 1, 3, 6, nullptr, 0, nullptr), n, true, LWG_OK);
    n = stubs::g_launches; check("inverse ok", lwg_window_inverse_build(8, 182, 90, 2, 6, 12, 1, 3, 6, T(A), 8 * 182 * 90, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("inverse len", lwg_window_inverse_build(8, 182, 90, 2, 6, 12, 1, 3, 6, T(A), m, nullptr), n, false, LWG_ERR_SIZE_MISMATCH);
    if (lwg_window_token_count(INT32_MAX, INT32_MAX, INT32_MAX, 1, 1, 1) != -1) {
        ++g_failures;
        std::fprintf(stderr, "FAIL token count of a huge grid is not -1\n");
    }
    if (lwg_window_token_count(8, 182, 90, 2, 6, 12) != 142848) {
        ++g_failures;
        std::fprintf(stderr, "FAIL level-1 token count\n");
    }
    // gathers
    n = stubs::g_launches; check("gather ok", lwg_window_gather(P(A), 100, 192, T(B), 120, P(Cc), nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("gather no source", lwg_window_gather(nullptr, 0, 192, T(B), 120, P(Cc), nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("gather out=x", lwg_window_gather(P(A), 100, 192, T(B), 120, P(A), nullptr), n, false, LWG_ERR_ALIASING);
    n = stubs::g_launches; check("norm gather eps", lwg_norm_gather(P(A), 100, 384, T(B), 120, -1.0, P(Cc), nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("norm gather table over out", lwg_norm_gather(P(A), 100, 192, T(Cc + 64), 120, kEps, P(Cc), nullptr), n, false, LWG_ERR_ALIASING);
    // fused
    n = stubs::g_launches; check("reverse ok", lwg_window_reverse_add_ln(P(A), 120, T(B), P(Cc), P(D), P(E), 100, 192, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("reverse out over win", lwg_window_reverse_add_ln(P(A), 120, T(B), P(Cc), P(A), P(E), 100, 192, kEps, nullptr), n, false, LWG_ERR_ALIASING);
    n = stubs::g_launches; check("add norm gather ok", lwg_add_norm_gather(P(A), P(B), P(B), 100, 192, T(Cc), 120, kEps, P(D), nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("add norm gather partial", lwg_add_norm_gather(P(A), P(B), P(B + 32), 100, 192, T(Cc), 120, kEps, P(D), nullptr), n, false, LWG_ERR_ALIASING);
    // affine and GELU
    n = stubs::g_launches; check("affine ok", lwg_ln_affine(P(A), P(B), P(Cc), P(D), 10, 192, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("affine y over gamma", lwg_ln_affine(P(A), P(B), P(Cc), P(B), 10, 192, kEps, nullptr), n, false, LWG_ERR_ALIASING);
    n = stubs::g_launches; check("add affine ok", lwg_add_ln_affine(P(A), P(B), P(Cc), P(D), P(E), P(F), 10, 384, kEps, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("gelu ok", lwg_bias_gelu(P(A), P(B), P(Cc), 4, 768, nullptr), n, false, LWG_OK);
    n = stubs::g_launches; check("gelu cols", lwg_bias_gelu(P(A), P(B), P(Cc), 4, 766, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("gelu too many", lwg_bias_gelu(P(A), P(B), P(Cc), INT32_MAX, 8, nullptr), n, false, LWG_ERR_INVALID_ARGUMENT);
    n = stubs::g_launches; check("gelu in place", lwg_bias_gelu(P(A), P(B), P(A), 4, 768, nullptr), n, false, LWG_OK);
    (void)G;
}

template <class V, size_t N>
V pick(std::mt19937_64& rng, const V (&v)[N]) {
    return v[rng() % N];
}

void sweep(long iterations) {
    std::mt19937_64 rng(20260716);
    const int64_t rows_set[] = {-1, 0, 1, 3, 8, 65, 131040, INT32_MAX, int64_t{1} << 31, INT64_MAX, INT64_MIN, -131040};
    const int32_t width_set[] = {192, 384, 768, 0, 1, 191, 193, 256, 1536, -192, INT32_MAX, INT32_MIN};
    const double eps_set[] = {kEps, 1e-12, 1.0, 0.0, -1e-5, std::nan(""), INFINITY, -INFINITY,
                              std::numeric_limits<double>::denorm_min(), std::numeric_limits<double>::max()};
    const uintptr_t ptr_set[] = {0, A, B, Cc, D, A + 4, A + 8, A + 16, A + 384, B + 2, ~uintptr_t{0} - 15,
                                 uintptr_t{1} << 47};
    const int32_t ext_set[] = {-1, 0, 1, 2, 5, 8, 12, 91, 182, 1093, 65536, INT32_MAX, INT32_MIN};
    const int32_t win_set[] = {-1, 0, 1, 2, 6, 12, 7, 1000, INT32_MAX};
    const int32_t shift_set[] = {-1, 0, 1, 3, 6, 1000, INT32_MAX};
    const int32_t cols_set[] = {4, 8, 768, 1024, 2048, 0, -4, 3, 6, INT32_MAX - 3};
    for (long it = 0; it < iterations; ++it) {
        const int op = static_cast<int>(rng() % 12);
        const int64_t r1 = pick(rng, rows_set), r2 = pick(rng, rows_set);
        const int32_t C = pick(rng, width_set);
        const double eps = pick(rng, eps_set);
        void *p1 = P(pick(rng, ptr_set)), *p2 = P(pick(rng, ptr_set)), *p3 = P(pick(rng, ptr_set)),
             *p4 = P(pick(rng, ptr_set)), *p5 = P(pick(rng, ptr_set)), *p6 = P(pick(rng, ptr_set));
        const long before = stubs::g_launches;
        int32_t st = 0;
        bool empty = false;
        switch (op) {
            case 0: st = lwg_ln_fixed(p1, p2, r1, C, eps, nullptr); empty = r1 == 0; break;
            case 1: st = lwg_add_ln(p1, p2, p3, p4, r1, C, eps, nullptr); empty = r1 == 0; break;
            case 2: st = lwg_window_gather(p1, r1, C, static_cast<int32_t*>(p2), r2, p3, nullptr); empty = r2 == 0; break;
            case 3: st = lwg_norm_gather(p1, r1, C, static_cast<int32_t*>(p2), r2, eps, p3, nullptr); empty = r2 == 0; break;
            case 4: st = lwg_window_reverse_add_ln(p1, r1, static_cast<int32_t*>(p2), p3, p4, p5, r2, C, eps, nullptr); empty = r2 == 0; break;
            case 5: st = lwg_add_norm_gather(p1, p2, p3, r1, C, static_cast<int32_t*>(p4), r2, eps, p5, nullptr); empty = r2 == 0; break;
            case 6: st = lwg_ln_affine(p1, p2, p3, p4, r1, C, eps, nullptr); empty = r1 == 0; break;
            case 7: st = lwg_add_ln_affine(p1, p2, p3, p4, p5, p6, r1, C, eps, nullptr); empty = r1 == 0; break;
            case 8: {
                const int32_t cols = pick(rng, cols_set);
                st = lwg_bias_gelu(p1, p2, p3, r1, cols, nullptr);
                empty = r1 == 0;
                break;
            }
            case 9:
            case 10: {
                const int32_t Z = pick(rng, ext_set), H = pick(rng, ext_set), W = pick(rng, ext_set);
                const int32_t wz = pick(rng, win_set), wh = pick(rng, win_set), ww = pick(rng, win_set);
                const int32_t sz = pick(rng, shift_set), sh = pick(rng, shift_set), sw = pick(rng, shift_set);
                const int64_t m = lwg_window_token_count(Z, H, W, wz, wh, ww);
                const __int128 t128 = static_cast<__int128>(Z) * H * W;
                const int64_t tokens = (Z >= 0 && H >= 0 && W >= 0 && t128 <= INT32_MAX) ? static_cast<int64_t>(t128) : -1;
                const bool right_len = rng() % 4 != 0;
                if (op == 9) {
                    const int64_t len = right_len ? m : r1;
                    st = lwg_window_index_build(Z, H, W, wz, wh, ww, sz, sh, sw, static_cast<int32_t*>(p1), len, nullptr);
                    empty = st == LWG_OK && m == 0;
                } else {
                    const int64_t len = right_len ? tokens : r1;
                    st = lwg_window_inverse_build(Z, H, W, wz, wh, ww, sz, sh, sw, static_cast<int32_t*>(p1), len, nullptr);
                    empty = st == LWG_OK && tokens == 0;
                }
                break;
            }
            default: {
                const int32_t Z = pick(rng, ext_set), H = pick(rng, ext_set), W = pick(rng, ext_set);
                const int32_t wz = pick(rng, win_set), wh = pick(rng, win_set), ww = pick(rng, win_set);
                const int64_t m = lwg_window_token_count(Z, H, W, wz, wh, ww);
                if (m < -1 || m > INT32_MAX) {
                    ++g_failures;
                    std::fprintf(stderr, "FAIL token count %lld out of range\n", static_cast<long long>(m));
                }
                continue;
            }
        }
        char what[64];
        std::snprintf(what, sizeof what, "sweep op %d iteration %ld", op, it);
        check(what, st, before, empty);
    }
}

}  // namespace

int main(int argc, char** argv) {
    const long iterations = argc > 1 ? std::atol(argv[1]) : 200000;
    fixed_cases();
    sweep(iterations);
    std::printf("abi_sanitize: %ld launches reached, %ld launcher precondition violations, %d failures\n",
                stubs::g_launches.load(), stubs::g_violations.load(), g_failures);
    return (g_failures == 0 && stubs::g_violations == 0) ? 0 : 1;
}

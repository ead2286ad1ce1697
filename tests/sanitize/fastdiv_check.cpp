// Exhaustive-at-the-edges check of the multiply-shift division used by the
// window-table kernels (make_fastdiv in lwg_launch.h): for every divisor
// d in [1, 2^16] and the dividends around every multiple of d near zero, near
// 2^31 - 1 and at seeded random points below 2^31, (n * m) >> s == n / d.
// Also every divisor that is a power of two or one off it up to 2^31 - 1.
#include <cstdint>
#include <cstdio>
#include <random>

#include "lwg_launch.h"

namespace {

long g_checked = 0, g_wrong = 0;

void check(const lwg::FastDiv& f, uint32_t n) {
    const uint32_t q = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.s);
    ++g_checked;
    if (q != n / f.d && g_wrong++ < 10) std::fprintf(stderr, "wrong: %u / %u -> %u\n", n, f.d, q);
}

void check_divisor(uint32_t d, std::mt19937_64& rng) {
    const lwg::FastDiv f = lwg::make_fastdiv(d);
    const uint32_t top = 0x7FFFFFFFu;
    for (uint32_t k = 0; k < 64; ++k) {                 // around the first multiples of d
        const uint64_t base = static_cast<uint64_t>(k) * d;
        for (int e = -1; e <= 1; ++e) {
            const int64_t n = static_cast<int64_t>(base) + e;
            if (n >= 0 && n <= top) check(f, static_cast<uint32_t>(n));
        }
    }
    const uint32_t last = top / d * d;                   // around the last multiples below 2^31
    for (uint32_t k = 0; k < 64 && last >= static_cast<uint64_t>(k) * d; ++k) {
        const uint64_t base = last - static_cast<uint64_t>(k) * d;
        for (int e = -1; e <= 1; ++e) {
            const int64_t n = static_cast<int64_t>(base) + e;
            if (n >= 0 && n <= top) check(f, static_cast<uint32_t>(n));
        }
    }
    check(f, top);
    for (int i = 0; i < 64; ++i) check(f, static_cast<uint32_t>(rng() & top));
}

}  // namespace

int main() {
    std::mt19937_64 rng(20260716);
    for (uint32_t d = 1; d <= (1u << 16); ++d) check_divisor(d, rng);
    for (int b = 1; b < 31; ++b)
        for (int e = -1; e <= 1; ++e) check_divisor((1u << b) + e, rng);
    check_divisor(0x7FFFFFFFu, rng);
    for (int i = 0; i < 20000; ++i) check_divisor(1 + static_cast<uint32_t>(rng() % 0x7FFFFFFFu), rng);
    std::printf("fastdiv_check: %ld divisions checked, %ld wrong\n", g_checked, g_wrong);
    return g_wrong == 0 ? 0 : 1;
}

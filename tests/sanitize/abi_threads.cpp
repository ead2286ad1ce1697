// Concurrent callers of the C ABI, host-only, with the stand-in launchers of
// abi_stubs.cpp (nothing is launched and no pointer is dereferenced). Each
// thread alternates a refused call that carries a value of its own with
// accepted calls to other entry points, and checks after every call that
// lwg_last_error() is that thread's own message: its refusal, or empty after
// its own success. Built with ThreadSanitizer, which also reports any data
// race in the argument checks.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "abi_stubs.h"
#include "lwg.h"

namespace {

// Stand-in device buffers: large enough for every call below, never touched.
alignas(256) unsigned char g_a[1 << 16], g_b[1 << 16], g_c[1 << 16], g_d[1 << 16];
alignas(256) int32_t g_table[1 << 12];

constexpr double kEps = 1e-5;
constexpr int kAcceptedPerIteration = 3;

void worker(int tid, int iterations, std::atomic<long>& failures) {
    const int32_t bad_width = 200 + tid;      // never a served width
    char want[64];
    std::snprintf(want, sizeof want, "C=%d is not served", bad_width);
    // a 2 x 6 x 12 grid under a (2, 6, 12) window: exactly one window, 144 rows
    const int64_t m = lwg_window_token_count(2, 6, 12, 2, 6, 12);
    for (int i = 0; i < iterations; ++i) {
        if (lwg_ln_fixed(g_a, g_b, 10, bad_width, kEps, nullptr) != LWG_ERR_UNSUPPORTED_WIDTH ||
            std::strstr(lwg_last_error(), want) == nullptr)
            ++failures;
        if (lwg_add_ln(g_a, g_b, g_c, g_d, 7, 384, kEps, nullptr) != LWG_OK || lwg_last_error()[0] != '\0')
            ++failures;
        if (lwg_norm_gather(g_a, 3, bad_width, g_table, 5, kEps, g_b, nullptr) != LWG_ERR_UNSUPPORTED_WIDTH ||
            std::strstr(lwg_last_error(), want) == nullptr)
            ++failures;
        if (lwg_window_index_build(2, 6, 12, 2, 6, 12, 1, 3, 6, g_table, m, nullptr) != LWG_OK ||
            lwg_last_error()[0] != '\0')
            ++failures;
        if (lwg_window_gather(g_a, 20, 192, g_table, 9 + tid, g_c, nullptr) != LWG_OK || lwg_last_error()[0] != '\0')
            ++failures;
    }
}

}  // namespace

int main(int argc, char** argv) {
    const int threads = argc > 1 ? std::atoi(argv[1]) : 8;
    const int iterations = argc > 2 ? std::atoi(argv[2]) : 20000;
    std::atomic<long> failures{0};
    const long before = stubs::g_launches.load();
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) pool.emplace_back(worker, t, iterations, std::ref(failures));
    for (auto& th : pool) th.join();
    const long launched = stubs::g_launches.load() - before;
    const long expected = static_cast<long>(threads) * iterations * kAcceptedPerIteration;
    std::printf("abi_threads: %d threads x %d iterations, %ld launches reached (expected %ld), "
                "%ld launcher precondition violations, %ld failures\n",
                threads, iterations, launched, expected, stubs::g_violations.load(), failures.load());
    return (failures == 0 && launched == expected && stubs::g_violations == 0) ? 0 : 1;
}

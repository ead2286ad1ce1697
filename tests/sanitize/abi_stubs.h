// Counters kept by the stand-in launchers of abi_stubs.cpp.
#ifndef LWG_ABI_STUBS_H
#define LWG_ABI_STUBS_H
#include <atomic>
namespace stubs {
extern std::atomic<long> g_launches;    // launchers reached
extern std::atomic<long> g_violations;  // launcher preconditions found false
}  // namespace stubs
#endif

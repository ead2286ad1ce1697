// Counters kept by the stand-in launchers of abi_stubs.cpp.
#ifndef LWG_ABI_STUBS_H
#define LWG_ABI_STUBS_H
namespace stubs {
extern long g_launches;    // launchers reached
extern long g_violations;  // launcher preconditions found false
}  // namespace stubs
#endif

// Kernel launches stubbed out for the host sanitizer build of afd_host.cpp
// (test infrastructure): that build checks only host code paths that refuse
// or compute before launching anything; reaching a launch is an error.
#include <cstdio>
#include <cstdlib>

#include "../../combine_afd_slot_amd/csrc/afd_internal.h"

namespace afd {
[[noreturn]] static void reached(const char* what) {
    std::fprintf(stderr, "host sanitizer build: %s reached\n", what);
    std::abort();
}
hipError_t launch_pack_weights(const DevCtx&, const afd_moe_weights&, char*, const int64_t*, int64_t, hipStream_t) {
    reached("launch_pack_weights");
}
hipError_t launch_pack(const DevCtx&, int, int, int, int, const void*, const float*, uint32_t, int, hipStream_t) {
    reached("launch_pack");
}
hipError_t launch_unpack_ranks(const DevCtx* const*, int, int, int, int, const int*, void*, const long long*,
                               hipStream_t) {
    reached("launch_unpack_ranks");
}
hipError_t launch_unpack(const DevCtx&, int, int, int, int, void*, long long, hipStream_t) { reached("launch_unpack"); }
hipError_t launch_ffn(const DevCtx&, int, int, const Weights&, long long, int, hipEvent_t*, hipStream_t, int, long long,
                      int) {
    reached("launch_ffn");
}
hipError_t launch_serve_begin(const DevCtx&, hipStream_t) { reached("launch_serve_begin"); }
hipError_t launch_zero(void*, int64_t, hipStream_t) { reached("launch_zero"); }
}  // namespace afd

// Host-only stand-ins for the kernel launchers of libkda.so, so that the C
// ABI's validation (kda_api.cpp) can be built with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.
// Each stand-in counts the launches that reach it and returns success.
#include "kda_bwd.h"
#include "kda_internal.h"

int g_launches = 0;

namespace kda {

hipError_t launch_step(int, int, int, const StepArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_chunk(int, int, int, const ChunkArgs&, hipStream_t, hipEvent_t*, int) {
    ++g_launches;
    return hipSuccess;
}
int chunk_kernel_count(int, int, int, int, int NC) { return NC > 0 ? 2 : 1; }
hipError_t launch_layer(int, int, int, const ChunkArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_compose(int, const ComposeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fixup(int, int, const FixupArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
int short_conv_tile() { return 32; }
hipError_t launch_short_conv(int, const ShortConvArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_output_gate(int, int, const GateArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_chunk_bwd(int, int, const BwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
// the launch stand-ins never touch memory, so any aligned address serves
hipError_t scratch_pointer(void** ptr) {
    alignas(256) static unsigned char host_stand_in[256];
    *ptr = host_stand_in;
    return hipSuccess;
}

}  // namespace kda

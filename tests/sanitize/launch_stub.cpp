// launch_stub.cpp -- host-only stand-ins for the HIP launchers and
// hipGetLastError, so that the C ABI's validation (gdn_api.cpp) can be built
// and run under AddressSanitizer/UBSan on a machine without a GPU. Each stub
// checks the invariants validation promises its launcher and counts the call.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include "gdn_launch.h"

int g_launches = 0;

static void require(bool ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "launcher invariant violated: %s\n", what);
        abort();
    }
}

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace gdn {

hipError_t launch_prefill(const PrefillArgs& a, int dtype, hipStream_t) {
    require(a.q && a.k && a.v && a.g_log && a.beta && a.state && a.out, "prefill pointers");
    require(a.B >= 1 && a.Hk >= 1 && a.Hv % a.Hk == 0 && a.S >= 1, "prefill shape");
    require(a.Dk % 16 == 0 && a.Dv % 16 == 0 && a.Dk <= 128 && a.Dv <= 128, "prefill dims");
    require(dtype == 0 || dtype == 1, "prefill dtype");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t) {
    require(a.g_log && a.beta && a.state && a.out, "decode pointers");
    require(a.B >= 1 && a.Hk >= 1 && a.Hv % a.Hk == 0, "decode shape");
    require(dtype == 0 || dtype == 1, "decode dtype");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_conv1d(const ConvArgs& a, int dtype, bool, hipStream_t) {
    require(a.x && a.w && a.out && a.state && a.B >= 1 && a.C >= 1 && a.T >= 1, "conv args");
    require(a.K >= 1 && a.K <= 8 && (dtype == 0 || dtype == 1), "conv taps/dtype");
    require(a.T <= 2147483647 - 65536, "conv token headroom");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_decode_block(const DecodeArgs& a, const BlockArgs& b, int dtype, hipStream_t) {
    require(a.state && a.out && b.mixed && b.z && b.conv_in && b.conv_out, "block pointers");
    require(b.K >= 1 && b.K <= 8 && (dtype == 0 || dtype == 1), "block taps/dtype");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_rmsnorm_gated(const NormArgs& a, int dtype, hipStream_t) {
    require(a.o && a.z && a.w && a.out && a.B >= 1 && a.Hv >= 1 && a.S >= 1, "norm args");
    require(a.S <= 2147483647 - 65536 && (dtype == 0 || dtype == 1), "norm tokens/dtype");
    ++g_launches;
    return hipSuccess;
}

}  // namespace gdn

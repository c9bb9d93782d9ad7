// Stand-ins for the GPU side of libfa in a host-only sanitizer build of its
// C ABI (fa_api.cpp).  No device is reported, so every call that passes
// argument validation stops at the device check with FA_ERR_DEVICE; the
// launchers are never reached and abort if they are.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "fa_internal.hpp"

extern "C" hipError_t hipGetDevice(int *device)
{
    if (device) *device = -1;
    return hipErrorNoDevice;
}

extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *, int)
{
    return hipErrorNoDevice;
}

namespace fa {
int fwd_f32_kv_tile(int d) { return d == 64 ? 64 : 32; }
int fwd_mfma_kv_tile(int, long long, long long, long long) { return 32; }
int decode_chunk_keys(int) { return 512; }
int fwd_fp8_kv_tile() { return 64; }
hipError_t launch_fwd_mfma(const FwdProblem &, hipStream_t) { std::abort(); }
hipError_t launch_fwd_f32(const FwdProblem &, hipStream_t) { std::abort(); }
hipError_t launch_decode(const DecodeProblem &, hipStream_t) { std::abort(); }
hipError_t launch_bwd(const BwdProblem &, hipStream_t) { std::abort(); }
hipError_t launch_quant(const QuantProblem &, hipStream_t) { std::abort(); }
hipError_t launch_fwd_fp8(const Fp8Problem &, hipStream_t) { std::abort(); }
hipError_t launch_cast_e4m3(const float *, uint8_t *, float *, size_t, hipStream_t) { std::abort(); }
hipError_t decode_scratch(void **) { std::abort(); }
}  // namespace fa

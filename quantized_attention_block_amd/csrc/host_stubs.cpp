// Host-only stand-ins for the kernel launchers, linked only into the
// sanitizer build of the C ABI (g++ with -fsanitize=address,undefined): that
// build exercises argument validation, workspace sizing and error reporting,
// which all run before any launch.  Every launcher here fails with
// hipErrorNoDevice, so a call that passes validation reports SAGE_ERR_HIP; no
// computation exists outside the HIP kernels.
#include "sage_launch.hpp"

namespace sage {

hipError_t launch_k_mean_partial(const HalfView&, int, int, int, int, double*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_k_mean_final(double*, int, int, int, int, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_qk_int8(const HalfView&, const HalfView&, int, int, int, int, int, int, bool, double*,
                                uint64_t*, float*, int8_t*, float*, int8_t*, float*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_quant_v(const HalfView&, int, int, int, int, float*, uint64_t*, uint8_t*, float*, hipStream_t) {
    return hipErrorNoDevice;
}
void set_quant_wait_us(int) {}
hipError_t launch_quant_qk_mxfp4(const HalfView&, const HalfView&, int, int, int, int, int, const float*,
                                 const void*, const void*, float, float*, uint8_t*, uint8_t*, uint8_t*,
                                 uint8_t*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_attn_fwd(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_qk(const int8_t*, const int8_t*, int, int, int, int, int, int, int, int, int, int32_t*,
                           hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_debug_qk_mx(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int, int, int,
                              int, int, int, int, int, float*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_debug_cvt_e4m3(const float*, uint8_t*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_cvt_e2m1(const float*, uint8_t*, int64_t, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_paged_decode(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t decode_scratch(void**) { return hipErrorNoDevice; }
hipError_t launch_hadamard_build(int, void*, void*, hipStream_t) { return hipErrorNoDevice; }

}  // namespace sage

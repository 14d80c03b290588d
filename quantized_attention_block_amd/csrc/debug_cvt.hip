// Test hooks for the two hardware number conversions the kernels code with:
//  - fp32 -> OCP e4m3 (`cvt_pk_fp8`): P8 = e4m3(448 p) in attention and decode,
//    V8 in the V quantizers, the decode's per-row query codes;
//  - fp32 -> E2M1 after division by 2^ex (`cvt_pk_e2m1` with
//    `mx_scale_operand`): the MXFP4 quantizer's and the fused-Q prologue's
//    element codes (OCP MX v1.0 shared-exponent blocks).
// Each thread codes one pair of inputs with the same device function, in the
// same pairing (element 2i low, 2i + 1 high), and stores one code per byte, so
// that a test can hold every code against the oracle's encoder.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {
namespace {

constexpr int kCvtThreads = 256;
constexpr int kCvtBlocks = 8192;   // grid-stride: any n with a fixed grid

__global__ __launch_bounds__(kCvtThreads) void k_debug_cvt_e4m3(const float* x, uint8_t* out, int64_t n) {
    const int64_t pairs = (n + 1) / 2;
    for (int64_t p = (int64_t)blockIdx.x * kCvtThreads + threadIdx.x; p < pairs;
         p += (int64_t)gridDim.x * kCvtThreads) {
        const int64_t i = 2 * p;
        const bool two = i + 1 < n;
        const uint32_t w = cvt_pk_fp8<false>(x[i], two ? x[i + 1] : 0.0f, 0u);
        out[i] = (uint8_t)w;
        if (two) out[i + 1] = (uint8_t)(w >> 8);
    }
}

__global__ __launch_bounds__(kCvtThreads) void k_debug_cvt_e2m1(const float* x, uint8_t* out, int64_t n, int ex) {
    const float sc = mx_scale_operand(ex);
    const int64_t pairs = (n + 1) / 2;
    for (int64_t p = (int64_t)blockIdx.x * kCvtThreads + threadIdx.x; p < pairs;
         p += (int64_t)gridDim.x * kCvtThreads) {
        const int64_t i = 2 * p;
        const bool two = i + 1 < n;
        const uint32_t w = cvt_pk_e2m1<0>(0u, x[i], two ? x[i + 1] : 0.0f, sc);
        out[i] = (uint8_t)(w & 0xF);
        if (two) out[i + 1] = (uint8_t)((w >> 4) & 0xF);
    }
}

int cvt_grid(int64_t n) {
    const int64_t blocks = ((n + 1) / 2 + kCvtThreads - 1) / kCvtThreads;
    return (int)(blocks < kCvtBlocks ? (blocks > 0 ? blocks : 1) : kCvtBlocks);
}

}  // namespace

hipError_t launch_debug_cvt_e4m3(const float* x, uint8_t* out, int64_t n, hipStream_t stream) {
    k_debug_cvt_e4m3<<<cvt_grid(n), kCvtThreads, 0, stream>>>(x, out, n);
    return hipGetLastError();
}

hipError_t launch_debug_cvt_e2m1(const float* x, uint8_t* out, int64_t n, int ex, hipStream_t stream) {
    k_debug_cvt_e2m1<<<cvt_grid(n), kCvtThreads, 0, stream>>>(x, out, n, ex);
    return hipGetLastError();
}

}  // namespace sage

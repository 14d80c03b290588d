// Device-side helpers shared by the gfx950 kernels of the quantized-attention
// library: vector types, MFMA wrappers, number-format conversions.
//
// MFMA lane layouts used throughout (gfx950, wave64; checked on hardware):
//   v_mfma_i32_32x32x32_i8 / v_mfma_f32_32x32x64_f8f6f4 / ..._32x32x16_bf16:
//     A operand: lane l holds row (l % 32), K-slice (l / 32) of the
//                instruction's K (16 int8, 32 fp8, 32 fp4 or 8 bf16 values,
//                in order; fp4 nibble 2i is the low nibble of byte i).
//     B operand: lane l holds column (l % 32), the same K-slice.
//     C/D:       lane l holds column (l % 32); element e = 4 i + j is row
//                8 i + 4 (l / 32) + j.
//   With the scaled f8f6f4 form, each lane's E8M0 scale multiplies the 32
//   values it supplies (one MX block).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kFp8Max = 448.0f;   // OCP e4m3 largest finite value

// ---- MFMA wrappers --------------------------------------------------------
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// e4m3 x e4m3, fp32 accumulate (format code 0 on both operands, unit scales)
__device__ __forceinline__ v16f mfma_f8_32x32x64(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// e4m3 x e4m3 16x16x128: lane l supplies row / column l % 16 and K-slice
// [32 (l / 16), +32); element i of the result is row 4 (l / 16) + i, column l % 16
__device__ __forceinline__ v4f mfma_f8_16x16x128(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// E2M1 x E2M1 with per-lane E8M0 scales (byte 0 of sa / sb); only the first
// four dwords of a and b are read.
// A: E2M1 (low four dwords) with E8M0 block scale sa; B: e4m3, scale 2^0.
__device__ __forceinline__ v4f mfma_f4f8_16x16x128(v8i a, v8i b, v4f c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, 127);
}

__device__ __forceinline__ v16f mfma_f4_32x32x64(v8i a, v8i b, v16f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}
__device__ __forceinline__ v16f mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16_32x32x16(f16x8 a, f16x8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---- conversions ----------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Two fp32 -> two OCP e4m3 codes in the low (word 0) or high (word 1) half of
// `old`.  Hardware conversion: round to nearest even, exact for |x| <= 448
// (inputs of this library never exceed 448 by more than rounding slack, which
// still rounds to 448).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_fp8(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// fp32 -> E2M1 nibble, round to nearest even, saturating at 6 (|x| < 8 on the
// quantization path: x = value * 2^-e with amax * 2^-e in [4, 8)).
__device__ __forceinline__ uint32_t e2m1_rne(float x) {
    uint32_t s = (__float_as_uint(x) >> 31) << 3;
    float a = fabsf(x);
    uint32_t c;
    if (a < 2.0f) {
        c = (uint32_t)__builtin_rintf(a * 2.0f);           // 0, 0.5, 1, 1.5, 2
    } else if (a < 4.0f) {
        c = 4u + (uint32_t)__builtin_rintf(a - 2.0f);      // 2, 3, 4
    } else {
        float t = __builtin_rintf((a - 4.0f) * 0.5f);      // 4, 6 (ties to 4)
        c = 6u + (uint32_t)fminf(t, 1.0f);
    }
    return s | c;
}

// MX shared exponent of a block: floor(log2(amax)) - 2 from the fp32 bits,
// clamped to [-127, 127]; amax == 0 -> -127.
__device__ __forceinline__ int mx_exponent(float amax) {
    uint32_t b = __float_as_uint(amax);
    if (b == 0) return -127;
    int ef = (int)((b >> 23) & 0xFF);
    int fl;
    if (ef != 0) {
        fl = ef - 127;
    } else {
        fl = (31 - __builtin_clz(b & 0x7FFFFF)) - 149;
    }
    int e = fl - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---- wave reductions ------------------------------------------------------
// Max of v over the lane pair (l % 32, l % 32 + 32): v_permlane32_swap hands
// each lane both halves' values without an LDS round trip.
__device__ __forceinline__ float half_pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Raw buffer resource over [base, base + bytes): stride 0, loads past the end
// return 0 and stores past it are dropped (bounds clamped to 2^31 - 1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                             0x00020000);   // gfx9 raw-buffer config
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

}  // namespace sage

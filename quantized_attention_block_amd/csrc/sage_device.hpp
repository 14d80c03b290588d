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

typedef int v2i __attribute__((ext_vector_type(2)));
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
// still rounds to 448); the GPU tests compare it with the oracle's encoder
// over every fp32 input of magnitude below 464.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_fp8(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
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

// ---- Hadamard rotation + MXFP4 quantization of one wave's 32 tokens -------
// Shared by the MXFP4 quantizer and the attention kernel's fused-Q prologue, so
// that both give the same codes bit for bit.  Lane l holds token (l % 32):
//   xb[kc]: its channels [16 kc + 8 (l / 32), +8) (half precision, bf16 or fp16)
//   hs:     the 128 x 128 +-1 Hadamard matrix in LDS, row-major, same precision,
//           16-byte chunk c of row r stored at chunk c ^ (r % 16) of the row (the
//           256-byte rows are one full sweep of the LDS banks: unswizzled, the
//           16 rows one read pass fetches at one column meet on the same banks)
// Y^T = H X^T on MFMA (H's entries and the inputs are exact, fp32 accumulation
// over kc ascending), then y = (Y - sub) * inv_sqrt_r, with y[cb][e] channel
// 32 cb + 8 (e / 4) + 4 (l / 32) + (e % 4) of the token.  Invalid tokens give 0.

// The MFMA chain of output channels [32 cb, +32).
template <bool BF16>
__device__ __forceinline__ v16f mx_rotate_block(const uint16_t* hs, const uint4 (&xb)[8], int cb) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
    v16f acc = {0};
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
        const int hr = 32 * cb + col, hc = (2 * kc + half) ^ (hr & 15);
        const uint4 ha = *(const uint4*)&hs[hr * D + 8 * hc];
        if constexpr (BF16)
            acc = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ha), __builtin_bit_cast(bf16x8, xb[kc]), acc);
        else
            acc = mfma_f16_32x32x16(__builtin_bit_cast(f16x8, ha), __builtin_bit_cast(f16x8, xb[kc]), acc);
    }
    return acc;
}

// Input precision fixed at compile time; sub (per channel, e.g. the rotated K
// mean, zeros for none; 16-byte aligned) is never NULL.  Subtracting +0 leaves every value,
// -0 included, as it is, so rows with a zero sub get the codes of the form
// below.
template <bool BF16>
__device__ __forceinline__ void mx_rotate_rows(const uint16_t* hs, const uint4 (&xb)[8], float inv_sqrt_r,
                                               const float* sub, bool valid, float (&y)[4][16]) {
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const v16f acc = mx_rotate_block<BF16>(hs, xb, cb);
        // (sub is read unconditionally: a read inside the selection becomes a
        // branch around each load)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 sv = *(const float4*)&sub[32 * cb + 8 * i + 4 * half];
            const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float r = (acc[4 * i + j] - sc[j]) * inv_sqrt_r;
                y[cb][4 * i + j] = valid ? r : 0.0f;
            }
        }
    }
}

// Precision chosen at run time, nothing subtracted (the fused Q of attention).
__device__ __forceinline__ void mx_rotate_rows(const uint16_t* hs, const uint4 (&xb)[8], bool bf16,
                                               float inv_sqrt_r, bool valid, float (&y)[4][16]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const v16f acc = bf16 ? mx_rotate_block<true>(hs, xb, cb) : mx_rotate_block<false>(hs, xb, cb);
#pragma unroll
        for (int e = 0; e < 16; ++e) y[cb][e] = valid ? acc[e] * inv_sqrt_r : 0.0f;
    }
}

// Scale operand of gfx950's scaled conversions for the MX exponent ex in
// [-127, 127]: the E8M0 byte ex + 127 in the fp32 exponent field (field 0
// stands for 2^-127).
__device__ __forceinline__ float mx_scale_operand(int ex) {
    return __builtin_bit_cast(float, (uint32_t)(ex + 127) << 23);
}

// E2M1 codes of a * 2^-ex and b * 2^-ex (sc = mx_scale_operand(ex)) into
// byte SEL of w, a in the low nibble.  gfx950's scaled conversion divides by
// the E8M0 value of the scale and rounds to the nearest E2M1 value (0, 0.5,
// 1, 1.5, 2, 3, 4, 6; ties to the even code), saturating at 6; the GPU tests
// compare it with the oracle's encoder over every fp32 input below 8 * 2^ex
// for ex = 0 and over the rounding boundaries of every ex.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_e2m1(uint32_t w, float a, float b, float sc) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, sc, SEL);
}

// MX blocks of the values above: per 32-channel block cb the shared exponent
// ex[cb] = floor(log2 amax) - 2 (the lane and its partner l ^ 32 hold the
// block's two halves) and the E2M1 codes of y * 2^-ex, packed four per
// uint16: pk[cb][i] holds channels 32 cb + 8 i + 4 (l / 32) + 0..3, i.e.
// bytes 4 i + 2 (l / 32) + {0, 1} of the block's 16 packed bytes.
__device__ __forceinline__ void mx_quant_rows(const float (&y)[4][16], int (&ex)[4], uint16_t (&pk)[4][4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(y[cb][e]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        ex[cb] = mx_exponent(amax);
        // the E2M1 code of y * 2^-ex, two values per instruction
        const float sc = mx_scale_operand(ex[cb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w = cvt_pk_e2m1<0>(0u, y[cb][4 * i], y[cb][4 * i + 1], sc);
            w = cvt_pk_e2m1<1>(w, y[cb][4 * i + 2], y[cb][4 * i + 3], sc);
            pk[cb][i] = (uint16_t)w;
        }
    }
}

// Max over the wave, in every lane, by an xor butterfly of lane shuffles
// (LDS permutes).  Used where registers are at their limit: the DPP form
// below needs one more live register.
__device__ __forceinline__ float wave_max_xor(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// max of v and the value of the lane that DPP control CTRL names (all rows
// and banks enabled; the controls used stay inside a 16-lane row)
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF,
                                                                 0xF, false)));
}

// Max over the wave, in every lane, with no LDS round trip: within each quad
// (lane ^ 1, lane ^ 2: quad_perm), across the two quads of a half-row
// (row_half_mirror), the two halves of a row (row_mirror), then across rows
// with v_permlane16_swap (lane ^ 16) and v_permlane32_swap (lane ^ 32).
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_max<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_max<0x141>(v);   // row_half_mirror
    v = dpp_max<0x140>(v);   // row_mirror
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return half_pair_max(v);
}

}  // namespace sage

// Host-side launch interface between the C ABI layer (abi.cpp) and the gfx950
// kernels.  Every launcher only enqueues on `stream` and returns the launch
// status; all argument validation has already happened in abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// A logical [B, L, H, D] half-precision view with element strides (stride of
// D is 1).
struct HalfView {
    const void* ptr;
    int64_t sB, sL, sH;
    int bf16;   // 1: bfloat16, 0: float16
};

// Output view [B, L, H, D] with element strides.
constexpr int kOutF16 = 0, kOutBF16 = 1, kOutF32 = 2;
struct OutView {
    void* ptr;
    int64_t sB, sL, sH;
    int dtype;   // kOutF16 / kOutBF16 / kOutF32
};

constexpr int kKvTile = 64;        // KV tile of the attention kernel (online-softmax block)
constexpr int kMeanChunk = 256;    // tokens per partial sum of the K mean
constexpr int kDecodeTile = 256;   // decode split length (tokens)

__host__ __device__ inline int pad128(int L) { return (L + 127) / 128 * 128; }
inline int mean_chunks(int L) { return (L + kMeanChunk - 1) / kMeanChunk; }

// K mean: partial binary64 sums [B*H, nchunk, D] (nchunk = mean_chunks(L));
// the final mean mu fp32 [B*H, D] (sum in chunk order / L; mu may be NULL),
// also left, as binary64, over chunk 0 of the partials.
hipError_t launch_k_mean_partial(const HalfView& k, int B, int H, int L, int D, double* partial,
                                 hipStream_t stream);
hipError_t launch_k_mean_final(double* partial, int B, int H, int L, int D, float* mu,
                               hipStream_t stream);

// INT8 block quantization of Q (128-row blocks) and K (k_block rows, 64 or
// 128), K smoothed by its channel mean when `smooth` (written to mu_out when
// not NULL).  Scratch (used when smooth): mean_partial fp64 [B*H,
// mean_chunks(Lk), D] and sync uint64 [quant_sync_words(B*H, Lk)].
hipError_t launch_quant_qk_int8(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                int Lk, int D, int k_block, bool smooth, double* mean_partial,
                                uint64_t* sync, float* mu_out, int8_t* q_out, float* q_scale,
                                int8_t* k_out, float* k_scale, hipStream_t stream);

// V -> e4m3 transposed [B, H, D, pad128(Lk)] with per-channel scales.
// Scratch: amax_partial fp32 [B*H, mean_chunks(Lk), D] and sync uint64
// [quant_sync_words(B*H, Lk)].
hipError_t launch_quant_v(const HalfView& v, int B, int H, int Lk, int D, float* amax_partial,
                          uint64_t* sync, uint8_t* v_out, float* v_scale, hipStream_t stream);

// Microseconds a block of the single-read quantizers waits for the other
// blocks of its head before computing the head's statistic itself (default
// 2000; the outputs are the same either way).
void set_quant_wait_us(int us);

// Words of the quantizers' head-synchronization scratch (arrival flags and
// epochs; needs no initialization).
inline int64_t quant_sync_words(int64_t BH, int Lk) { return BH * mean_chunks(Lk) + BH; }

// Hadamard rotation (optional) + MXFP4 quantization of Q and smoothed K.
// hadamard_bf16 / hadamard_f16: 128x128 +-1 matrices (NULL: no rotation);
// mu_rot_ws: fp32 [B*H, D] scratch for mu * H.
hipError_t launch_quant_qk_mxfp4(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                 int Lk, int D, const float* mu, const void* hadamard_bf16,
                                 const void* hadamard_f16, float inv_sqrt_r, float* mu_rot_ws,
                                 uint8_t* q_out, uint8_t* q_e8, uint8_t* k_out, uint8_t* k_e8,
                                 hipStream_t stream);

struct AttnArgs {
    const void* q;        // int8 [B,H,Lqp,D] or fp4x2 [B,H,Lqp,D/2]
    const void* q_scale;  // fp32 [B,H,Lqp/q_block] or e8m0 [B,H,Lqp,D/32]
    const void* k;
    const void* k_scale;
    const uint8_t* v;     // e4m3 [B,Hkv,D,Lkp]
    const float* v_scale; // [B,Hkv,D]
    OutView out;
    int B, H, Hkv, Lq, Lk, D;
    int q_block, k_block;
    int causal;
    int mxfp4;
    int pingpong;         // the wave-pair schedule (INT8, D 128): 8-wave workgroups
    float sm_scale;
    // q_fused: Q is the caller's fp16/bf16 [B, Lq, H, D] view qh (q and
    // q_scale unused), quantized in the prologue: INT8 per 128-row block, or
    // (mxfp4) rotated by the Hadamard matrices below (NULL: no rotation) and
    // quantized to MXFP4
    int q_fused;
    HalfView qh;
    const void* hmat_bf16;
    const void* hmat_f16;
    float inv_sqrt_r;
};
// The part of AttnArgs the attention kernel itself takes (the fused-Q view
// travels as a kernel argument of its own).
struct AttnKernelArgs {
    const void* q;
    const void* q_scale;
    const void* k;
    const void* k_scale;
    const uint8_t* v;
    const float* v_scale;
    OutView out;
    int B, H, Hkv, Lq, Lk, D;
    int q_block, k_block;
    int causal;
    const void* hmat;     // fused MXFP4 Q: the 128 x 128 Hadamard in Q's precision (NULL: none)
    float inv_sqrt_r;
};
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);

hipError_t launch_debug_qk(const int8_t* q, const int8_t* k, int B, int H, int Lqp, int Lkp,
                           int D, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t stream);
// MXFP4 codes [B,H,Lqp,64] / [B,H,Lkp,64] with E8M0 scales [.., 4]; D = 128
hipError_t launch_debug_qk_mx(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                              const uint8_t* k_scale, int B, int H, int Lqp, int Lkp, int q0, int nq,
                              int k0, int nk, float* out, hipStream_t stream);

// fp32 -> e4m3 codes (the kernels' conversion), and fp32 * 2^-ex -> E2M1
// codes (the MXFP4 quantizer's), one code per byte, n >= 1
hipError_t launch_debug_cvt_e4m3(const float* x, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_debug_cvt_e2m1(const float* x, uint8_t* out, int64_t n, int ex, hipStream_t stream);

constexpr int kQueryBF16 = 0, kQueryF16 = 1, kQueryE4M3 = 2;
struct DecodeArgs {
    const void* q;            // bf16 / fp16 / e4m3 (q_kind)
    int64_t q_sB, q_sM, q_sH;
    const uint8_t* k_cache;   // [P,Hkv,page,D]
    const uint8_t* v_cache;   // [P,Hkv,D,page] or [P,Hkv,page,D]
    const float* k_scale;     // [P,Hkv,page]
    const float* v_scale;
    const int32_t* page_table;
    int64_t pt_stride;
    const int32_t* ctx_lens;
    void* out;                // bf16
    int64_t o_sB, o_sM, o_sH;
    int B, MTP, Hq, Hkv, D, page, num_pages, max_pages;
    int window, v_transposed, num_splits;
    int max_ctx;              // context lengths are clamped to it (it sizes the split plan)
    int mx;                   // 1: MXFP4 cache (E2M1 codes, E8M0 scales) as documented in sage.h
    int scale_per_tensor;     // e4m3 cache: k_scale / v_scale hold one value each
    int q_kind;               // kQueryBF16 / kQueryF16 / kQueryE4M3
    const float* q_scale;     // e4m3 q: [1] or [B, MTP, Hq]
    int q_scale_per_tensor;
    int out_f16;              // out is fp16 (else bf16)
    float sm_scale;
    float* partials;          // [B, Hkv, num_splits, rows] rows of fp16 h[DD], fp32 m, l, vmax, pad
};
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

// Fixed scratch of the no-allocation decode entry point (a file-scope device
// array of this many bytes per device); decode_scratch returns the current
// device's address of it.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

hipError_t launch_hadamard_build(int R, void* bf16_mat, void* f16_mat, hipStream_t stream);

}  // namespace sage

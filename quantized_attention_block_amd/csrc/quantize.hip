// Quantization kernels for gfx950: K channel mean, INT8 block quantization of
// Q and smoothed K, FP8 e4m3 per-channel quantization of V (written
// transposed), and Hadamard rotation + MXFP4 quantization of Q and K.
//
// Method sources (titles and sections of the pages):
//  - SageAttention2 as used by "Sage v2" (xDiT pull request 665, "Sage v2
//    improvements"): per-block INT8 Q/K, K smoothed by its channel mean, FP8
//    V with a per-channel scale; the MXFP4 variant rotates Q and K by a
//    Hadamard matrix of order BLOCK_R = 128 that is built once.
//  - "Sage2 SM89 Temporal Pair Experiment" README, Candidate: the V scale is
//    fused into the attention epilogue, so V is stored as e4m3 codes plus one
//    fp32 scale per channel.
// These kernels are HBM-bound: each reads its input once per pass and keeps
// the block it quantizes in registers between the amax pass and the code pass.
#include "sage_device.hpp"
#include "sage_launch.hpp"

#pragma clang fp contract(off)

namespace sage {
namespace {

constexpr int kThreads = 256;

template <int D>
struct Rows {
    static constexpr int kLanesPerRow = D / 8;            // 16-byte chunks per row
    static constexpr int kRowsPerPass = kThreads / kLanesPerRow;
};

// Loads 8 consecutive channels [8 c8, 8 c8 + 8) of token l of head h, batch b.
__device__ __forceinline__ void load8(const HalfView& v, int b, int l, int h, int c8, float out[8]) {
    const uint16_t* p = (const uint16_t*)v.ptr + (int64_t)b * v.sB + (int64_t)l * v.sL +
                        (int64_t)h * v.sH + c8 * 8;
    uint4 u = *(const uint4*)p;
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (v.bf16) {
            out[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFF);
            out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        } else {
            out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFF);
            out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
        }
    }
}

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// ---- K mean ----------------------------------------------------------------
// Partial binary64 sums over chunks of kMeanChunk tokens; fixed summation
// order (per thread ascending rows, then ascending row groups), so the result
// is deterministic.
template <int D>
__global__ __launch_bounds__(kThreads) void k_mean_partial(HalfView k, int H, int L, int nchunk,
                                                           double* partial) {
    using G = Rows<D>;
    const int bh = blockIdx.y, b = bh / H, h = bh % H, chunk = blockIdx.x;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int lo = chunk * kMeanChunk, hi = min(L, lo + kMeanChunk);
    for (int l = lo + r0; l < hi; l += G::kRowsPerPass) {
        float x[8];
        load8(k, b, l, h, c8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
    }
    __shared__ double sm[kThreads][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = acc[i];
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        double s = 0.0;
        for (int r = 0; r < G::kRowsPerPass; ++r) s += sm[r * G::kLanesPerRow + d / 8][d % 8];
        partial[((int64_t)bh * nchunk + chunk) * D + d] = s;
    }
}

template <int D>
__global__ void k_mean_final(const double* partial, int nchunk, int L, float* mu) {
    const int bh = blockIdx.x, d = threadIdx.x;
    double s = 0.0;
    for (int c = 0; c < nchunk; ++c) s += partial[((int64_t)bh * nchunk + c) * D + d];
    mu[(int64_t)bh * D + d] = L > 0 ? (float)(s / (double)L) : 0.0f;
}

// ---- INT8 block quantization -------------------------------------------------
// One block per (token block, b*h).  Q blocks first, then K blocks.  Per block:
// amax over the valid rows (K: of fp32(K - mu)), scale = amax / 127,
// codes = clamp(rne(x * (127 / amax)), -127, 127); padded rows get code 0.
template <int D>
__global__ __launch_bounds__(kThreads) void k_quant_int8(HalfView q, HalfView k, int H, int Lq,
                                                         int Lk, int q_block, int k_block, int nqb,
                                                         const float* mu, int8_t* q_out,
                                                         float* q_scale, int8_t* k_out,
                                                         float* k_scale) {
    using G = Rows<D>;
    constexpr int kMaxPass = 128 / G::kRowsPerPass;
    const bool isq = (int)blockIdx.x < nqb;
    const int blk = isq ? blockIdx.x : blockIdx.x - nqb;
    const int BLK = isq ? q_block : k_block;
    const int L = isq ? Lq : Lk;
    const int Lp = pad128(L);
    const HalfView& src = isq ? q : k;
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int passes = BLK / G::kRowsPerPass;
    const int row0 = blk * BLK;

    float mu8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mu8[i] = (!isq && mu) ? mu[(int64_t)bh * D + c8 * 8 + i] : 0.0f;

    float vals[kMaxPass][8];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        const int row = row0 + p * G::kRowsPerPass + r0;
        if (p < passes && row < L) {
            load8(src, b, row, h, c8, vals[p]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                vals[p][i] = vals[p][i] - mu8[i];
                amax = fmaxf(amax, fabsf(vals[p][i]));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) vals[p][i] = 0.0f;
        }
    }
    __shared__ float red[kThreads / 64];
    amax = block_max(amax, red);
    float inv = 0.0f, scale = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        scale = amax / 127.0f;
    }
    int8_t* out = isq ? q_out : k_out;
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        const int row = row0 + p * G::kRowsPerPass + r0;
        if (p < passes && row < Lp) {
            uint32_t w[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float r = __builtin_rintf(vals[p][i] * inv);
                r = fminf(127.0f, fmaxf(-127.0f, r));
                w[i / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i % 4));
            }
            *(uint2*)(out + ((int64_t)bh * Lp + row) * D + c8 * 8) = make_uint2(w[0], w[1]);
        }
    }
    if (threadIdx.x == 0) {
        float* so = isq ? q_scale : k_scale;
        so[(int64_t)bh * (Lp / BLK) + blk] = scale;
    }
}

// ---- V: per-channel amax, then e4m3 codes written transposed ----------------
__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_v_amax(HalfView v, int H, int L, uint32_t* amax) {
    using G = Rows<D>;
    const int bh = blockIdx.y, b = bh / H, h = bh % H, chunk = blockIdx.x;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int lo = chunk * kMeanChunk, hi = min(L, lo + kMeanChunk);
    for (int l = lo + r0; l < hi; l += G::kRowsPerPass) {
        float x[8];
        load8(v, b, l, h, c8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(x[i]));
    }
    __shared__ float sm[kThreads][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = m[i];
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float r = 0.0f;
        for (int g = 0; g < G::kRowsPerPass; ++g) r = fmaxf(r, sm[g * G::kLanesPerRow + d / 8][d % 8]);
        // non-negative floats order like their bit patterns
        atomicMax(amax + (int64_t)bh * D + d, __float_as_uint(r));
    }
}

// One block per 64 keys of one (b, h): codes = e4m3(v * (448 / amax[d])),
// transposed through LDS so that each channel row of the output receives 64
// contiguous key bytes.
template <int D>
__global__ __launch_bounds__(kThreads) void k_v_quant(HalfView v, int H, int L,
                                                      const uint32_t* amax, uint8_t* v_out,
                                                      float* v_scale) {
    using G = Rows<D>;
    constexpr int kKeys = 64;
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int k0 = blockIdx.x * kKeys;
    const int Lp = pad128(L);
    __shared__ float inv_s[D];
    __shared__ uint8_t tile[D][kKeys];
    if (threadIdx.x < D) {
        const float a = __uint_as_float(amax[(int64_t)bh * D + threadIdx.x]);
        inv_s[threadIdx.x] = a > 0.0f ? kFp8Max / a : 0.0f;
        if (blockIdx.x == 0) v_scale[(int64_t)bh * D + threadIdx.x] = a / kFp8Max;
    }
    __syncthreads();
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
#pragma unroll
    for (int p = 0; p < kKeys / G::kRowsPerPass; ++p) {
        const int kl = p * G::kRowsPerPass + r0, key = k0 + kl;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (key < L) load8(v, b, key, h, c8, x);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float a0 = x[i] * inv_s[c8 * 8 + i];
            const float a1 = x[i + 1] * inv_s[c8 * 8 + i + 1];
            const uint32_t c = cvt_pk_fp8<false>(a0, a1, 0);
            tile[c8 * 8 + i][kl] = (uint8_t)(c & 0xFF);
            tile[c8 * 8 + i + 1][kl] = (uint8_t)((c >> 8) & 0xFF);
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D * (kKeys / 16); c += kThreads) {
        const int d = c / (kKeys / 16), part = c % (kKeys / 16);
        const uint4 val = *(const uint4*)&tile[d][part * 16];
        *(uint4*)(v_out + ((int64_t)bh * D + d) * Lp + k0 + part * 16) = val;
    }
}

// ---- MXFP4 -------------------------------------------------------------------
// mu * H per (b, h) in fp32 (channel-ascending sums), so that the rotated
// smoothed key is rot(K) - rot(mu).
__global__ void k_mu_rot(const float* mu, const uint16_t* hadamard_bf16, float* mu_rot) {
    constexpr int D = 128;
    const int bh = blockIdx.x, j = threadIdx.x;
    float s = 0.0f;
    for (int d = 0; d < D; ++d)
        s = s + mu[(int64_t)bh * D + d] * bf16_bits_to_f32(hadamard_bf16[d * D + j]);
    mu_rot[(int64_t)bh * D + j] = s;
}

__global__ void k_hadamard_build(int R, uint16_t* hb, uint16_t* hf) {
    const int i = blockIdx.x, j = threadIdx.x;
    const bool neg = __builtin_popcount((unsigned)(i & j)) & 1;
    hb[i * R + j] = neg ? 0xBF80 : 0x3F80;   // bf16 -1 / +1
    hf[i * R + j] = neg ? 0xBC00 : 0x3C00;   // fp16 -1 / +1
}

// One block = 4 waves x 32 tokens of one (b, h); blockIdx.x < nqb are Q blocks.
// Rotation Y^T = H X^T on bf16/fp16 MFMA (H's +-1 entries and the half-precision
// inputs are exact, accumulation in fp32), then times 1/sqrt(128).  Each lane
// ends with token (l % 32) and channels 32 cb + 8 i + 4 (l / 32) + j, so one
// MX block's amax needs a single cross-lane step and channel pairs (2t, 2t+1)
// sit in the same lane for nibble packing.
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(
    HalfView q, HalfView k, int H, int Lq, int Lk, int nqb, const float* mu,
    const uint16_t* hmat_bf16, const uint16_t* hmat_f16, float inv_sqrt_r, const float* mu_rot,
    uint8_t* q_out, uint8_t* q_e8, uint8_t* k_out, uint8_t* k_e8) {
    constexpr int D = 128;
    const bool isq = (int)blockIdx.x < nqb;
    const int blk = isq ? blockIdx.x : blockIdx.x - nqb;
    const int L = isq ? Lq : Lk;
    const int Lp = pad128(L);
    const HalfView& src = isq ? q : k;
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int token = blk * 128 + wave * 32 + col;
    const bool valid = token < L;
    const bool rotate = hmat_bf16 != nullptr;

    __shared__ uint16_t hs[D * D];   // 32 KB: the Hadamard matrix for this block
    if (rotate) {
        const uint16_t* hm = src.bf16 ? hmat_bf16 : hmat_f16;
        for (int c = threadIdx.x; c < D * D / 8; c += kThreads)
            *(uint4*)&hs[c * 8] = *(const uint4*)&hm[c * 8];
        __syncthreads();
    }

    float y[4][16];   // [cb][e]: channel 32 cb + 8 (e / 4) + 4 half + (e % 4)
    if (rotate) {
        // B operand: this lane's token, channels 16 kc + 8 half + 0..7
        uint4 xb[8];
        const uint16_t* row = (const uint16_t*)src.ptr + (int64_t)b * src.sB +
                              (int64_t)(valid ? token : 0) * src.sL + (int64_t)h * src.sH;
#pragma unroll
        for (int kc = 0; kc < 8; ++kc)
            xb[kc] = valid ? *(const uint4*)(row + 16 * kc + 8 * half) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            v16f acc = {0};
#pragma unroll
            for (int kc = 0; kc < 8; ++kc) {
                const uint4 ha = *(const uint4*)&hs[(32 * cb + col) * D + 16 * kc + 8 * half];
                if (src.bf16)
                    acc = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ha),
                                             __builtin_bit_cast(bf16x8, xb[kc]), acc);
                else
                    acc = mfma_f16_32x32x16(__builtin_bit_cast(f16x8, ha),
                                            __builtin_bit_cast(f16x8, xb[kc]), acc);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ch = 32 * cb + 8 * (e / 4) + 4 * half + (e % 4);
                float t = acc[e];
                if (!isq && mu_rot) t = t - mu_rot[(int64_t)bh * D + ch];
                y[cb][e] = valid ? t * inv_sqrt_r : 0.0f;
            }
        }
    } else {
        const uint16_t* row = (const uint16_t*)src.ptr + (int64_t)b * src.sB +
                              (int64_t)(valid ? token : 0) * src.sL + (int64_t)h * src.sH;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * cb + 8 * i + 4 * half;
                uint2 u = valid ? *(const uint2*)(row + ch0) : make_uint2(0, 0);
                uint32_t w[2] = {u.x, u.y};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t bits = (w[j / 2] >> (16 * (j % 2))) & 0xFFFF;
                    float t = src.bf16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
                    if (!isq && mu) t = t - mu[(int64_t)bh * D + ch0 + j];
                    y[cb][4 * i + j] = valid ? t : 0.0f;
                }
            }
    }

    uint8_t* out = isq ? q_out : k_out;
    uint8_t* oe = isq ? q_e8 : k_e8;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(y[cb][e]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int ex = mx_exponent(amax);
        if (half == 0 && token < Lp) oe[((int64_t)bh * Lp + token) * (D / 32) + cb] = (uint8_t)(ex + 127);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t n[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) n[j] = e2m1_rne(__builtin_ldexpf(y[cb][4 * i + j], -ex));
            const uint16_t packed = (uint16_t)(n[0] | (n[1] << 4) | (n[2] << 8) | (n[3] << 12));
            if (token < Lp)
                *(uint16_t*)(out + ((int64_t)bh * Lp + token) * (D / 2) + 16 * cb + 4 * i + 2 * half) =
                    packed;
        }
    }
}

}  // namespace

hipError_t launch_k_mean(const HalfView& k, int B, int H, int L, int D, double* partial,
                         float* mu, hipStream_t stream) {
    const int nchunk = mean_chunks(L);
    dim3 grid(nchunk, B * H);
    if (D == 128) {
        k_mean_partial<128><<<grid, kThreads, 0, stream>>>(k, H, L, nchunk, partial);
        k_mean_final<128><<<B * H, 128, 0, stream>>>(partial, nchunk, L, mu);
    } else {
        k_mean_partial<64><<<grid, kThreads, 0, stream>>>(k, H, L, nchunk, partial);
        k_mean_final<64><<<B * H, 64, 0, stream>>>(partial, nchunk, L, mu);
    }
    return hipGetLastError();
}

hipError_t launch_quant_qk_int8(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                int Lk, int D, int q_block, int k_block, const float* mu,
                                int8_t* q_out, float* q_scale, int8_t* k_out, float* k_scale,
                                hipStream_t stream) {
    const int nqb = pad128(Lq) / q_block, nkb = pad128(Lk) / k_block;
    dim3 grid(nqb + nkb, B * H);
    if (D == 128)
        k_quant_int8<128><<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, q_block, k_block, nqb, mu,
                                                         q_out, q_scale, k_out, k_scale);
    else
        k_quant_int8<64><<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, q_block, k_block, nqb, mu,
                                                        q_out, q_scale, k_out, k_scale);
    return hipGetLastError();
}

hipError_t launch_quant_v(const HalfView& v, int B, int H, int Lk, int D, uint32_t* amax_ws,
                          uint8_t* v_out, float* v_scale, hipStream_t stream) {
    const int64_t n = (int64_t)B * H * D;
    k_fill_u32<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(amax_ws, n, 0u);
    dim3 g1(mean_chunks(Lk), B * H), g2(pad128(Lk) / 64, B * H);
    if (D == 128) {
        k_v_amax<128><<<g1, kThreads, 0, stream>>>(v, H, Lk, amax_ws);
        k_v_quant<128><<<g2, kThreads, 0, stream>>>(v, H, Lk, amax_ws, v_out, v_scale);
    } else {
        k_v_amax<64><<<g1, kThreads, 0, stream>>>(v, H, Lk, amax_ws);
        k_v_quant<64><<<g2, kThreads, 0, stream>>>(v, H, Lk, amax_ws, v_out, v_scale);
    }
    return hipGetLastError();
}

hipError_t launch_quant_qk_mxfp4(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                 int Lk, int D, const float* mu, const void* hadamard_bf16,
                                 const void* hadamard_f16, float inv_sqrt_r, float* mu_rot_ws,
                                 uint8_t* q_out, uint8_t* q_e8, uint8_t* k_out, uint8_t* k_e8,
                                 hipStream_t stream) {
    (void)D;
    const float* mrot = nullptr;
    if (hadamard_bf16 && mu) {
        k_mu_rot<<<B * H, 128, 0, stream>>>(mu, (const uint16_t*)hadamard_bf16, mu_rot_ws);
        mrot = mu_rot_ws;
    }
    const int nqb = pad128(Lq) / 128, nkb = pad128(Lk) / 128;
    dim3 grid(nqb + nkb, B * H);
    k_quant_mxfp4<<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, nqb, mu,
                                                 (const uint16_t*)hadamard_bf16,
                                                 (const uint16_t*)hadamard_f16, inv_sqrt_r, mrot,
                                                 q_out, q_e8, k_out, k_e8);
    return hipGetLastError();
}

hipError_t launch_hadamard_build(int R, void* bf16_mat, void* f16_mat, hipStream_t stream) {
    k_hadamard_build<<<R, R, 0, stream>>>(R, (uint16_t*)bf16_mat, (uint16_t*)f16_mat);
    return hipGetLastError();
}

}  // namespace sage

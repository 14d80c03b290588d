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
// Grids put the head index fastest (blockIdx.x), so blocks launched together
// read adjacent pieces of the same token rows ([B, L, H, D]: a token's heads
// are contiguous) instead of rows one head-stride apart.
//
// Partial binary64 channel sums over chunks of kMeanChunk tokens; fixed
// summation order (per thread ascending rows, then ascending row groups), so
// the result is deterministic.
template <int D>
__global__ __launch_bounds__(kThreads) void k_mean_partial(HalfView k, int H, int L, int nchunk,
                                                           double* partial) {
    using G = Rows<D>;
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int lo = chunk * kMeanChunk, hi = min(L, lo + kMeanChunk);
    for (int l = lo + r0; l < hi; l += G::kRowsPerPass) {
        float x[8];
        load8(k, b, l, h, c8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
    }
    __shared__ double sm[kThreads][8 + 1];
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
// One block per (b*h, 128 token rows), Q blocks first, then K blocks; a Q
// block is one q_block (128 rows), a K block holds 128 / k_block k_blocks.  A
// thread owns 16 channels [16 c16, +16) of rows r0 + kRowsPass p: its loads
// and its code stores are 16-byte accesses.  Per quantization block: amax over
// the valid rows (K: of fp32(K - mu)), scale = amax / 127,
// codes = clamp(rne(x * (127 / amax)), -127, 127); padded rows get code 0.
// K blocks first finish the channel mean from the binary64 partial sums
// (summed in chunk order, divided by L in binary64, rounded to fp32); the
// first K block of each head also writes it out.
template <int D>
struct Rows16 {
    static constexpr int kLanesPerRow = D / 16;
    static constexpr int kRowsPass = kThreads / kLanesPerRow;   // 32 (D 128) or 64 (D 64)
    static constexpr int kPasses = 128 / kRowsPass;              // 4 or 2
};

__device__ __forceinline__ void unpack8(const uint4& u, bool bf16, float out[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16 ? bf16_bits_to_f32(w[i] & 0xFFFF) : f16_bits_to_f32(w[i] & 0xFFFF);
        out[2 * i + 1] = bf16 ? bf16_bits_to_f32(w[i] >> 16) : f16_bits_to_f32(w[i] >> 16);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_quant_int8(HalfView q, HalfView k, int H, int Lq,
                                                         int Lk, int k_block, int nqb,
                                                         const double* mean_partial, int nchunk,
                                                         float* mu_out, int8_t* q_out,
                                                         float* q_scale, int8_t* k_out,
                                                         float* k_scale) {
    using G = Rows16<D>;
    const bool isq = (int)blockIdx.y < nqb;
    const int blk = isq ? blockIdx.y : blockIdx.y - nqb;   // 128-row block
    const int L = isq ? Lq : Lk;
    const int Lp = pad128(L);
    const HalfView& src = isq ? q : k;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int c16 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int row0 = blk * 128;

    // all row loads first, unconditional: rows past L read the last row and
    // are replaced by zeros afterwards
    uint4 raw[G::kPasses][2];
    {
        const uint16_t* base = (const uint16_t*)src.ptr + (int64_t)b * src.sB + (int64_t)h * src.sH + 16 * c16;
#pragma unroll
        for (int p = 0; p < G::kPasses; ++p) {
            const uint16_t* ptr = base + (int64_t)min(row0 + p * G::kRowsPass + r0, L - 1) * src.sL;
            raw[p][0] = *(const uint4*)ptr;
            raw[p][1] = *(const uint4*)(ptr + 8);
        }
#pragma unroll
        for (int p = 0; p < G::kPasses; ++p)
            if (row0 + p * G::kRowsPass + r0 >= L) raw[p][0] = raw[p][1] = make_uint4(0, 0, 0, 0);
    }

    __shared__ float mu_s[D];
    __shared__ float red[kThreads / 64][2];
    const bool smooth = !isq && mean_partial != nullptr;
    if (smooth) {
        if (threadIdx.x < D) {
            const int d = threadIdx.x;
            double acc = 0.0;
            for (int c = 0; c < nchunk; ++c) acc += mean_partial[((int64_t)bh * nchunk + c) * D + d];
            const float m = L > 0 ? (float)(acc / (double)L) : 0.0f;
            mu_s[d] = m;
            if (blk == 0 && mu_out) mu_out[(int64_t)bh * D + d] = m;
        }
        __syncthreads();
    }
    float mu16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mu16[i] = smooth ? mu_s[16 * c16 + i] : 0.0f;

    // x = fp32(value - mu); amax per quantization block.  Passes [0, kPasses/2)
    // hold rows 0..63 of the 128, the rest rows 64..127.
    auto xval = [&](int p, float x[16]) {
        unpack8(raw[p][0], src.bf16, x);
        unpack8(raw[p][1], src.bf16, x + 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = x[i] - mu16[i];
    };
    float am[2] = {0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
        const int row = row0 + p * G::kRowsPass + r0;
        float x[16];
        xval(p, x);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
        if (row < L) am[p < G::kPasses / 2 ? 0 : 1] = fmaxf(am[p < G::kPasses / 2 ? 0 : 1], m);
    }
    am[0] = wave_max(am[0]);
    am[1] = wave_max(am[1]);
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x / 64][0] = am[0];
        red[threadIdx.x / 64][1] = am[1];
    }
    // keep only the raw rows live across the barrier (the conversion is redone
    // below rather than holding the converted values)
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            asm("" : "+v"(raw[p][j].x), "+v"(raw[p][j].y), "+v"(raw[p][j].z), "+v"(raw[p][j].w));
    __syncthreads();
    float bm[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        bm[j] = red[0][j];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) bm[j] = fmaxf(bm[j], red[w][j]);
    }
    // quantization blocks: Q one of 128 rows; K 128 / k_block of k_block rows
    const bool halves = !isq && k_block == 64;
    const float amax_all = fmaxf(bm[0], bm[1]);
    int8_t* out = isq ? q_out : k_out;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
        const int row = row0 + p * G::kRowsPass + r0;
        const float a = halves ? bm[p < G::kPasses / 2 ? 0 : 1] : amax_all;
        const float inv = a > 0.0f ? 127.0f / a : 0.0f;
        float x[16];
        xval(p, x);
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float r = __builtin_rintf(x[i] * inv);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            if (row >= L) r = 0.0f;
            w[i / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i % 4));
        }
        if (row < Lp)
            *(uint4*)(out + ((int64_t)bh * Lp + row) * D + 16 * c16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (threadIdx.x == 0) {
        if (isq) {
            q_scale[(int64_t)bh * (Lp / 128) + blk] = amax_all > 0.0f ? amax_all / 127.0f : 0.0f;
        } else if (halves) {
            k_scale[(int64_t)bh * (Lp / 64) + 2 * blk] = bm[0] > 0.0f ? bm[0] / 127.0f : 0.0f;
            k_scale[(int64_t)bh * (Lp / 64) + 2 * blk + 1] = bm[1] > 0.0f ? bm[1] / 127.0f : 0.0f;
        } else {
            k_scale[(int64_t)bh * (Lp / 128) + blk] = amax_all > 0.0f ? amax_all / 127.0f : 0.0f;
        }
    }
}

// ---- V: per-channel amax, then e4m3 codes written transposed ----------------
// Pass 1: per chunk of kMeanChunk tokens, the channel amax of |v| (no atomics:
// one partial row per chunk); head-fastest grid like the K mean.
template <int D>
__global__ __launch_bounds__(kThreads) void k_v_amax(HalfView v, int H, int L, int nchunk,
                                                     float* partial) {
    using G = Rows<D>;
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int lo = chunk * kMeanChunk, hi = min(L, lo + kMeanChunk);
    for (int l = lo + r0; l < hi; l += G::kRowsPerPass) {
        float x[8];
        load8(v, b, l, h, c8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(x[i]));
    }
    __shared__ float sm[kThreads][8 + 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = m[i];
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float r = 0.0f;
        for (int g = 0; g < G::kRowsPerPass; ++g) r = fmaxf(r, sm[g * G::kLanesPerRow + d / 8][d % 8]);
        partial[((int64_t)bh * nchunk + chunk) * D + d] = r;
    }
}

// Pass 2: one block per 128 keys of one (b, h).  amax[d] = max over the chunk
// partials; codes = e4m3(v * (448 / amax[d])), scale = amax / 448 (written by
// the first block of each head).  A thread converts 4 keys x 8 channels and
// packs, per channel, the 4 keys' codes into one dword, stored into an LDS
// tile [D][128 keys] whose 16-byte chunks are XOR-swizzled by row; the tile is
// then written out as 128-byte V^T rows with 16-byte stores.
template <int D>
__global__ __launch_bounds__(kThreads) void k_v_quant(HalfView v, int H, int L, int nchunk,
                                                      const float* partial, uint8_t* v_out,
                                                      float* v_scale) {
    constexpr int kKeys = 128;
    constexpr int kGroups = D / 8;                         // 8-channel groups (16 or 8)
    constexpr int kKeyGroups = kThreads / kGroups;         // 4-key groups per pass (16 or 32)
    constexpr int kPasses = kKeys / (4 * kKeyGroups);      // 2 or 1
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int k0 = blockIdx.y * kKeys;
    const int Lp = pad128(L);
    const int c8 = threadIdx.x % kGroups, kg0 = threadIdx.x / kGroups;

    // row loads first: keys k0 + 4 kg + j, channels [8 c8, +8)
    uint4 raw[kPasses][4];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * (p * kKeyGroups + kg0) + j;
            raw[p][j] = key < L ? *(const uint4*)((const uint16_t*)v.ptr + (int64_t)b * v.sB +
                                                  (int64_t)key * v.sL + (int64_t)h * v.sH + 8 * c8)
                                : make_uint4(0, 0, 0, 0);
        }

    __shared__ float inv_s[D];
    __shared__ __attribute__((aligned(16))) uint32_t tile[D * kKeys / 4];
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float a = 0.0f;
        for (int c = 0; c < nchunk; ++c) a = fmaxf(a, partial[((int64_t)bh * nchunk + c) * D + d]);
        inv_s[d] = a > 0.0f ? kFp8Max / a : 0.0f;
        if (blockIdx.y == 0) v_scale[(int64_t)bh * D + d] = a / kFp8Max;
    }
    __syncthreads();
    float inv8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) inv8[i] = inv_s[8 * c8 + i];
    // tile word (d, kg): row d holds kKeys / 16 chunks of 4 words; chunk
    // kg / 4 is stored at (kg / 4) ^ ((d >> 3) & 7)
    auto word = [](int d, int kg) { return d * (kKeys / 4) + 4 * ((kg >> 2) ^ ((d >> 3) & 7)) + (kg & 3); };
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int kg = p * kKeyGroups + kg0;
        float x[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(raw[p][j], v.bf16, x[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t c = cvt_pk_fp8<false>(x[0][i] * inv8[i], x[1][i] * inv8[i], 0);
            c = cvt_pk_fp8<true>(x[2][i] * inv8[i], x[3][i] * inv8[i], c);
            tile[word(8 * c8 + i, kg)] = c;
        }
    }
    __syncthreads();
    // out row d: 8 chunks of 16 keys; lanes 8 t .. 8 t + 7 write one row
    for (int c = threadIdx.x; c < D * (kKeys / 16); c += kThreads) {
        const int d = c / (kKeys / 16), j = c % (kKeys / 16);
        const uint4 val = *(const uint4*)&tile[word(d, 4 * j)];
        *(uint4*)(v_out + ((int64_t)bh * D + d) * Lp + k0 + 16 * j) = val;
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

hipError_t launch_k_mean_partial(const HalfView& k, int B, int H, int L, int D, double* partial,
                                 hipStream_t stream) {
    const int nchunk = mean_chunks(L);
    dim3 grid(B * H, nchunk);
    if (D == 128)
        k_mean_partial<128><<<grid, kThreads, 0, stream>>>(k, H, L, nchunk, partial);
    else
        k_mean_partial<64><<<grid, kThreads, 0, stream>>>(k, H, L, nchunk, partial);
    return hipGetLastError();
}

hipError_t launch_k_mean_final(const double* partial, int B, int H, int L, int D, float* mu,
                               hipStream_t stream) {
    const int nchunk = mean_chunks(L);
    if (D == 128)
        k_mean_final<128><<<B * H, 128, 0, stream>>>(partial, nchunk, L, mu);
    else
        k_mean_final<64><<<B * H, 64, 0, stream>>>(partial, nchunk, L, mu);
    return hipGetLastError();
}

hipError_t launch_quant_qk_int8(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                int Lk, int D, int k_block, const double* mean_partial,
                                float* mu_out, int8_t* q_out, float* q_scale, int8_t* k_out,
                                float* k_scale, hipStream_t stream) {
    const int nqb = pad128(Lq) / 128, nkb = pad128(Lk) / 128;
    const int nchunk = mean_chunks(Lk);
    dim3 grid(B * H, nqb + nkb);
    if (D == 128)
        k_quant_int8<128><<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, k_block, nqb, mean_partial,
                                                             nchunk, mu_out, q_out, q_scale, k_out, k_scale);
    else
        k_quant_int8<64><<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, k_block, nqb, mean_partial,
                                                            nchunk, mu_out, q_out, q_scale, k_out, k_scale);
    return hipGetLastError();
}

hipError_t launch_quant_v(const HalfView& v, int B, int H, int Lk, int D, float* amax_partial,
                          uint8_t* v_out, float* v_scale, hipStream_t stream) {
    const int nchunk = mean_chunks(Lk);
    dim3 g1(B * H, nchunk), g2(B * H, pad128(Lk) / 128);
    if (D == 128) {
        k_v_amax<128><<<g1, kThreads, 0, stream>>>(v, H, Lk, nchunk, amax_partial);
        k_v_quant<128><<<g2, kThreads, 0, stream>>>(v, H, Lk, nchunk, amax_partial, v_out, v_scale);
    } else {
        k_v_amax<64><<<g1, kThreads, 0, stream>>>(v, H, Lk, nchunk, amax_partial);
        k_v_quant<64><<<g2, kThreads, 0, stream>>>(v, H, Lk, nchunk, amax_partial, v_out, v_scale);
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

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

#include <atomic>
#include <chrono>
#include <map>
#include <mutex>
#include <utility>

#pragma clang fp contract(off)

namespace sage {
namespace {

constexpr int kThreads = 256;

template <int D>
struct Rows {
    static constexpr int kLanesPerRow = D / 8;            // 16-byte chunks per row
    static constexpr int kRowsPerPass = kThreads / kLanesPerRow;
};

template <bool BF16>
__device__ __forceinline__ void unpack8t(const uint4& u, float out[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = BF16 ? bf16_bits_to_f32(w[i] & 0xFFFF) : f16_bits_to_f32(w[i] & 0xFFFF);
        out[2 * i + 1] = BF16 ? bf16_bits_to_f32(w[i] >> 16) : f16_bits_to_f32(w[i] >> 16);
    }
}

// The rows of one kMeanChunk-token chunk [lo, lo + kMeanChunk) that a thread
// of the chunk kernels reads: rows lo + r0 + kRowsPerPass i, channels
// [8 c8, +8), all loads issued before any is used (one memory round trip per
// chunk instead of one per row).  Rows at or past L (L >= 1) are read at row
// L - 1, in bounds, and must be skipped by the caller.
template <int D>
struct ChunkRows {
    static constexpr int kN = kMeanChunk / Rows<D>::kRowsPerPass;
    uint4 raw[kN];
    __device__ __forceinline__ void load(const HalfView& v, int b, int h, int L, int lo, int r0, int c8) {
        const uint16_t* base = (const uint16_t*)v.ptr + (int64_t)b * v.sB + (int64_t)h * v.sH + 8 * c8;
#pragma unroll
        for (int i = 0; i < kN; ++i)
            raw[i] = *(const uint4*)(base + (int64_t)min(lo + r0 + Rows<D>::kRowsPerPass * i, L - 1) * v.sL);
    }
};

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max_xor(v);
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
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void k_mean_partial(HalfView k, int H, int L, int nchunk,
                                                           double* partial) {
    using G = Rows<D>;
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int lo = chunk * kMeanChunk;
    ChunkRows<D> rows;
    rows.load(k, b, h, L, lo, r0, c8);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < ChunkRows<D>::kN; ++j) {
        if (lo + r0 + G::kRowsPerPass * j >= L) continue;
        float x[8];
        unpack8t<BF16>(rows.raw[j], x);
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

// Finish of one head's channel statistics: thread d folds channel d of the
// head's nchunk chunk partials in chunk order.  The loads go out a batch at a
// time (32 binary64 or 64 fp32 values, as many as fit in registers), all in
// flight together, ahead of the (ordered) folds: one at a time, the loop
// waited one memory latency per chunk (128 chunks: ~36 us).
template <typename T>
constexpr int kFinishBatch = sizeof(T) == 8 ? 32 : 64;

// mu = fp32(sum / L) in binary64, chunk order.  Written to mu (if any) and,
// as a binary64 value, over chunk 0's partial, where k_quant_int8 reads it.
template <int D>
__global__ void k_mean_final(double* partial, int nchunk, int L, float* mu) {
    const int bh = blockIdx.x, d = threadIdx.x;
    double* col = partial + (int64_t)bh * nchunk * D + d;
    double s = 0.0;
    for (int c0 = 0; c0 < nchunk; c0 += kFinishBatch<double>) {
        double v[kFinishBatch<double>];
#pragma unroll
        for (int u = 0; u < kFinishBatch<double>; ++u) v[u] = c0 + u < nchunk ? col[(int64_t)(c0 + u) * D] : 0.0;
#pragma unroll
        for (int u = 0; u < kFinishBatch<double>; ++u)
            if (c0 + u < nchunk) s += v[u];
    }
    const float m = L > 0 ? (float)(s / (double)L) : 0.0f;
    if (mu) mu[(int64_t)bh * D + d] = m;
    col[0] = (double)m;   // this thread has read every chunk of its own column above
}

// V: amax = max over the chunk partials (order-free), written over chunk 0's
// partial, where k_v_quant reads it, and scale = amax / 448.
template <int D>
__global__ void k_v_amax_final(float* partial, int nchunk, float* v_scale) {
    const int bh = blockIdx.x, d = threadIdx.x;
    float* col = partial + (int64_t)bh * nchunk * D + d;
    float a = 0.0f;
    for (int c0 = 0; c0 < nchunk; c0 += kFinishBatch<float>) {
        float v[kFinishBatch<float>];
#pragma unroll
        for (int u = 0; u < kFinishBatch<float>; ++u) v[u] = c0 + u < nchunk ? col[(int64_t)(c0 + u) * D] : 0.0f;
#pragma unroll
        for (int u = 0; u < kFinishBatch<float>; ++u) a = fmaxf(a, v[u]);
    }
    v_scale[(int64_t)bh * D + d] = a / kFp8Max;
    col[0] = a;
}

// ---- INT8 block quantization -------------------------------------------------
// One block per (b*h, 128 token rows), block index y: Q's row blocks, then
// K's (dispatched last-first, see below); a Q block is one q_block (128
// rows), a K block holds 128 / k_block k_blocks.  A thread owns 16 channels
// [16 c16, +16) of rows r0 + kRowsPass p: its loads and its code stores are
// 16-byte accesses.  Per quantization block: amax over the valid rows (K: of fp32(K - mu)), scale = amax / 127,
// codes = clamp(rne(x * (127 / amax)), -127, 127); padded rows get code 0.
// K blocks take the channel mean that k_mean_final left over chunk 0 of the
// binary64 partials (summed in chunk order, divided by L in binary64, rounded
// to fp32).
template <int D>
struct Rows16 {
    static constexpr int kLanesPerRow = D / 16;
    static constexpr int kRowsPass = kThreads / kLanesPerRow;   // 32 (D 128) or 64 (D 64)
    static constexpr int kPasses = 128 / kRowsPass;              // 4 or 2
};

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void k_quant_int8(HalfView q, HalfView k, int H, int Lq,
                                                         int Lk, int k_block, int nqb,
                                                         const double* mean_final, int nchunk,
                                                         int8_t* q_out, float* q_scale, int8_t* k_out,
                                                         float* k_scale) {
    using G = Rows16<D>;
    // Row blocks run last-first: the statistics pass before this one read the
    // tokens first-first, so its last ~256 MB (the size of the GPU's
    // memory-side cache) are still cached when this pass starts on them
    // (32760 tokens x 40 heads: quantize_qk step 176 -> 154 us; the same
    // order measured no gain for the MXFP4 quantizer, which is not bound by
    // its reads)
    const int yy = (int)gridDim.y - 1 - (int)blockIdx.y;
    const bool isq = yy < nqb;
    const int blk = isq ? yy : yy - nqb;   // 128-row block
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

    // the subtracted mean: K's (zeros without smoothing), zeros for Q; read
    // unconditionally (a read under the condition becomes a branch per read)
    __shared__ __attribute__((aligned(16))) float mu_s[D];
    __shared__ float red[kThreads / 64][2];
    const bool smooth = !isq && mean_final != nullptr;
    if (threadIdx.x < D) mu_s[threadIdx.x] = smooth ? (float)mean_final[(int64_t)bh * nchunk * D + threadIdx.x] : 0.0f;
    __syncthreads();
    float mu16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mu16[i] = mu_s[16 * c16 + i];

    // x = fp32(value - mu); amax per quantization block.  Passes [0, kPasses/2)
    // hold rows 0..63 of the 128, the rest rows 64..127.
    auto xval = [&](int p, float x[16]) {
        unpack8t<BF16>(raw[p][0], x);
        unpack8t<BF16>(raw[p][1], x + 8);
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
    am[0] = wave_max_xor(am[0]);
    am[1] = wave_max_xor(am[1]);
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
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void k_v_amax(HalfView v, int H, int L, int nchunk,
                                                     float* partial) {
    using G = Rows<D>;
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int lo = chunk * kMeanChunk;
    ChunkRows<D> rows;
    rows.load(v, b, h, L, lo, r0, c8);
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < ChunkRows<D>::kN; ++j) {
        if (lo + r0 + G::kRowsPerPass * j >= L) continue;
        float x[8];
        unpack8t<BF16>(rows.raw[j], x);
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

// Pass 2: one block per 128 keys of one (b, h).  amax[d] from
// k_v_amax_final (chunk 0 of the partials); codes = e4m3(v * (448 / amax[d])).  A thread converts 4 keys x 8 channels and
// packs, per channel, the 4 keys' codes into one dword, stored into an LDS
// tile [D][128 keys] whose 16-byte chunks are XOR-swizzled by row; the tile is
// then written out as 128-byte V^T rows with 16-byte stores.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void k_v_quant(HalfView v, int H, int L, int nchunk,
                                                      const float* partial, uint8_t* v_out) {
    constexpr int kKeys = 128;
    constexpr int kGroups = D / 8;                         // 8-channel groups (16 or 8)
    constexpr int kKeyGroups = kThreads / kGroups;         // 4-key groups per pass (16 or 32)
    constexpr int kPasses = kKeys / (4 * kKeyGroups);      // 2 or 1
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int k0 = ((int)gridDim.y - 1 - (int)blockIdx.y) * kKeys;   // last-first, as in k_quant_int8
    const int Lp = pad128(L);
    const int c8 = threadIdx.x % kGroups, kg0 = threadIdx.x / kGroups;

    // row loads first: keys k0 + 4 kg + j, channels [8 c8, +8); keys past L
    // read key L - 1 (in bounds, unconditional) and are zeroed afterwards
    uint4 raw[kPasses][4];
    const uint16_t* vbase = (const uint16_t*)v.ptr + (int64_t)b * v.sB + (int64_t)h * v.sH + 8 * c8;
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * (p * kKeyGroups + kg0) + j;
            raw[p][j] = *(const uint4*)(vbase + (int64_t)min(key, L - 1) * v.sL);
        }
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (k0 + 4 * (p * kKeyGroups + kg0) + j >= L) raw[p][j] = make_uint4(0, 0, 0, 0);

    __shared__ float inv_s[D];
    __shared__ __attribute__((aligned(16))) uint32_t tile[D * kKeys / 4];
    if (threadIdx.x < D) {
        const float a = partial[(int64_t)bh * nchunk * D + threadIdx.x];   // k_v_amax_final's result
        inv_s[threadIdx.x] = a > 0.0f ? kFp8Max / a : 0.0f;
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
        for (int j = 0; j < 4; ++j) unpack8t<BF16>(raw[p][j], x[j]);
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

// ---- single-read K and V quantizers -----------------------------------------
// When every block of the grid can be resident at once, K (and V) are read
// from HBM once instead of twice: a block holds one 256-token chunk of one head
// in registers, publishes that chunk's channel sums (K) or channel amax (V),
// waits for the other chunks of its head, finishes the statistic and
// quantizes the rows it holds.  The chunk results are the numbers the
// two-kernel path computes (k_mean_partial / k_v_amax: same chunks, same
// summation order), so both paths give identical outputs.  The host takes
// this path only when the whole grid fits on the device at once, so every
// block a head waits for is running; the wait is bounded regardless.

// Every value exchanged between blocks (chunk results, flags, epochs) is read
// and written with device-scope atomic accesses, which are coherent across
// the XCDs' L2 caches by themselves; a full release/acquire fence would
// instead write back and invalidate a whole L2 per block, which serializes
// (measured: ~250 us per kernel).  A writer waits for its stores to complete
// before its arrival is published.
template <typename T>
__device__ __forceinline__ void publish(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T fetch(const T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// op-fold of p[0], p[stride], ..., p[(n - 1) stride] in index order, sixteen
// loads in flight at a time (one round trip for a 4096-token head)
template <typename T, typename Op>
__device__ __forceinline__ T fold_published(const T* p, int64_t stride, int n, T acc, Op op) {
    constexpr int kBatch = 16;
    int c = 0;
    for (; c + kBatch <= n; c += kBatch) {
        T v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = fetch(p + (c + j) * stride);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) acc = op(acc, v[j]);
    }
    for (; c < n; ++c) acc = op(acc, fetch(p + c * stride));
    return acc;
}

// Meeting point of the chunks of one head, with no clearing launch.  Each
// block publishes, on its chunk's flag, the call's token once its chunk
// results are complete, and waits until every flag of the head holds it.
// The token mixes a number the host draws afresh for every launch with the
// head's epoch word e, which every block reads when it starts and chunk 0's
// block alone advances to e + 1 once its own wait is over.  Flags therefore
// never match across launches -- nor across replays of one captured launch,
// which share the host number but not the epoch -- and the workspace needs no
// initialization.  Separate flags rather than one counter, and one epoch
// writer rather than every block: device-scope writes to one address
// serialize (16 arrivals on one counter took ~12 us; 16 blocks storing the
// epoch cost ~3 us per launch).
//
// The wait is bounded in time.  If the other chunks do not all arrive -- the
// host checks that the grid fits on the device, but kernels of other streams
// may hold part of it -- the block withdraws its arrival (flag 0, never a
// token) and computes its head's statistic itself from the inputs, in the
// same order, so the result is the same, only slower.  A block that starts
// after chunk 0 advanced the epoch carries the next token, meets nobody, and
// withdraws.  So when a launch ends every flag of a head is 0 or the token of
// the epoch that launch started with, never the token the next one will wait
// for.
struct HeadSync {
    uint64_t* flags;      // [B*H, nchunk]
    uint64_t* epoch;      // [B*H]
    uint64_t nonce;       // drawn by the host for each launch
    int64_t wait_ticks;   // wall-clock ticks a block waits for its head
};

// splitmix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014)
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t head_token(const HeadSync& hs, uint64_t e) {
    const uint64_t t = mix64(hs.nonce ^ mix64(e));
    return t ? t : 1;
}

__device__ __forceinline__ void head_arrive(const HeadSync& hs, int bh, int chunk, int nchunk, uint64_t token) {
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this thread's published stores completed
    __syncthreads();
    if (threadIdx.x == 0) publish(hs.flags + (int64_t)bh * nchunk + chunk, token);
}

// true when every chunk of the head arrived in time
__device__ __forceinline__ bool head_wait(const HeadSync& hs, int bh, int chunk, int nchunk, uint64_t e,
                                          uint64_t token, int* met_lds) {
    if (threadIdx.x < 64) {   // wave 0 polls, one flag per lane and pass
        const uint64_t* f = hs.flags + (int64_t)bh * nchunk;
        const int64_t t0 = wall_clock64();
        int met = 0;
        for (int i = 1;; ++i) {
            int missing = 0;
            for (int c = threadIdx.x; c < nchunk; c += 64) missing |= fetch(f + c) != token;
            if (!__any(missing)) {
                met = 1;
                break;
            }
            // the clock is read every 16 polls only (a read delays the next
            // poll about as much as a poll takes); lane 0's reading decides,
            // so the wave leaves the loop as one
            if (hs.wait_ticks == 0 ||
                ((i & 15) == 0 && __builtin_amdgcn_readfirstlane((int)(wall_clock64() - t0 > hs.wait_ticks))))
                break;
            __builtin_amdgcn_s_sleep(4);
        }
        if (threadIdx.x == 0) {   // the thread that published the arrival
            *met_lds = met;
            if (!met) publish(hs.flags + (int64_t)bh * nchunk + chunk, (uint64_t)0);
            if (chunk == 0) publish(hs.epoch + bh, e + 1);
        }
    }
    __syncthreads();
    return *met_lds != 0;
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// One 128-row INT8 block of Q: amax over the valid rows, scale amax / 127,
// codes clamp(rne(x * (127 / amax)), -127, 127), padded rows code 0 (the
// arithmetic of k_quant_int8's Q blocks).  A thread owns channels [8 c8, +8)
// of rows r0 + kRowsPerPass p; rows are read through a buffer resource that
// ends with row L - 1 (rows past L read as zeros).  red: LDS [4] floats.
template <int D, bool BF16>
__device__ __forceinline__ void quant_q_block(const HalfView& q, int b, int h, int bh, int blk, int L,
                                              int8_t* q_out, float* q_scale, float* red) {
    using G = Rows<D>;
    constexpr int kPasses = 128 / G::kRowsPerPass;   // 8 (D 128) or 4 (D 64)
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int row0 = blk * 128, Lp = pad128(L);
    uint4 raw[kPasses];
    {
        const uint16_t* head = (const uint16_t*)q.ptr + (int64_t)b * q.sB + (int64_t)h * q.sH;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(head, ((int64_t)(L - 1) * q.sL + D) * 2);
        const int off = (int)(((int64_t)(row0 + r0) * q.sL + 8 * c8) * 2);
        const int step = (int)(G::kRowsPerPass * q.sL * 2);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) raw[p] = load16(rs, off + p * step);
    }
    float am = 0.0f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float x[8];
        unpack8t<BF16>(raw[p], x);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
        if (row0 + p * G::kRowsPerPass + r0 < L) am = fmaxf(am, m);
    }
    am = wave_max_xor(am);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = am;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) asm("" : "+v"(raw[p].x), "+v"(raw[p].y), "+v"(raw[p].z), "+v"(raw[p].w));
    __syncthreads();
    float amax = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, red[w]);
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    const __amdgpu_buffer_rsrc_t os = make_rsrc(q_out + (int64_t)bh * Lp * D, (int64_t)Lp * D);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int row = row0 + p * G::kRowsPerPass + r0;
        float x[8];
        unpack8t<BF16>(raw[p], x);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = __builtin_rintf(x[i] * inv);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            if (row >= L) r = 0.0f;
            w[i / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i % 4));
        }
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned,
                                                                 make_uint2(w[0], w[1])),
                                              os, row * D + 8 * c8, 0, 0);
    }
    if (threadIdx.x == 0) q_scale[(int64_t)bh * (Lp / 128) + blk] = amax > 0.0f ? amax / 127.0f : 0.0f;
    __syncthreads();   // red is reused
}

// INT8 Q and smoothed K in one launch.  Grid (B*H, chunks of 256 K tokens);
// block (bh, c) holds K chunk c of head bh and also quantizes the Q blocks
// c, c + nchunk, ... of that head between publishing its chunk sums and
// waiting for the other chunks.  For K a thread owns channels [8 c8, +8) of
// rows r0 + kRowsPerPass p.  Quantization blocks (k_block 64 or 128 rows) lie
// inside a chunk; rows past L get code 0, rows past pad128(L) are not written.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_quant_qk_fused(
    HalfView q, HalfView k, int H, int Lq, int L, int k_block, int nchunk, double* partial, HeadSync hs,
    float* mu_out, int8_t* q_out, float* q_scale, int8_t* k_out, float* k_scale) {
    using G = Rows<D>;
    constexpr int kPasses = kMeanChunk / G::kRowsPerPass;   // 16 (D 128) or 8 (D 64)
    constexpr int kPer64 = 64 / G::kRowsPerPass;            // passes per 64-row block
    constexpr int kB64 = kMeanChunk / 64;                   // 64-row blocks per chunk
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int c8 = threadIdx.x % G::kLanesPerRow, r0 = threadIdx.x / G::kLanesPerRow;
    const int row0 = chunk * kMeanChunk;
    const int Lp = pad128(L);
    const uint64_t e = fetch(hs.epoch + bh);
    const uint64_t token = head_token(hs, e);

    const uint16_t* khead = (const uint16_t*)k.ptr + (int64_t)b * k.sB + (int64_t)h * k.sH;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(khead, ((int64_t)(L - 1) * k.sL + D) * 2);
    // rows r0 + kRowsPerPass p of chunk c, channels [8 c8, +8)
    auto row_off = [&](int c, int p) {
        return (int)(((int64_t)(c * kMeanChunk + p * G::kRowsPerPass + r0) * k.sL + 8 * c8) * 2);
    };
    uint4 raw[kPasses];
    auto load_chunk = [&]() {
        // four passes in flight at a time: with every block of the grid
        // loading at once, unthrottled requests left some blocks waiting ~3x
        // longer than the median for their rows
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            raw[p] = load16(krs, row_off(chunk, p));
            if (p % 4 == 3 && p + 1 < kPasses) __builtin_amdgcn_s_waitcnt(0x3f70);
        }
    };
    load_chunk();

    // chunk channel sums in binary64: rows ascending per thread, then the
    // threads of a channel in row order (zero rows add nothing)
    __shared__ double sm[kThreads][8 + 1];
    {
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            float x[8];
            unpack8t<BF16>(raw[p], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = acc[i];
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        double s = 0.0;
        for (int r = 0; r < G::kRowsPerPass; ++r) s += sm[r * G::kLanesPerRow + d / 8][d % 8];
        publish(&partial[((int64_t)bh * nchunk + chunk) * D + d], s);
    }
    // conversions are redone after the wait rather than kept live across it
#pragma unroll
    for (int p = 0; p < kPasses; ++p) asm("" : "+v"(raw[p].x), "+v"(raw[p].y), "+v"(raw[p].z), "+v"(raw[p].w));
    head_arrive(hs, bh, chunk, nchunk, token);

    __shared__ float red[kThreads / 64][kB64];
    const int nqb = pad128(Lq) / 128;
    for (int qb = chunk; qb < nqb; qb += nchunk)
        quant_q_block<D, BF16>(q, b, h, bh, qb, Lq, q_out, q_scale, &red[0][0]);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) asm("" : "+v"(raw[p].x), "+v"(raw[p].y), "+v"(raw[p].z), "+v"(raw[p].w));
    __shared__ int met_s;
    const bool met = head_wait(hs, bh, chunk, nchunk, e, token, &met_s);

    __shared__ float mu_s[D];
    double acc = 0.0;   // channel sum over the head (thread d < D)
    if (met) {
        if (threadIdx.x < D)
            acc = fold_published(partial + (int64_t)bh * nchunk * D + threadIdx.x, (int64_t)D, nchunk, 0.0,
                                 [](double x, double y) { return x + y; });
    } else {
        // every chunk's sums from the inputs, in the order of the published ones
        for (int c = 0; c < nchunk; ++c) {
            double cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
            for (int p = 0; p < kPasses; ++p) {
                float x[8];
                unpack8t<BF16>(load16(krs, row_off(c, p)), x);
#pragma unroll
                for (int i = 0; i < 8; ++i) cs[i] += (double)x[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = cs[i];
            __syncthreads();
            if (threadIdx.x < D) {
                const int d = threadIdx.x;
                double s = 0.0;
                for (int r = 0; r < G::kRowsPerPass; ++r) s += sm[r * G::kLanesPerRow + d / 8][d % 8];
                acc += s;
            }
            __syncthreads();
        }
    }
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        const float m = L > 0 ? (float)(acc / (double)L) : 0.0f;
        mu_s[d] = m;
        if (chunk == 0 && mu_out) mu_out[(int64_t)bh * D + d] = m;
    }
    __syncthreads();
    float mu8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mu8[i] = mu_s[8 * c8 + i];

    // amax of fp32(K - mu) per 64-row block (a 128-row block is two of them)
    float am[kB64];
#pragma unroll
    for (int j = 0; j < kB64; ++j) am[j] = 0.0f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float x[8];
        unpack8t<BF16>(raw[p], x);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i] - mu8[i]));
        if (row0 + p * G::kRowsPerPass + r0 < L) am[p / kPer64] = fmaxf(am[p / kPer64], m);
    }
#pragma unroll
    for (int j = 0; j < kB64; ++j) am[j] = wave_max_xor(am[j]);
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < kB64; ++j) red[threadIdx.x / 64][j] = am[j];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) asm("" : "+v"(raw[p].x), "+v"(raw[p].y), "+v"(raw[p].z), "+v"(raw[p].w));
    __syncthreads();
    float ba[kB64];   // amax of the quantization block holding 64-row block j
    {
        float bm[kB64];
#pragma unroll
        for (int j = 0; j < kB64; ++j) {
            bm[j] = red[0][j];
#pragma unroll
            for (int w = 1; w < kThreads / 64; ++w) bm[j] = fmaxf(bm[j], red[w][j]);
        }
#pragma unroll
        for (int j = 0; j < kB64; ++j) ba[j] = k_block == 64 ? bm[j] : fmaxf(bm[j & ~1], bm[j | 1]);
    }

    const __amdgpu_buffer_rsrc_t os = make_rsrc(k_out + (int64_t)bh * Lp * D, (int64_t)Lp * D);
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int row = row0 + p * G::kRowsPerPass + r0;
        const float a = ba[p / kPer64];
        const float inv = a > 0.0f ? 127.0f / a : 0.0f;
        float x[8];
        unpack8t<BF16>(raw[p], x);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = __builtin_rintf((x[i] - mu8[i]) * inv);
            r = fminf(127.0f, fmaxf(-127.0f, r));
            if (row >= L) r = 0.0f;
            w[i / 4] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (i % 4));
        }
        // rows past pad128(L) fall outside the resource and are dropped
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned,
                                                                 make_uint2(w[0], w[1])),
                                              os, row * D + 8 * c8, 0, 0);
    }
    if (threadIdx.x == 0) {
        const int nsc = Lp / k_block;
#pragma unroll
        for (int j = 0; j < kB64; ++j) {
            if (k_block == 128 && (j & 1)) continue;
            const int idx = (row0 + 64 * j) / k_block;
            if (idx < nsc) k_scale[(int64_t)bh * nsc + idx] = ba[j] > 0.0f ? ba[j] / 127.0f : 0.0f;
        }
    }
}

// V: one block per 256 keys of one head; chunk channel amax, head barrier,
// amax over the chunks, then e4m3 codes transposed through an LDS tile
// [D][256 keys] (as in k_v_quant: per channel, 4 keys' codes packed per
// dword; 16-byte chunks XOR-swizzled by row) written as V^T rows.
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_quant_v_fused(
    HalfView v, int H, int L, int nchunk, float* partial, HeadSync hs, uint8_t* v_out, float* v_scale) {
    constexpr int kKeys = kMeanChunk;                      // 256
    constexpr int kGroups = D / 8;                         // 8-channel groups
    constexpr int kKeyGroups = kThreads / kGroups;         // 4-key groups per pass (16 or 32)
    constexpr int kPasses = kKeys / (4 * kKeyGroups);      // 4 or 2
    const int bh = blockIdx.x, b = bh / H, h = bh % H, chunk = blockIdx.y;
    const int k0 = chunk * kKeys;
    const int Lp = pad128(L);
    const int c8 = threadIdx.x % kGroups, kg0 = threadIdx.x / kGroups;
    const uint64_t e = fetch(hs.epoch + bh);
    const uint64_t token = head_token(hs, e);

    const uint16_t* vhead = (const uint16_t*)v.ptr + (int64_t)b * v.sB + (int64_t)h * v.sH;
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vhead, ((int64_t)(L - 1) * v.sL + D) * 2);
    uint4 raw[kPasses][4];   // keys k0 + 4 (p kKeyGroups + kg0) + j
    auto load_chunk = [&]() {
        const int off = (int)(((int64_t)(k0 + 4 * kg0) * v.sL + 8 * c8) * 2);
        const int sk = (int)(v.sL * 2), sp = (int)(4 * kKeyGroups * v.sL * 2);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
#pragma unroll
            for (int j = 0; j < 4; ++j) raw[p][j] = load16(vrs, off + p * sp + j * sk);
            if (p + 1 < kPasses) __builtin_amdgcn_s_waitcnt(0x3f70);   // four rows in flight (see K)
        }
    };
    load_chunk();

    // LDS: the chunk-amax exchange, later the transpose tile
    constexpr int kTileWords = D * kKeys / 4;
    constexpr int kRedWords = kThreads * 9;
    __shared__ __attribute__((aligned(16))) uint32_t lds[kTileWords > kRedWords ? kTileWords : kRedWords];
    float(*sm)[9] = (float(*)[9])lds;
    {
        float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x[8];
                unpack8t<BF16>(raw[p][j], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(x[i]));
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = m[i];
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float r = 0.0f;
        for (int g = 0; g < kKeyGroups; ++g) r = fmaxf(r, sm[g * kGroups + d / 8][d % 8]);
        publish(&partial[((int64_t)bh * nchunk + chunk) * D + d], r);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            asm("" : "+v"(raw[p][j].x), "+v"(raw[p][j].y), "+v"(raw[p][j].z), "+v"(raw[p][j].w));
    head_arrive(hs, bh, chunk, nchunk, token);
    __shared__ int met_s;
    const bool met = head_wait(hs, bh, chunk, nchunk, e, token, &met_s);

    __shared__ float inv_s[D];
    float a = 0.0f;   // channel amax over the head (thread d < D)
    if (met) {
        if (threadIdx.x < D)
            a = fold_published(partial + (int64_t)bh * nchunk * D + threadIdx.x, (int64_t)D, nchunk, 0.0f,
                               [](float x, float y) { return fmaxf(x, y); });
    } else {
        // every chunk's amax from the inputs (max is order-free)
        float mm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
        for (int row = kg0; row < nchunk * kKeys; row += kKeyGroups) {
            float x[8];
            unpack8t<BF16>(load16(vrs, (int)(((int64_t)row * v.sL + 8 * c8) * 2)), x);
#pragma unroll
            for (int i = 0; i < 8; ++i) mm[i] = fmaxf(mm[i], fabsf(x[i]));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sm[threadIdx.x][i] = mm[i];
        __syncthreads();
        if (threadIdx.x < D)
            for (int g = 0; g < kKeyGroups; ++g) a = fmaxf(a, sm[g * kGroups + threadIdx.x / 8][threadIdx.x % 8]);
        __syncthreads();
    }
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        inv_s[d] = a > 0.0f ? kFp8Max / a : 0.0f;
        if (chunk == 0) v_scale[(int64_t)bh * D + d] = a / kFp8Max;
    }
    __syncthreads();
    float inv8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) inv8[i] = inv_s[8 * c8 + i];
    auto word = [](int d, int kg) { return d * (kKeys / 4) + 4 * ((kg >> 2) ^ ((d >> 3) & 7)) + (kg & 3); };
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int kg = p * kKeyGroups + kg0;
        float x[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8t<BF16>(raw[p][j], x[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t c = cvt_pk_fp8<false>(x[0][i] * inv8[i], x[1][i] * inv8[i], 0);
            c = cvt_pk_fp8<true>(x[2][i] * inv8[i], x[3][i] * inv8[i], c);
            lds[word(8 * c8 + i, kg)] = c;
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D * (kKeys / 16); c += kThreads) {
        const int d = c / (kKeys / 16), j = c % (kKeys / 16);
        const int key = k0 + 16 * j;
        if (key < Lp) {
            const uint4 val = *(const uint4*)&lds[word(d, 4 * j)];
            *(uint4*)(v_out + ((int64_t)bh * D + d) * Lp + key) = val;
        }
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

// One block = kMxRowBlocks consecutive 128-token row blocks of one (b, h),
// 4 waves x 32 tokens each; row blocks < nqb are Q's, the rest K's.  Rotation
// Y^T = H X^T on bf16/fp16 MFMA (H's +-1 entries and the half-precision inputs
// are exact, accumulation in fp32), then times 1/sqrt(128).  Each lane ends
// with token (l % 32) and channels 32 cb + 8 i + 4 (l / 32) + j, so one MX
// block's amax needs a single cross-lane step and channel pairs (2t, 2t+1) sit
// in the same lane for nibble packing.  The 32 KB Hadamard matrix is staged in
// LDS once per block, for all its row blocks (staged per 128-token row block,
// it moved as many bytes through L2 as K itself).
constexpr int kMxRowBlocks = 4;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_quant_mxfp4(
    HalfView q, HalfView k, int H, int Lq, int Lk, int nqb, int nrb, const float* mu,
    const uint16_t* hmat_bf16, const uint16_t* hmat_f16, float inv_sqrt_r, const float* mu_rot,
    uint8_t* q_out, uint8_t* q_e8, uint8_t* k_out, uint8_t* k_e8) {
    constexpr int D = 128;
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const bool rotate = hmat_bf16 != nullptr;

    // 32 KB: the Hadamard matrix in the inputs' half format (Q and K share it);
    // what the rows lose before quantization, per channel: nothing for Q rows
    // (zeros), the K mean for K rows (rotated when rotating; zeros without
    // smoothing)
    __shared__ uint16_t hs[D * D];
    __shared__ __attribute__((aligned(16))) float sub_s[2][D];
    if (rotate) {
        const uint16_t* hm = BF16 ? hmat_bf16 : hmat_f16;
        for (int c = threadIdx.x; c < D * D / 8; c += kThreads)
            *(uint4*)&hs[8 * (16 * (c / 16) + ((c % 16) ^ ((c / 16) & 15)))] = *(const uint4*)&hm[c * 8];
    }
    const float* ksub = rotate ? mu_rot : mu;
    if (threadIdx.x < D) {
        sub_s[0][threadIdx.x] = 0.0f;
        sub_s[1][threadIdx.x] = ksub ? ksub[(int64_t)bh * D + threadIdx.x] : 0.0f;
    }
    __syncthreads();

#pragma unroll 1
    for (int rb = 0; rb < kMxRowBlocks; ++rb) {
    const int gblk = blockIdx.x * kMxRowBlocks + rb;
    if (gblk >= nrb) break;   // block-uniform
    const bool isq = gblk < nqb;
    const int blk = isq ? gblk : gblk - nqb;
    const int L = isq ? Lq : Lk;
    const int Lp = pad128(L);
    const HalfView& src = isq ? q : k;
    const int token = blk * 128 + wave * 32 + col;
    const bool valid = token < L;
    const float* sub = sub_s[isq ? 0 : 1];

    float y[4][16];   // [cb][e]: channel 32 cb + 8 (e / 4) + 4 half + (e % 4)
    if (rotate) {
        // B operand: this lane's token, channels 16 kc + 8 half + 0..7
        uint4 xb[8];
        const uint16_t* row = (const uint16_t*)src.ptr + (int64_t)b * src.sB +
                              (int64_t)(valid ? token : 0) * src.sL + (int64_t)h * src.sH;
        // loaded unconditionally (row 0 stands in for tokens past L; the
        // rotation zeroes their outputs)
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) xb[kc] = *(const uint4*)(row + 16 * kc + 8 * half);
        mx_rotate_rows<BF16>(hs, xb, inv_sqrt_r, sub, valid, y);
    } else {
        const uint16_t* row = (const uint16_t*)src.ptr + (int64_t)b * src.sB +
                              (int64_t)(valid ? token : 0) * src.sL + (int64_t)h * src.sH;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * cb + 8 * i + 4 * half;
                const uint2 u = *(const uint2*)(row + ch0);   // row 0 for tokens past L
                const float4 sv = *(const float4*)&sub[ch0];
                const uint32_t w[2] = {u.x, u.y};
                const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t bits = (w[j / 2] >> (16 * (j % 2))) & 0xFFFF;
                    const float t = (BF16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits)) - sc[j];
                    y[cb][4 * i + j] = valid ? t : 0.0f;
                }
            }
    }

    uint8_t* out = isq ? q_out : k_out;
    uint8_t* oe = isq ? q_e8 : k_e8;
    int ex[4];
    uint16_t pk[4][4];
    mx_quant_rows(y, ex, pk);
    // Whole 16-byte stores: the token's 64 code bytes are split between the
    // lane pair (l, l ^ 32), bytes 16 cb + 4 i + 2 h + {0, 1} in lane half h.
    // Lane half h collects MX blocks 2 h and 2 h + 1 from both (the partner's
    // halves of them through one exchange) and writes them as two 16-byte
    // chunks; the four E8M0 bytes go out as one dword.  (Byte and 16-bit
    // stores of the same data left the kernel write-bound on partial lines.)
    // (The blocks are picked with selects on the lane half: an array index
    // that depends on the lane compiles to compare-and-select chains and
    // divergent branches.)
    uint32_t mine[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = pk[j][i], hi = pk[2 + j][i];   // blocks j and 2 + j
            const uint32_t keep = half ? hi : lo, send = half ? lo : hi;
            const uint32_t other = (uint32_t)__shfl_xor((int)send, 32) & 0xFFFFu;
            mine[j][i] = half == 0 ? keep | (other << 16) : other | (keep << 16);
        }
    }
    if (token < Lp) {
        uint8_t* orow = out + ((int64_t)bh * Lp + token) * (D / 2);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *(uint4*)(orow + 16 * (2 * half + j)) = make_uint4(mine[j][0], mine[j][1], mine[j][2], mine[j][3]);
        if (half == 0)
            *(uint32_t*)(oe + ((int64_t)bh * Lp + token) * (D / 32)) =
                (uint32_t)(ex[0] + 127) | ((uint32_t)(ex[1] + 127) << 8) | ((uint32_t)(ex[2] + 127) << 16) |
                ((uint32_t)(ex[3] + 127) << 24);
    }
    }   // row blocks
}

}  // namespace

// Blocks of kThreads threads of `kernel` the current device holds at once (0
// if unknown); cached per device and kernel.
static int resident_blocks(const void* kernel) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per_cu = 0;
    int n = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) == hipSuccess)
        n = cus * per_cu;
    cache.emplace(key, n);
    return n;
}

// Single-read head barrier: microseconds a block waits for the other chunks
// of its head before it computes the head's statistic itself.
static std::atomic<int> g_wait_us{2000};

void set_quant_wait_us(int us) { g_wait_us.store(us, std::memory_order_relaxed); }

static HeadSync head_sync(uint64_t* sync, int64_t BH, int nchunk) {
    static std::atomic<uint64_t> nonce{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count()};
    static std::mutex mu;
    static std::map<int, int> khz;   // wall-clock rate per device
    int dev = 0, rate = 0;
    (void)hipGetDevice(&dev);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = khz.find(dev);
        if (it == khz.end()) {
            if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate <= 0)
                rate = 100000;
            it = khz.emplace(dev, rate).first;
        }
        rate = it->second;
    }
    return {sync, sync + BH * nchunk, nonce.fetch_add(1, std::memory_order_relaxed),
            (int64_t)g_wait_us.load(std::memory_order_relaxed) * rate / 1000};
}

// The single-read path: the grid fits on the device at once, token rows do not
// overlap (sL >= D, so rows past L fall outside the buffer resource) and byte
// offsets within one head fit in 32 bits.
static bool single_read_ok(const HalfView& x, int L, int D, int64_t blocks, const void* kernel) {
    if (x.sL < D || (int64_t)(pad128(L) + kMeanChunk) * x.sL * 2 >= 0x7FFFFFFF) return false;
    return kernel == nullptr || blocks <= resident_blocks(kernel);
}

hipError_t launch_k_mean_partial(const HalfView& k, int B, int H, int L, int D, double* partial,
                                 hipStream_t stream) {
    const int nchunk = mean_chunks(L);
    dim3 grid(B * H, nchunk);
    auto kern = D == 128 ? (k.bf16 ? k_mean_partial<128, true> : k_mean_partial<128, false>)
                         : (k.bf16 ? k_mean_partial<64, true> : k_mean_partial<64, false>);
    kern<<<grid, kThreads, 0, stream>>>(k, H, L, nchunk, partial);
    return hipGetLastError();
}

hipError_t launch_k_mean_final(double* partial, int B, int H, int L, int D, float* mu,
                               hipStream_t stream) {
    const int nchunk = mean_chunks(L);
    if (D == 128)
        k_mean_final<128><<<B * H, 128, 0, stream>>>(partial, nchunk, L, mu);
    else
        k_mean_final<64><<<B * H, 64, 0, stream>>>(partial, nchunk, L, mu);
    return hipGetLastError();
}

hipError_t launch_quant_qk_int8(const HalfView& q, const HalfView& k, int B, int H, int Lq,
                                int Lk, int D, int k_block, bool smooth, double* mean_partial,
                                uint64_t* sync, float* mu_out, int8_t* q_out, float* q_scale,
                                int8_t* k_out, float* k_scale, hipStream_t stream) {
    const int nqb = pad128(Lq) / 128, nkb = pad128(Lk) / 128;
    const int nchunk = mean_chunks(Lk);
    const int BH = B * H;
    if (smooth && q.bf16 == k.bf16) {
        auto fused = D == 128 ? (k.bf16 ? k_quant_qk_fused<128, true> : k_quant_qk_fused<128, false>)
                              : (k.bf16 ? k_quant_qk_fused<64, true> : k_quant_qk_fused<64, false>);
        if (single_read_ok(k, Lk, D, BH * nchunk, (const void*)fused) && single_read_ok(q, Lq, D, 0, nullptr)) {
            const HeadSync hs = head_sync(sync, BH, nchunk);
            fused<<<dim3(BH, nchunk), kThreads, 0, stream>>>(q, k, H, Lq, Lk, k_block, nchunk, mean_partial, hs,
                                                             mu_out, q_out, q_scale, k_out, k_scale);
            return hipGetLastError();
        }
    }
    if (smooth) {
        hipError_t e = launch_k_mean_partial(k, B, H, Lk, D, mean_partial, stream);
        if (e == hipSuccess) e = launch_k_mean_final(mean_partial, B, H, Lk, D, mu_out, stream);
        if (e != hipSuccess) return e;
    }
    // Q shares K's precision when both are given (the ABI refuses a mix)
    auto quant = D == 128 ? (k.bf16 ? k_quant_int8<128, true> : k_quant_int8<128, false>)
                          : (k.bf16 ? k_quant_int8<64, true> : k_quant_int8<64, false>);
    quant<<<dim3(BH, nqb + nkb), kThreads, 0, stream>>>(q, k, H, Lq, Lk, k_block, nqb,
                                                        smooth ? mean_partial : nullptr, nchunk,
                                                        q_out, q_scale, k_out, k_scale);
    return hipGetLastError();
}

hipError_t launch_quant_v(const HalfView& v, int B, int H, int Lk, int D, float* amax_partial,
                          uint64_t* sync, uint8_t* v_out, float* v_scale, hipStream_t stream) {
    const int nchunk = mean_chunks(Lk);
    const int BH = B * H;
    auto vfused = D == 128 ? (v.bf16 ? k_quant_v_fused<128, true> : k_quant_v_fused<128, false>)
                           : (v.bf16 ? k_quant_v_fused<64, true> : k_quant_v_fused<64, false>);
    if (single_read_ok(v, Lk, D, BH * nchunk, (const void*)vfused)) {
        const HeadSync hs = head_sync(sync, BH, nchunk);
        vfused<<<dim3(BH, nchunk), kThreads, 0, stream>>>(v, H, Lk, nchunk, amax_partial, hs, v_out, v_scale);
        return hipGetLastError();
    }
    dim3 g1(BH, nchunk), g2(BH, pad128(Lk) / 128);
    if (D == 128) {
        (v.bf16 ? k_v_amax<128, true> : k_v_amax<128, false>)<<<g1, kThreads, 0, stream>>>(v, H, Lk, nchunk,
                                                                                         amax_partial);
        k_v_amax_final<128><<<BH, 128, 0, stream>>>(amax_partial, nchunk, v_scale);
        (v.bf16 ? k_v_quant<128, true> : k_v_quant<128, false>)<<<g2, kThreads, 0, stream>>>(v, H, Lk, nchunk,
                                                                                           amax_partial, v_out);
    } else {
        (v.bf16 ? k_v_amax<64, true> : k_v_amax<64, false>)<<<g1, kThreads, 0, stream>>>(v, H, Lk, nchunk,
                                                                                       amax_partial);
        k_v_amax_final<64><<<BH, 64, 0, stream>>>(amax_partial, nchunk, v_scale);
        (v.bf16 ? k_v_quant<64, true> : k_v_quant<64, false>)<<<g2, kThreads, 0, stream>>>(v, H, Lk, nchunk,
                                                                                         amax_partial, v_out);
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
    const int nrb = nqb + nkb;   // K-only calls come with Lq = 0: no Q row blocks
    dim3 grid((nrb + kMxRowBlocks - 1) / kMxRowBlocks, B * H);
    auto kern = k.bf16 ? k_quant_mxfp4<true> : k_quant_mxfp4<false>;   // Q shares K's precision
    kern<<<grid, kThreads, 0, stream>>>(q, k, H, Lq, Lk, nqb, nrb, mu, (const uint16_t*)hadamard_bf16,
                                        (const uint16_t*)hadamard_f16, inv_sqrt_r, mrot, q_out, q_e8, k_out,
                                        k_e8);
    return hipGetLastError();
}

hipError_t launch_hadamard_build(int R, void* bf16_mat, void* f16_mat, hipStream_t stream) {
    k_hadamard_build<<<R, R, 0, stream>>>(R, (uint16_t*)bf16_mat, (uint16_t*)f16_mat);
    return hipGetLastError();
}

}  // namespace sage

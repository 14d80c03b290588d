// Paged decode over an FP8 e4m3 KV cache with split-KV partials and a merge,
// for gfx950.
//
// Source: ROCm/aiter pull request 7388 (FlyDSL pa_decode), sections Changes
// and "Batch-first plan grid removal": paged attention decode with an FP8 KV
// cache and per-token scales, MTP query tokens, GQA, sliding windows; the work
// is cut into 256-token window tiles, "each tile is its own task"; a reduce
// step merges the partitions and is timed together with the decode; Q and P
// are quantized to the cache's FP8 format (FP8_MAX = 448 on gfx950's OCP e4m3).
//
// Readings (the page does not spell these out): the MTP query tokens are the
// last positions of the context, causal among themselves; with window W a
// query at position p sees keys [p - W + 1, p]; each Q row gets its own e4m3
// scale; the per-token V scale is folded into P before its FP8 conversion,
// with the tile's largest V scale as the conversion scale.
//
// gfx950 design: one block (4 waves) per (sequence, KV head, 256-token tile).
// The 64 query rows of a KV head (MTP x query heads per KV head, padded) are
// quantized once into LDS.  Wave w computes S^T for keys [64 w, 64 w + 64) of
// the tile on v_mfma_f32_32x32x64 (e4m3 x e4m3), reading the K rows straight
// from the paged cache into the A operand (each cache byte is read once per
// block; the loads are issued first so that HBM latency overlaps the Q
// quantization).  After a cross-wave max / sum through LDS, P (scaled by the
// per-token V scale) is written to LDS as e4m3 and wave w computes O^T for
// channels [32 w, 32 w + 32) over all 256 keys, with the transposed V cache
// [page][Hkv][D][page_size] feeding the A operand directly.  Partials (m, l,
// O) go to the workspace; a second kernel merges them.
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;            // query rows per KV head (padded)
constexpr int kTile = kDecodeTile;   // 256 keys per split
constexpr int kD = 128;
constexpr int kPartStride = kD + 4;  // floats per partial row: O[D], m, l, pad

__device__ __forceinline__ int kappa_dec(int r) {
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Keeps the first n (< 16) bytes of v, zeroes the rest.
__device__ __forceinline__ uint4 keep_bytes(uint4 v, int n) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = n - 4 * i;   // bytes of this dword to keep
        const uint32_t m = k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
        w[i] &= m;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__global__ __launch_bounds__(kThreads) void k_paged_decode(DecodeArgs a, float alpha) {
    const int s = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv, hk = bk % a.Hkv;
    const int ctx = a.ctx_lens[b];
    if (ctx <= 0) return;
    const int G = a.Hq / a.Hkv, R = a.MTP * G;
    const int lo_b = a.window > 0 ? max(0, ctx - a.MTP - a.window + 1) : 0;
    const int T = lo_b / kTile + s;
    if (T > (ctx - 1) / kTile) return;            // this sequence has fewer splits
    const int t0 = T * kTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int32_t* ptab = a.page_table + (int64_t)b * a.pt_stride;

    __shared__ __attribute__((aligned(16))) uint8_t q8s[kRows][kD];
    __shared__ __attribute__((aligned(16))) uint8_t p8s[kRows][kTile];
    __shared__ float qss[kRows], kss[kTile], vss[kTile];
    __shared__ float red_m[4][kRows], red_l[4][kRows], red_v[4];

    // ---- 1. issue the K loads of this wave's 64 keys (A operand rows) -----
    // sub-tile t, row r = col: key 64 wave + 32 t + kappa(col); 32 bytes of
    // D-slice [64 c + 32 half, +32) per (t, c).
    uint4 kreg[2][2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int kpos = t0 + 64 * wave + 32 * t + kappa_dec(col);
        const uint8_t* row = nullptr;
        if (kpos < ctx) {
            const int pg = ptab[kpos / a.page];
            row = a.k_cache + (((int64_t)pg * a.Hkv + hk) * a.page + kpos % a.page) * kD;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                kreg[t][c][j] = row ? *(const uint4*)(row + 64 * c + 32 * half + 16 * j)
                                    : make_uint4(0, 0, 0, 0);
    }
    // ---- 2. issue the V^T loads of this wave's channels (A operand of PV)
    // row d = 32 wave + col; keys [64 u + 32 half, +32) of the tile.
    uint4 vreg[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int kpos = t0 + 64 * u + 32 * half;
        const uint8_t* src = nullptr;
        if (kpos < ctx) {
            const int pg = ptab[kpos / a.page];
            src = a.v_cache + (((int64_t)pg * a.Hkv + hk) * kD + 32 * wave + col) * a.page +
                  kpos % a.page;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            vreg[u][j] = src ? *(const uint4*)(src + 16 * j) : make_uint4(0, 0, 0, 0);
            // page slots at or beyond ctx may hold any bytes (e4m3 NaN codes
            // included) and 0 * NaN would poison the product: zero them
            const int nv = ctx - (kpos + 16 * j);
            if (src && nv < 16) vreg[u][j] = keep_bytes(vreg[u][j], nv);
        }
    }
    // ---- 3. per-token scales of the tile ----------------------------------
    {
        const int kpos = t0 + tid;
        float ks = 0.0f, vs = 0.0f;
        if (kpos < ctx) {
            const int pg = ptab[kpos / a.page];
            const int64_t o = ((int64_t)pg * a.Hkv + hk) * a.page + kpos % a.page;
            ks = a.k_scale[o];
            vs = a.v_scale[o];
        }
        kss[tid] = ks;
        vss[tid] = vs;
        // the tile's largest V scale over keys inside [lo_b, ctx)
        float vm = (kpos >= lo_b && kpos < ctx) ? vs : 0.0f;
        vm = wave_max(vm);
        if (lane == 0) red_v[wave] = vm;
    }
    // ---- 4. Q rows -> e4m3 with a per-row scale ------------------------------
    // thread: rows tid / 16 + 16 i, 8 channels [8 (tid % 16), +8)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = tid / 16 + 16 * i, ch = tid % 16;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < R) {
            const int mt = r / G, g = r % G;
            const uint16_t* qp = (const uint16_t*)a.q + (int64_t)b * a.q_sB + (int64_t)mt * a.q_sM +
                                 (int64_t)(hk * G + g) * a.q_sH + 8 * ch;
            const uint4 u = *(const uint4*)qp;
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = bf16_bits_to_f32(w[k] & 0xFFFF);
                x[2 * k + 1] = bf16_bits_to_f32(w[k] >> 16);
            }
        }
        float am = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[k]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
        const float inv = am > 0.0f ? kFp8Max / am : 0.0f;
        uint32_t c0 = cvt_pk_fp8<false>(x[0] * inv, x[1] * inv, 0);
        c0 = cvt_pk_fp8<true>(x[2] * inv, x[3] * inv, c0);
        uint32_t c1 = cvt_pk_fp8<false>(x[4] * inv, x[5] * inv, 0);
        c1 = cvt_pk_fp8<true>(x[6] * inv, x[7] * inv, c1);
        *(uint2*)&q8s[r][8 * ch] = make_uint2(c0, c1);
        if (ch == 0) qss[r] = am / kFp8Max;
    }
    __syncthreads();
    const float vmax = fmaxf(fmaxf(red_v[0], red_v[1]), fmaxf(red_v[2], red_v[3]));

    // ---- 5. S^T = K Q^T for this wave's 64 keys x 64 rows ---------------------
    float x[2][2][16];   // [query block][sub-tile][e]
    float rmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = 32 * qb + col;
        const float qs = qss[r];
        const int mt = r / G;
        const int pos = ctx - a.MTP + mt;
        const int lo = a.window > 0 ? pos - a.window + 1 : 0;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            v16f acc = {0};
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const v4i blo = *(const v4i*)&q8s[r][64 * c + 32 * half];
                const v4i bhi = *(const v4i*)&q8s[r][64 * c + 32 * half + 16];
                const v8i bq = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
                const uint4 k0 = kreg[t][c][0], k1 = kreg[t][c][1];
                const v8i ak = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                                (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
                acc = mfma_f8_32x32x64(ak, bq, acc);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kl = 64 * wave + 32 * t + 16 * half + e;
                const int kpos = t0 + kl;
                const bool ok = r < R && kpos < ctx && kpos <= pos && kpos >= lo;
                const float xv = ((acc[e] * qs) * kss[kl]) * alpha;
                x[qb][t][e] = ok ? xv : -INFINITY;
                rmax[qb] = fmaxf(rmax[qb], x[qb][t][e]);
            }
        }
        rmax[qb] = fmaxf(rmax[qb], __shfl_xor(rmax[qb], 32));
        if (half == 0) red_m[wave][r] = rmax[qb];
    }
    __syncthreads();

    // ---- 6. p = 2^(x - m); P' = p * v_scale -> e4m3 with the tile's vmax ----
    const float pinv = vmax > 0.0f ? kFp8Max / vmax : 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = 32 * qb + col;
        const float M = fmaxf(fmaxf(red_m[0][r], red_m[1][r]), fmaxf(red_m[2][r], red_m[3][r]));
        const float Mb = M == -INFINITY ? 0.0f : M;
        float ls = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint32_t pk[4];
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                float pp[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 4 * w4 + j;
                    const int kl = 64 * wave + 32 * t + 16 * half + e;
                    const float p = __builtin_amdgcn_exp2f(x[qb][t][e] - Mb);
                    ls += p;
                    pp[j] = (p * vss[kl]) * pinv;
                }
                uint32_t v = cvt_pk_fp8<false>(pp[0], pp[1], 0);
                pk[w4] = cvt_pk_fp8<true>(pp[2], pp[3], v);
            }
            *(uint4*)&p8s[r][64 * wave + 32 * t + 16 * half] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
        ls += __shfl_xor(ls, 32);
        if (half == 0) red_l[wave][r] = ls;
    }
    __syncthreads();

    // ---- 7. O^T = V^T P^T for channels [32 wave, +32) ---------------------------
    const float back = vmax / kFp8Max;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int r = 32 * qb + col;
        v16f acc = {0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4i blo = *(const v4i*)&p8s[r][64 * u + 32 * half];
            const v4i bhi = *(const v4i*)&p8s[r][64 * u + 32 * half + 16];
            const v8i bp = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
            const uint4 v0 = vreg[u][0], v1 = vreg[u][1];
            const v8i av = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                            (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
            acc = mfma_f8_32x32x64(av, bp, acc);
        }
        if (r < R) {
            float* prow = a.partials + (((int64_t)bk * a.num_splits + s) * kRows + r) * kPartStride;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * wave + 8 * i + 4 * half;
                *(float4*)(prow + d0) = make_float4(acc[4 * i] * back, acc[4 * i + 1] * back,
                                                    acc[4 * i + 2] * back, acc[4 * i + 3] * back);
            }
            if (wave == 0 && half == 0) {
                const float M = fmaxf(fmaxf(red_m[0][r], red_m[1][r]), fmaxf(red_m[2][r], red_m[3][r]));
                const float L = red_l[0][r] + red_l[1][r] + red_l[2][r] + red_l[3][r];
                prow[kD] = M;
                prow[kD + 1] = L;
            }
        }
    }
}

// Merge of the split partials of one (sequence, KV head, row): m* = max m_s,
// out = sum 2^(m_s - m*) O_s / sum 2^(m_s - m*) l_s (fp32, split order), bf16.
// One wave per row: lane s holds split s's (m, l) (splits beyond 64 are
// folded in lane order); the weights are broadcast and every lane then merges
// two output channels over all splits with coalesced loads.
constexpr int kMergeRowsPerBlock = 4;

__global__ __launch_bounds__(64 * kMergeRowsPerBlock) void k_decode_merge(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int rowg = blockIdx.x * kMergeRowsPerBlock + (threadIdx.x >> 6);
    const int R = a.MTP * (a.Hq / a.Hkv);
    const int bk = rowg / kRows, r = rowg % kRows;
    if (bk >= a.B * a.Hkv || r >= R) return;
    const int b = bk / a.Hkv, hk = bk % a.Hkv;
    const int ctx = a.ctx_lens[b];
    const int G = a.Hq / a.Hkv;
    const int lo_b = a.window > 0 ? max(0, ctx - a.MTP - a.window + 1) : 0;
    const int nsp = ctx > 0 ? (ctx - 1) / kTile - lo_b / kTile + 1 : 0;
    const float* base = a.partials + ((int64_t)bk * a.num_splits * kRows + r) * kPartStride;
    const int64_t sstride = (int64_t)kRows * kPartStride;
    float M = -INFINITY;
    for (int sp = lane; sp < nsp; sp += 64) M = fmaxf(M, base[sp * sstride + kD]);
    M = wave_max(M);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s0 = 0; s0 < nsp; s0 += 64) {
        const int sp = s0 + lane;
        float w = 0.0f, lw = 0.0f;
        if (sp < nsp) {
            const float ms = base[sp * sstride + kD];
            w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            lw = w * base[sp * sstride + kD + 1];
        }
        const int n = min(64, nsp - s0);
        for (int j = 0; j < n; ++j) {
            const float wj = __shfl(w, j);
            L = L + __shfl(lw, j);
            const float2 o = *(const float2*)(base + (s0 + j) * sstride + 2 * lane);
            o0 = o0 + wj * o.x;
            o1 = o1 + wj * o.y;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int mt = r / G, g = r % G;
    uint16_t* op = (uint16_t*)a.out + (int64_t)b * a.o_sB + (int64_t)mt * a.o_sM +
                   (int64_t)(hk * G + g) * a.o_sH + 2 * lane;
    *(uint32_t*)op = f32_to_bf16_bits(o0 * inv) | ((uint32_t)f32_to_bf16_bits(o1 * inv) << 16);
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    const float alpha = a.sm_scale * kLog2e;
    dim3 grid(a.num_splits, a.B * a.Hkv);
    k_paged_decode<<<grid, kThreads, 0, stream>>>(a, alpha);
    const int rows = a.B * a.Hkv * kRows;
    k_decode_merge<<<(rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock, 64 * kMergeRowsPerBlock, 0,
                     stream>>>(a);
    return hipGetLastError();
}

}  // namespace sage

// Quantized attention forward for gfx950 (SageAttention2 style).
//
// Numeric sequence per KV tile, in the order of the "Sage2 SM89 Temporal Pair
// Experiment" README (Candidate section: QK -> update_mdo -> accumulate_d ->
// RS_32_to_8 -> PV):
//   S   = Q8 K8^T on INT8 MFMA (int32, exact), or the scaled-MXFP4 MFMA (fp32)
//   x   = S * q_scale * k_scale * sm_scale * log2(e)          (INT8)
//       = S * sm_scale * log2(e)                              (MXFP4)
//   m'  = max(m, rowmax x); O *= 2^(m - m'); l *= 2^(m - m')
//   p   = 2^(x - m'); l += sum p                              (fp32, before FP8)
//   P8  = e4m3(448 p)   (448 = FP8_MAX of OCP e4m3, per ROCm/aiter pull request
//                         7388, Changes: Q and P are quantized to FP8_MAX's format)
//   O  += P8 V8 on FP8 MFMA, fp32 accumulation
// Epilogue: out = O * v_scale[d] / (448 l)  (the V scale is fused here, as in
// the README's fuse_v_scale kernel; 1/FP8_MAX as in the aiter epilogue).
//
// gfx950 design:
//  - Block = 4 waves = 128 query rows (one Q scale block); each wave owns 32
//    query rows for the whole KV loop (Q fragments stay in VGPRs).
//  - KV tiles of 128 keys are staged through LDS with a two-stage double
//    buffer (global -> VGPR prefetch of tile j+1 overlaps the math of tile j;
//    one barrier per tile).  16-byte chunks are XOR-swizzled per row so the
//    MFMA operand reads do not collide on LDS banks.
//  - The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_i32_32x32x32_i8: each lane then holds one query and, per 32-key
//    sub-tile, 16 consecutive keys (K rows are fed to the A operand in a
//    permuted order that makes this so).  That register layout is exactly the
//    B operand of the PV product O^T = V^T P^T (v_mfma_f32_32x32x64 e4m3), so
//    P never leaves registers, and V^T (stored transposed, keys contiguous)
//    is read in natural key order, two 16-byte LDS reads per operand.
//  - Row max is taken on the int32 scores (rounding is monotone, so
//    max fp32(S c) = fp32(max S c)); the O/l rescale is skipped when no row of
//    the wave changed its max; 448 is folded into the exp2 offset.
#include "sage_device.hpp"
#include "sage_launch.hpp"

#include <type_traits>

namespace sage {
namespace {

constexpr int kBM = 128;     // query rows per block
constexpr int kBN = kKvTile; // keys per KV tile
constexpr int kThreads = 256;
constexpr float kLog2Fp8Max = 8.807354922057604f;   // log2(448)

// Element size of one K row in bytes: INT8 codes D, packed E2M1 codes D/2.
template <int D, bool MX>
struct Geo {
    static constexpr int kRowBytes = MX ? D / 2 : D;       // K / Q row bytes
    static constexpr int kRowChunks = kRowBytes / 16;      // 16-byte chunks per row
    static constexpr int kKBytes = kBN * kRowBytes;
    static constexpr int kKScaleBytes = MX ? kBN * (D / 32) : 0;
    static constexpr int kVBytes = D * kBN;
    static constexpr int kStageBytes = kKBytes + kKScaleBytes + kVBytes;
    static constexpr int kVChunksPerRow = kBN / 16;        // 8
};

// A-operand row r of a 32-key sub-tile holds key kappa(r); with this order
// the D/C element e = 4 i + j of lane l is key 16 (l / 32) + e.
__device__ __forceinline__ int kappa(int r) {
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// XOR swizzles of the 16-byte chunks of an LDS row.  gfx950's LDS serves a
// 16-byte-per-lane read 16 lanes at a time over 64 four-byte banks, so the 16
// rows one such lane group reads (rows kappa(0..15) or kappa(16..31) of a
// sub-tile for K, 16 consecutive channels for V) must land in 16 distinct
// 16-byte bank groups.
template <int D, bool MX>
__device__ __forceinline__ int k_swz(int r) {
    if constexpr (Geo<D, MX>::kRowChunks == 8)          // 128-byte rows: 2 rows per bank sweep
        return ((r >> 1) & 3) | ((r >> 2) & 4);
    else                                               // 64-byte rows: 4 rows per bank sweep
        return ((r >> 2) & 1) | ((r >> 3) & 2);
}

__device__ __forceinline__ int v_swz(int d) { return (d >> 1) & 7; }

template <int D, bool MX>
__device__ __forceinline__ uint8_t* k_lds_addr(uint8_t* base, int r, int c) {
    using G = Geo<D, MX>;
    return base + r * G::kRowBytes + 16 * (c ^ k_swz<D, MX>(r));
}
__device__ __forceinline__ uint8_t* v_lds_addr(uint8_t* vbase, int d, int c) {
    return vbase + d * kBN + 16 * (c ^ v_swz(d));
}

// One KV tile (K codes, K E8M0 scales for MXFP4, V^T codes) is copied from
// global memory straight into an LDS stage with gfx950's 16-byte global->LDS
// loads: each wave instruction fills 64 consecutive 16-byte LDS chunks (lane
// i -> chunk i), so the XOR swizzle is applied on the global side by letting
// lane i fetch the chunk that belongs at its LDS position.  Completion is
// awaited with s_waitcnt vmcnt(0) followed by a block barrier.
template <int D, bool MX, int NWAVES>
struct TileDma {
    using G = Geo<D, MX>;
    static constexpr int kKChunks = G::kKBytes / 16;
    static constexpr int kVChunks = G::kVBytes / 16;
    static constexpr int kKSChunks = G::kKScaleBytes / 16;
    static constexpr int kKRegions = kKChunks / 64;   // 1 KB regions
    static constexpr int kVRegions = kVChunks / 64;
    static_assert(kKChunks % 64 == 0 && kVChunks % 64 == 0, "tile must be whole 1 KB regions");
    static_assert(kKRegions % NWAVES == 0 && kVRegions % NWAVES == 0, "regions split evenly");
    static_assert(kKSChunks <= 64, "K scales fit one wave instruction");

    // kr: K codes of this (b, kv head) [Lkp][row bytes]; ksr: its E8M0 scales
    // [Lkp][D/32] (MXFP4); vr: V^T of this (b, kv head) [D][Lkp].  Buffer
    // resources bound to exactly those extents (reads outside return 0); the
    // tile offset goes in the scalar offset, the swizzled chunk offset in the
    // per-lane offset.
    __device__ __forceinline__ static void issue(uint8_t* stage, __amdgpu_buffer_rsrc_t kr,
                                                 __amdgpu_buffer_rsrc_t ksr,
                                                 __amdgpu_buffer_rsrc_t vr, int Lkp, int kt,
                                                 int wave, int lane, bool with_v = true) {
#pragma unroll
        for (int j = 0; j < kKRegions / NWAVES; ++j) {
            const int region = j * NWAVES + wave;
            const int p = region * 64 + lane;                  // LDS chunk position
            const int r = p / G::kRowChunks;
            const int c = (p % G::kRowChunks) ^ k_swz<D, MX>(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, stage + region * 1024, 16,
                                                     r * G::kRowBytes + 16 * c, kt * G::kKBytes, 0, 0);
        }
        if constexpr (MX) {
            if (wave == 0 && lane < kKSChunks)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ksr, stage + G::kKBytes, 16, 16 * lane,
                                                         kt * G::kKScaleBytes, 0, 0);
        }
        if (!with_v) return;
        uint8_t* vstage = stage + G::kKBytes + G::kKScaleBytes;
#pragma unroll
        for (int j = 0; j < kVRegions / NWAVES; ++j) {
            const int region = j * NWAVES + wave;
            const int p = region * 64 + lane;
            const int d = p / G::kVChunksPerRow;
            const int c = (p % G::kVChunksPerRow) ^ v_swz(d);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vstage + region * 1024, 16, d * Lkp + 16 * c,
                                                     kt * kBN, 0, 0);
        }
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    // raw buffer, stride 0, bounds = bytes; dword 3 = gfx9 raw-buffer config
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                             0x00020000);
}

__device__ __forceinline__ void wait_dma() {
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's LDS DMA has landed
}

// Q fragment of one wave: query row (l % 32) of the wave's 32 rows.
// INT8: 16-byte chunk (2 c + half) for c < D/32.  MXFP4: chunk (2 c + half)
// for c < D/64 plus the E8M0 byte of MX block (2 c + half).
template <int D, bool MX>
struct QFrag {
    static constexpr int kN = MX ? D / 64 : D / 32;
    v4i f[kN];
    int s[MX ? kN : 1];
};

// The QK step of one 32-key sub-tile t of the staged tile.  Shared by the
// attention kernel and the debug tile kernel.
template <int D>
__device__ __forceinline__ v16i qk_subtile_i8(uint8_t* stage, const QFrag<D, false>& q, int t,
                                              int lane) {
    const int half = lane >> 5;
    const int r = 32 * t + kappa(lane & 31);
    v16i acc = {0};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        const v4i a = *(const v4i*)k_lds_addr<D, false>(stage, r, 2 * c + half);
        acc = mfma_i8_32x32x32(a, q.f[c], acc);
    }
    return acc;
}

template <int D>
__device__ __forceinline__ v16f qk_subtile_mx(uint8_t* stage, const QFrag<D, true>& q, int t,
                                              int lane) {
    using G = Geo<D, true>;
    const int half = lane >> 5;
    const int r = 32 * t + kappa(lane & 31);
    const uint8_t* ks = stage + G::kKBytes;
    v16f acc = {0};
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        const v4i a4 = *(const v4i*)k_lds_addr<D, true>(stage, r, 2 * c + half);
        // fp4 operands occupy the low four dwords; the upper four are not read
        const v8i a = __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1);
        const v8i b = __builtin_shufflevector(q.f[c], q.f[c], 0, 1, 2, 3, -1, -1, -1, -1);
        const int sa = ks[r * (D / 32) + 2 * c + half];
        acc = mfma_f4_32x32x64(a, b, acc, sa, q.s[c]);
    }
    return acc;
}

// QK of the four 32-key sub-tiles of a staged tile, with the K fragments of
// sub-tile t+1 read from LDS before the MFMAs of sub-tile t.
template <int D, bool MX, class SAcc>
__device__ __forceinline__ void qk_tile(uint8_t* stage, const QFrag<D, MX>& q, int lane, SAcc* S) {
    if constexpr (MX) {
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = qk_subtile_mx<D>(stage, q, t, lane);
    } else {
        constexpr int NC = D / 32;
        const int half = lane >> 5, col = lane & 31;
        v4i kf[2][NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
            kf[0][c] = *(const v4i*)k_lds_addr<D, false>(stage, kappa(col), 2 * c + half);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t + 1 < 4) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    kf[(t + 1) & 1][c] = *(const v4i*)k_lds_addr<D, false>(
                        stage, 32 * (t + 1) + kappa(col), 2 * c + half);
            }
            v16i acc = {0};
#pragma unroll
            for (int c = 0; c < NC; ++c) acc = mfma_i8_32x32x32(kf[t & 1][c], q.f[c], acc);
            S[t] = acc;
        }
    }
}

template <int D, bool MX>
__device__ __forceinline__ void load_qfrag(QFrag<D, MX>& q, const uint8_t* qbase,
                                           const uint8_t* qsc, int row, int lane) {
    using G = Geo<D, MX>;
    const int half = lane >> 5;
#pragma unroll
    for (int c = 0; c < QFrag<D, MX>::kN; ++c)
        q.f[c] = *(const v4i*)(qbase + (int64_t)row * G::kRowBytes + 16 * (2 * c + half));
    if constexpr (MX) {
#pragma unroll
        for (int c = 0; c < QFrag<D, MX>::kN; ++c) q.s[c] = qsc[(int64_t)row * (D / 32) + 2 * c + half];
    }
}

template <int D, bool MX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_fwd(AttnArgs a, float alpha) {
    using G = Geo<D, MX>;
    constexpr int kNT = 4;              // 32-key sub-tiles per tile
    constexpr int kDB = D / 32;         // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * G::kStageBytes];

    const int Lqp = pad128(a.Lq), Lkp = pad128(a.Lk);
    const int nqb = Lqp / kBM;
    const int BH = a.B * a.H;
    // Block order: causal -> longest query blocks first; otherwise head-major
    // so that the blocks streaming one head's K/V run close together.
    int qb, bh;
    if (a.causal) {
        qb = nqb - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
    } else {
        bh = (int)(blockIdx.x / nqb);
        qb = (int)(blockIdx.x % nqb);
    }
    const int b = bh / a.H, h = bh % a.H;
    const int hk = h / (a.H / a.Hkv);
    const int bhk = b * a.Hkv + hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int half = lane >> 5, col = lane & 31;
    const int q0w = qb * kBM + wave * 32;
    const int qrow = q0w + col;

    const uint8_t* qbase = (const uint8_t*)a.q + (int64_t)bh * Lqp * G::kRowBytes;
    const uint8_t* qsc = MX ? (const uint8_t*)a.q_scale + (int64_t)bh * Lqp * (D / 32) : nullptr;
    const uint8_t* kbase = (const uint8_t*)a.k + (int64_t)bhk * Lkp * G::kRowBytes;
    const uint8_t* ksc = MX ? (const uint8_t*)a.k_scale + (int64_t)bhk * Lkp * (D / 32) : nullptr;
    const uint8_t* vbase = a.v + (int64_t)bhk * D * Lkp;

    // Number of KV tiles this block visits.
    int ntiles = Lkp / kBN;
    if (a.causal) ntiles = min(ntiles, (qb * kBM + kBM - 1) / kBN + 1);

    QFrag<D, MX> qf;
    load_qfrag<D, MX>(qf, qbase, qsc, qrow, lane);
    float q_s = 0.0f;
    if constexpr (!MX) q_s = ((const float*)a.q_scale)[(int64_t)bh * (Lqp / a.q_block) + qb * kBM / a.q_block];
    const float* kscale_f = MX ? nullptr : (const float*)a.k_scale + (int64_t)bhk * (Lkp / a.k_block);

    using Dma = TileDma<D, MX, 4>;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)Lkp * G::kRowBytes);
    const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(MX ? ksc : kbase, MX ? (int64_t)Lkp * (D / 32) : 16);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (int64_t)D * Lkp);
    Dma::issue(smem, krs, ksrs, vrs, Lkp, 0, wave, lane);
    // INT8: the two 64-key block scales of the next tile, folded with q_scale
    // and alpha (c = fp32(fp32(q_s k_s) alpha)); prefetched one tile ahead.
    const int kb_per_tile = MX ? 0 : kBN / a.k_block;
    float ksn[2] = {0.0f, 0.0f};
    if constexpr (!MX) {
        ksn[0] = kscale_f[0];
        ksn[1] = kscale_f[kb_per_tile - 1];
    }

    v16f O[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) O[i] = v16f{0};
    float m = -INFINITY, l = 0.0f;

    for (int kt = 0; kt < ntiles; ++kt) {
        uint8_t* stage = smem + (kt & 1) * G::kStageBytes;
        wait_dma();
        __syncthreads();
        float ksc_t[2] = {ksn[0], ksn[1]};
        if (kt + 1 < ntiles) {
            Dma::issue(smem + ((kt + 1) & 1) * G::kStageBytes, krs, ksrs, vrs, Lkp, kt + 1, wave, lane);
            if constexpr (!MX) {
                ksn[0] = kscale_f[(kt + 1) * kb_per_tile];
                ksn[1] = kscale_f[(kt + 1) * kb_per_tile + kb_per_tile - 1];
            }
        }

        const int key0 = kt * kBN;
        // waves whose every key of this tile is causally masked skip it
        if (a.causal && key0 > q0w + 31) continue;
        const bool full = (key0 + kBN <= a.Lk) && (!a.causal || key0 + kBN - 1 <= q0w);

        // S holds int32 (INT8) or fp32 (MXFP4) scores of the 4 sub-tiles;
        // element (t, e) is key key0 + 32 t + 16 half + e of query qrow.
        using SAcc = typename std::conditional<MX, v16f, v16i>::type;
        float c[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) c[t] = MX ? alpha : (q_s * ksc_t[t < 2 ? 0 : 1]) * alpha;

        // The tile body, instantiated once for full tiles and once for tiles
        // that cross the causal diagonal or the ragged end.  In the latter,
        // each 32-key sub-tile is (wave-uniformly) empty, crossing or full for
        // this wave's 32 rows: empty sub-tiles skip their MFMAs and exps and
        // only crossing ones test keys one by one.
        auto tile_body = [&](auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            int st[kNT];   // 0 empty, 1 crossing, 2 full
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                if constexpr (FULL) {
                    st[t] = 2;
                } else {
                    const int lo = key0 + 32 * t, hi = lo + 31;
                    const bool empty = lo >= a.Lk || (a.causal && lo > q0w + 31);
                    const bool whole = hi < a.Lk && (!a.causal || hi <= q0w);
                    st[t] = empty ? 0 : (whole ? 2 : 1);
                }
            }
            auto visible = [&](int t, int e) {
                const int key = key0 + 32 * t + 16 * half + e;
                return key < a.Lk && (!a.causal || key <= qrow);
            };
            SAcc S[kNT];
            if constexpr (FULL) {
                qk_tile<D, MX>(stage, qf, lane, S);
            } else {
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    if (st[t] == 0) continue;
                    if constexpr (MX)
                        S[t] = qk_subtile_mx<D>(stage, qf, t, lane);
                    else
                        S[t] = qk_subtile_i8<D>(stage, qf, t, lane);
                }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                if (st[t] == 2) {
                    auto mx = S[t][0];
#pragma unroll
                    for (int e = 1; e < 16; ++e) mx = S[t][e] > mx ? S[t][e] : mx;
                    tmax = fmaxf(tmax, (float)mx * c[t]);   // rounding is monotone
                } else if (st[t] == 1) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        tmax = fmaxf(tmax, visible(t, e) ? (float)S[t][e] * c[t] : -INFINITY);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

            // ---- online softmax update -------------------------------------
            const float m_new = fmaxf(m, tmax);
            if (__any(m_new > m)) {
                const float sc = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
                l *= sc;
#pragma unroll
                for (int i = 0; i < kDB; ++i) O[i] *= sc;
            }
            m = m_new;
            const float mb = (m_new == -INFINITY ? 0.0f : m_new) - kLog2Fp8Max;

            // q = 448 * 2^(x - m) evaluated as 2^(fma(S, c, -(m - log2 448))); l
            // accumulates q (so l = 448 * sum p).  Packed into the PV B operand:
            // byte 16 t' + e of group u is key 64 u + 32 t' + 16 half + e; the PV
            // MFMAs of group u follow its conversion so they overlap group u+1's.
            uint8_t* vb = stage + G::kKBytes + G::kKScaleBytes;
            float ls = 0.0f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (st[2 * u] == 0 && st[2 * u + 1] == 0) continue;
                v8i pf;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const int t = 2 * u + w / 4, e0 = 4 * (w % 4);
                    if (st[t] == 0) {
                        pf[w] = 0;
                        continue;
                    }
                    float p[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float xv = __builtin_fmaf((float)S[t][e0 + j], c[t], -mb);
                        if (st[t] == 1 && !visible(t, e0 + j)) xv = -INFINITY;
                        p[j] = __builtin_amdgcn_exp2f(xv);
                    }
                    ls += (p[0] + p[1]) + (p[2] + p[3]);
                    uint32_t pk = cvt_pk_fp8<false>(p[0], p[1], 0);
                    pk = cvt_pk_fp8<true>(p[2], p[3], pk);
                    pf[w] = (int)pk;
                }
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    const int d = 32 * db + col;
                    const v4i lo = *(const v4i*)v_lds_addr(vb, d, 4 * u + half);
                    const v4i hi = *(const v4i*)v_lds_addr(vb, d, 4 * u + 2 + half);
                    const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    O[db] = mfma_f8_32x32x64(av, pf, O[db]);
                }
            }
            l += ls;
        };
        if (full)
            tile_body(std::true_type{});
        else
            tile_body(std::false_type{});
    }

    // ---- epilogue: out = (O * v_scale) / l (times the reciprocal of l), written
    // with the caller's strides
    const float lt = l + __shfl_xor(l, 32);
    const float inv_l = lt > 0.0f ? 1.0f / lt : 0.0f;   // one division per row
    if (qrow < a.Lq) {
        const float* vs = a.v_scale + (int64_t)bhk * D;
        const int64_t ooff = (int64_t)b * a.out.sB + (int64_t)qrow * a.out.sL + (int64_t)h * a.out.sH;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * half;
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = (O[db][4 * i + j] * vs[d0 + j]) * inv_l;
                if (a.out.dtype == kOutF32) {
                    *(float4*)((float*)a.out.ptr + ooff + d0) = make_float4(o[0], o[1], o[2], o[3]);
                } else {
                    uint32_t w[2];
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        uint32_t h0, h1;
                        if (a.out.dtype == kOutBF16) {
                            h0 = __builtin_bit_cast(uint16_t, (__bf16)o[j]);
                            h1 = __builtin_bit_cast(uint16_t, (__bf16)o[j + 1]);
                        } else {
                            h0 = __builtin_bit_cast(uint16_t, (_Float16)o[j]);
                            h1 = __builtin_bit_cast(uint16_t, (_Float16)o[j + 1]);
                        }
                        w[j / 2] = h0 | (h1 << 16);
                    }
                    *(uint2*)((uint16_t*)a.out.ptr + ooff + d0) = make_uint2(w[0], w[1]);
                }
            }
    }
}

// Test hook: int32 S = Q8 K8^T through the same staging and qk_subtile_i8 as
// the attention kernel.  One wave per (32 queries, 128 keys, b*h).
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk(const int8_t* q, const int8_t* k, int Lqp, int Lkp,
                                                 int q0, int k0, int nq, int nk, int32_t* out) {
    using G = Geo<D, false>;
    __shared__ __attribute__((aligned(16))) uint8_t stage[G::kStageBytes];
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    const int qg = blockIdx.x, kg = blockIdx.y, bh = blockIdx.z;
    const uint8_t* qbase = (const uint8_t*)q + (int64_t)bh * Lqp * D;
    const uint8_t* kbase = (const uint8_t*)k + (int64_t)bh * Lkp * D + (int64_t)k0 * D;
    // stage K rows [k0 + 128 kg, +128); the V part of the stage is not used
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)nk * D);
    TileDma<D, false, 1>::issue(stage, krs, krs, krs, 0, kg, 0, lane, false);
    wait_dma();
    __syncthreads();
    QFrag<D, false> qf;
    load_qfrag<D, false>(qf, qbase, nullptr, q0 + 32 * qg + col, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const v16i s = qk_subtile_i8<D>(stage, qf, t, lane);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = 128 * kg + 32 * t + 16 * half + e;   // relative to k0
            const int qq = 32 * qg + col;                         // relative to q0
            out[((int64_t)bh * nq + qq) * nk + key] = s[e];
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    const int nqb = pad128(a.Lq) / kBM;
    const float alpha = a.sm_scale * kLog2e;
    dim3 grid((unsigned)(nqb * a.B * a.H));
    if (a.mxfp4) {
        k_attn_fwd<128, true><<<grid, kThreads, 0, stream>>>(a, alpha);
    } else if (a.D == 128) {
        k_attn_fwd<128, false><<<grid, kThreads, 0, stream>>>(a, alpha);
    } else {
        k_attn_fwd<64, false><<<grid, kThreads, 0, stream>>>(a, alpha);
    }
    return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q, const int8_t* k, int B, int H, int Lqp, int Lkp,
                           int D, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t stream) {
    dim3 grid(nq / 32, nk / 128, B * H);
    if (D == 128)
        k_debug_qk<128><<<grid, 64, 0, stream>>>(q, k, Lqp, Lkp, q0, k0, nq, nk, out);
    else
        k_debug_qk<64><<<grid, 64, 0, stream>>>(q, k, Lqp, Lkp, q0, k0, nq, nk, out);
    return hipGetLastError();
}

}  // namespace sage

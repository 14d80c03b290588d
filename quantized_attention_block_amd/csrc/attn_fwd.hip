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
//    query rows for the whole KV loop (Q fragments stay in VGPRs).  Three
//    blocks share a CU (<= 168 VGPRs per lane, 48 KB of LDS per block), so
//    while one wave waits on an MFMA result, an LDS read or a barrier, the
//    other waves of its SIMD issue VALU and MFMA work.  (A software-pipelined
//    form of the loop, QK of tile j+1 and PV of tile j-1 around the softmax of
//    tile j, needs ~226 VGPRs and so runs two waves per SIMD; it measured
//    7-10 % slower.  The wave-pair ping-pong schedule further down, two waves
//    per SIMD alternating MFMA and softmax phases between barriers, is kept
//    as an option; it measured about 1.4x slower.)
//  - KV tiles of 64 keys are copied global -> LDS with 16-byte
//    buffer_load ... lds instructions (no staging registers) into a ring of
//    three LDS stages, two tiles ahead of use.  The per-tile barrier waits
//    only for the tile it needs (s_waitcnt vmcnt(N) + s_barrier; the release
//    fence of __syncthreads() would drain every copy in flight).  16-byte
//    chunks are XOR-swizzled per row so the MFMA operand reads do not collide
//    on LDS banks.
//  - The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_i32_32x32x32_i8: each lane then holds one query and, per 32-key
//    sub-tile, 16 consecutive keys (K rows are fed to the A operand in a
//    permuted order that makes this so).  That register layout is exactly the
//    B operand of the PV product O^T = V^T P^T (v_mfma_f32_32x32x64 e4m3), so
//    P never leaves registers, and V^T (stored transposed, keys contiguous)
//    is read in natural key order, two 16-byte LDS reads per operand.
//  - INT8 scores are exact int32; fp32(S) is one exact v_cvt_f32_i32.  Row
//    max is taken on the integer scores (rounding is monotone, so
//    max fp32(S c) = fp32(max S c)); the O/l rescale is skipped when no row of
//    the wave that has seen a key changed its max; 448 is folded into the
//    exp2 offset.
//  - Q may arrive as the caller's fp16/bf16 tensor instead of INT8 codes: the
//    block's 128 rows are exactly one Q scale block, so the prologue quantizes
//    them with the quantize kernels' arithmetic (codes and scale bit-identical)
//    and no INT8 copy of Q is written or read.  The V scales of the KV head
//    are copied to LDS ahead of tile 0 for the epilogue.
#include "sage_device.hpp"
#include "sage_launch.hpp"

#include <type_traits>

namespace sage {
namespace {

constexpr int kBM = 128;            // query rows per block
constexpr int kBN = kKvTile;        // keys per KV tile
constexpr int kNT = kBN / 32;       // 32-key sub-tiles per tile
constexpr int kStages = 3;          // LDS ring: tile j read, j+1 and j+2 landing
constexpr int kWavesPerSimd = 3;    // occupancy target: 3 blocks of 4 waves per CU
constexpr int kThreads = 256;
constexpr float kLog2Fp8Max = 8.807354922057604f;   // log2(448)
static_assert(kBN == 64, "the PV operand packing assumes 64-key tiles");

// Byte geometry of one LDS stage: K codes (INT8: D bytes per key, E2M1: D/2),
// the E8M0 scales of K (MXFP4 only), then V^T codes (D rows of kBN keys).
template <int D, bool MX>
struct Geo {
    static constexpr int kRowBytes = MX ? D / 2 : D;       // K / Q row bytes
    static constexpr int kRowChunks = kRowBytes / 16;      // 16-byte chunks per row
    static constexpr int kKBytes = kBN * kRowBytes;
    static constexpr int kKScaleBytes = MX ? kBN * (D / 32) : 0;
    static constexpr int kVOff = kKBytes + kKScaleBytes;
    static constexpr int kVBytes = D * kBN;
    static constexpr int kStageBytes = kVOff + kVBytes;
    static constexpr int kVRowChunks = kBN / 16;           // 4
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

// V^T rows are 64 bytes (4 chunks): 4 channels share one bank sweep.
__device__ __forceinline__ int v_swz(int d) { return (d >> 2) & 3; }

template <int D, bool MX>
__device__ __forceinline__ uint8_t* k_lds_addr(uint8_t* base, int r, int c) {
    using G = Geo<D, MX>;
    return base + r * G::kRowBytes + 16 * (c ^ k_swz<D, MX>(r));
}
template <int D, bool MX>
__device__ __forceinline__ uint8_t* v_lds_addr(uint8_t* stage, int d, int c) {
    return stage + Geo<D, MX>::kVOff + d * kBN + 16 * (c ^ v_swz(d));
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

    // Per-lane parts of the copy offsets with four waves.  Region j * 4 + wave
    // of a tile starts at byte 1024 (j * 4 + wave) of the K block, or at V^T
    // row 16 (j * 4 + wave); the swizzle of a chunk depends on the lane and
    // the wave only (for K on row bits that region j * 4 adds nothing to, for
    // V^T on (row / 4) % 4 = lane / 16), so each copy's per-lane offset is
    // one of these two values and j moves only the scalar offset: two live
    // registers across the KV loop instead of one per copy instruction.
    struct LaneOffsets {
        int k, v;
    };
    __device__ __forceinline__ static LaneOffsets lane_offsets(int Lkp, int wave, int lane) {
        static_assert(NWAVES == 4, "offsets shared across regions need four waves");
        const int p = wave * 64 + lane;   // region `wave`, chunk `lane`
        const int r = p / G::kRowChunks, c = (p % G::kRowChunks) ^ k_swz<D, MX>(r);
        const int d = p / G::kVRowChunks, cv = (p % G::kVRowChunks) ^ v_swz(d);
        return {r * G::kRowBytes + 16 * c, d * Lkp + 16 * cv};
    }
    __device__ __forceinline__ static void issue4(uint8_t* stage, __amdgpu_buffer_rsrc_t kr,
                                                  __amdgpu_buffer_rsrc_t ksr, __amdgpu_buffer_rsrc_t vr,
                                                  int Lkp, int kt, int wave, int lane, const LaneOffsets& lo) {
#pragma unroll
        for (int j = 0; j < kKRegions / NWAVES; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, stage + (j * NWAVES + wave) * 1024, 16, lo.k,
                                                     kt * G::kKBytes + j * NWAVES * 1024, 0, 0);
        if constexpr (MX) {
            if (wave == 0 && lane < kKSChunks)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ksr, stage + G::kKBytes, 16, 16 * lane,
                                                         kt * G::kKScaleBytes, 0, 0);
        }
        uint8_t* vstage = stage + G::kVOff;
#pragma unroll
        for (int j = 0; j < kVRegions / NWAVES; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vstage + (j * NWAVES + wave) * 1024, 16, lo.v,
                                                     kt * kBN + j * NWAVES * 16 * Lkp, 0, 0);
    }

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
        uint8_t* vstage = stage + G::kVOff;
#pragma unroll
        for (int j = 0; j < kVRegions / NWAVES; ++j) {
            const int region = j * NWAVES + wave;
            const int p = region * 64 + lane;
            const int d = p / G::kVRowChunks;
            const int c = (p % G::kVRowChunks) ^ v_swz(d);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vstage + region * 1024, 16, d * Lkp + 16 * c,
                                                     kt * kBN, 0, 0);
        }
    }
};

__device__ __forceinline__ void wait_dma() {
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's LDS DMA has landed
}

// Workgroup barrier after this wave's LDS DMA of all but its last N loads has
// landed (loads complete in issue order) and its LDS reads and writes are
// done.  __syncthreads() would also wait for every load in flight, including
// the DMA of tiles that are not needed yet.  The empty asm statements keep
// the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void dma_barrier() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0070 | N);   // vmcnt(N) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

// INT8 scores are exact int32 (|S| <= D * 127^2); fp32(S) is one
// v_cvt_f32_i32, exact for |S| < 2^24.  (Accumulating on top of the bit
// pattern of 1.5 * 2^23 would make the conversion an add, but its sixteen
// accumulator registers pushed the kernel past its register budget into
// spills whose reloads inside the KV loop waited for every tile copy in
// flight.)  The row max is taken on the integer scores (rounding is monotone).
// Row max of raw scores: integer max for INT8, fmaxf for MXFP4 (scores are
// finite, so fmaxf's NaN rule never applies; a compare-and-select does not
// map to v_max3_f32).
__device__ __forceinline__ int vmax(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ float vmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float score_f(int s) { return (float)s; }
__device__ __forceinline__ float score_f(float s) { return s; }

// The QK step of one 32-key sub-tile t of a staged tile (int32 scores).
// Shared by the attention kernel and the debug tile kernel.
template <int D>
__device__ __forceinline__ v16i qk_subtile_i8(uint8_t* stage, const QFrag<D, false>& q, int t, int lane) {
    static_assert(D <= 1024, "int32 scores exact in fp32 need |S| < 2^24");
    const int half = lane >> 5;
    const int r = 32 * t + kappa(lane & 31);
    v4i kf[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) kf[c] = *(const v4i*)k_lds_addr<D, false>(stage, r, 2 * c + half);
    v16i acc = mfma_i8_32x32x32(kf[0], q.f[0], v16i{0});
#pragma unroll
    for (int c = 1; c < D / 32; ++c) acc = mfma_i8_32x32x32(kf[c], q.f[c], acc);
    return acc;
}

template <int D>
__device__ __forceinline__ v16f qk_subtile_mx(uint8_t* stage, const QFrag<D, true>& q, int t,
                                              int lane) {
    using G = Geo<D, true>;
    const int half = lane >> 5;
    const int r = 32 * t + kappa(lane & 31);
    const uint8_t* ks = stage + G::kKBytes;
    v4i kf[D / 64];
    int sa[D / 64];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        kf[c] = *(const v4i*)k_lds_addr<D, true>(stage, r, 2 * c + half);
        sa[c] = ks[r * (D / 32) + 2 * c + half];
    }
    v16f acc = {0};
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        // fp4 operands occupy the low four dwords; the upper four are not read
        const v8i a = __builtin_shufflevector(kf[c], kf[c], 0, 1, 2, 3, -1, -1, -1, -1);
        const v8i b = __builtin_shufflevector(q.f[c], q.f[c], 0, 1, 2, 3, -1, -1, -1, -1);
        acc = mfma_f4_32x32x64(a, b, acc, sa[c], q.s[c]);
    }
    return acc;
}

template <int D, bool MX>
using SAccT = typename std::conditional<MX, v16f, v16i>::type;

template <int D, bool MX>
__device__ __forceinline__ SAccT<D, MX> qk_subtile(uint8_t* stage, const QFrag<D, MX>& q, int t, int lane) {
    if constexpr (MX)
        return qk_subtile_mx<D>(stage, q, t, lane);
    else
        return qk_subtile_i8<D>(stage, q, t, lane);
}

// O^T += V^T P^T for one staged 64-key tile.  A operand: V^T row (channel
// 32 db + lane % 32), keys [16 half, +16) and [32 + 16 half, +16); B: the
// packed P of the tile (byte 16 t + e of lane l = key 32 t + 16 (l / 32) + e).
template <int D, bool MX>
__device__ __forceinline__ void pv_tile(uint8_t* stage, const v8i& pf, int lane, v16f* O) {
    const int half = lane >> 5, col = lane & 31;
    v8i av[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + col;
        const v4i lo = *(const v4i*)v_lds_addr<D, MX>(stage, d, half);
        const v4i hi = *(const v4i*)v_lds_addr<D, MX>(stage, d, 2 + half);
        av[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) O[db] = mfma_f8_32x32x64(av[db], pf, O[db]);
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

// Workgroup barrier once this wave's LDS accesses are done (vector memory
// operations in flight are not waited for, unlike __syncthreads()).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Fused Q quantization.  Lane l of a wave loads the fp16/bf16 channels of its
// Q fragment chunks, [16 (2 c + half), +16) for c < D/32, of query row qrow;
// rows past Lq read as zeros (the buffer resource ends with row Lq - 1).
template <int D>
__device__ __forceinline__ void load_q_rows(uint4 (&raw)[D / 16], const HalfView& q, int b, int h, int Lq,
                                            int qrow, int half) {
    const uint16_t* head = (const uint16_t*)q.ptr + (int64_t)b * q.sB + (int64_t)h * q.sH;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(head, ((int64_t)(Lq - 1) * q.sL + D) * 2);
    const int off = qrow < Lq ? (int)((int64_t)qrow * q.sL * 2) : 0x7FFFFF00;   // past the resource
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        const int o = off + 32 * (2 * c + half);
        raw[2 * c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
        raw[2 * c + 1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o + 16, 0, 0));
    }
}

// The 128 rows of four waves are one INT8 quantization block of Q: amax over
// the block (rows past Lq are zeros), codes clamp(rne(x * (127 / amax)),
// -127, 127), scale amax / 127 (returned) -- the arithmetic of the Q blocks of
// the quantize kernels, so the codes and the scale are theirs bit for bit.
// The clamp comes before the rounding (the bounds are integers, and a NaN
// product still gives -127), and the rounding is the addition of 1.5 * 2^23,
// whose result has spacing 1 and holds the code in its low byte.
// red: LDS floats for the waves' amax; wave w writes red[w], the block's four
// waves are red[red_base + 0..3]; one workgroup barrier between the writes
// and the reads, so every wave of the workgroup calls this once.
template <int D, bool BF16>
__device__ __forceinline__ float quant_qfrag(QFrag<D, false>& qf, const uint4 (&raw)[D / 16], float* red,
                                             int wave, int red_base = 0) {
    auto lo = [](uint32_t w) { return BF16 ? __uint_as_float(w << 16) : f16_bits_to_f32(w & 0xFFFFu); };
    auto hi = [](uint32_t w) { return BF16 ? __uint_as_float(w & 0xFFFF0000u) : f16_bits_to_f32(w >> 16); };
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) am = fmaxf(fmaxf(am, fabsf(lo(w[i]))), fabsf(hi(w[i])));
    }
    am = wave_max_xor(am);
    if ((threadIdx.x & 63) == 0) red[wave] = am;
    lds_barrier();
    float amax = red[red_base];
#pragma unroll
    for (int w = 1; w < 4; ++w) amax = fmaxf(amax, red[red_base + w]);   // the block's four waves
    amax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax)));   // uniform
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    // adding 1.5 * 2^23 rounds to the nearest integer (ties to even) and leaves
    // it in the low bits of the float
    constexpr float kRne = 12582912.0f;
    auto code = [&](float x) {   // float bits whose low byte is the code
        return __float_as_uint(fminf(127.0f, fmaxf(-127.0f, x * inv)) + kRne);
    };
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4& u = raw[2 * c + k / 2];
            const uint32_t a = (k & 1) ? u.z : u.x, b = (k & 1) ? u.w : u.y;
            // bytes [code(a.lo), code(a.hi)] and [code(b.lo), code(b.hi)], then both
            const uint32_t pa = __builtin_amdgcn_perm(code(hi(a)), code(lo(a)), 0x0C0C0400u);
            const uint32_t pb = __builtin_amdgcn_perm(code(hi(b)), code(lo(b)), 0x0C0C0400u);
            wd[k] = __builtin_amdgcn_perm(pb, pa, 0x05040100u);
        }
        qf.f[c] = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
    }
    return amax > 0.0f ? amax / 127.0f : 0.0f;
}

// Fused MXFP4 Q quantization (D = 128): lane (row, half) of a wave loads its
// query row's channels [16 kc + 8 half, +8), the Hadamard matrix a.hmat
// (NULL: no rotation) is copied to `ring` (the KV ring, still unused), and
// the rows are rotated and quantized as the MXFP4 quantizer does.  The lane
// keeps MX blocks 2 c + half (c = 0, 1), the A/B operand chunks of the QK
// step: its own halves of those blocks and, swapped with its partner lane
// l ^ 32, the partner's halves.  Returns after a block barrier, so the ring is
// free for the tile copies.
__device__ __forceinline__ void mx_fused_qfrag(QFrag<128, true>& qf, const AttnKernelArgs& a, const HalfView& qh,
                                               int b, int h, int qrow, uint8_t* ring) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const bool valid = qrow < a.Lq;
    const uint16_t* row = (const uint16_t*)qh.ptr + (int64_t)b * qh.sB + (int64_t)(valid ? qrow : 0) * qh.sL +
                          (int64_t)h * qh.sH;
    float y[4][16];
    if (a.hmat) {
        uint4 xb[8];
#pragma unroll
        for (int kc = 0; kc < 8; ++kc)
            xb[kc] = valid ? *(const uint4*)(row + 16 * kc + 8 * half) : make_uint4(0, 0, 0, 0);
        // 32 KB of +-1 entries: 32 regions of 1 KB, eight per wave.  LDS chunk
        // p holds chunk (p % 16) ^ (r % 16) of row r = p / 16 (the layout
        // mx_rotate_rows reads), so each lane fetches the global chunk that
        // belongs at its position.
        const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.hmat, D * D * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int region = 4 * j + wave;
            const int p = 64 * region + lane, r = p >> 4, c = (p & 15) ^ (r & 15);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, ring + 1024 * region, 16, 256 * r + 16 * c, 0, 0, 0);
        }
        wait_dma();
        __syncthreads();
        mx_rotate_rows((const uint16_t*)ring, xb, qh.bf16, a.inv_sqrt_r, valid, y);
    } else {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * cb + 8 * i + 4 * half;
                const uint2 u = valid ? *(const uint2*)(row + ch0) : make_uint2(0, 0);
                const uint32_t w[2] = {u.x, u.y};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t bits = (w[j / 2] >> (16 * (j % 2))) & 0xFFFF;
                    const float t = qh.bf16 ? bf16_bits_to_f32(bits) : f16_bits_to_f32(bits);
                    y[cb][4 * i + j] = valid ? t : 0.0f;
                }
            }
    }
    int ex[4];
    uint16_t pk[4][4];
    mx_quant_rows(y, ex, pk);
    // (blocks picked with selects and shifts on the lane half, not an array
    // index that depends on the lane: that compiles to compare-and-select
    // chains or a scratch array)
    const uint32_t e8 = (uint32_t)(ex[0] + 127) | ((uint32_t)(ex[1] + 127) << 8) |
                        ((uint32_t)(ex[2] + 127) << 16) | ((uint32_t)(ex[3] + 127) << 24);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        uint32_t wd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // bytes 4 i + {0, 1} of a block come from half 0, 4 i + {2, 3} from half 1
            const uint32_t lo = pk[2 * c][i], hi = pk[2 * c + 1][i];   // blocks 2 c and 2 c + 1
            const uint32_t mine = half ? hi : lo, theirs = half ? lo : hi;
            const uint32_t other = (uint32_t)__shfl_xor((int)theirs, 32) & 0xFFFFu;
            wd[i] = half == 0 ? mine | (other << 16) : other | (mine << 16);
        }
        qf.f[c] = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        qf.s[c] = (int)((e8 >> (8 * (2 * c + half))) & 0xFFu);
    }
    __syncthreads();   // every wave is done reading the Hadamard matrix from the ring
}

// Sub-tile states of the 64-key tile starting at key0 for one wave's query
// rows [q0w, +32): 0 no key visible to any of the rows, 2 every key visible to
// every row, 1 crossing (keys tested one by one).  FULL: all 2, no tests.
template <bool FULL>
__device__ __forceinline__ void tile_states(int (&st)[kNT], int key0, int Lk, bool causal, int q0w) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        if constexpr (FULL) {
            st[t] = 2;
        } else {
            const int lo = key0 + 32 * t, hi = lo + 31;
            const bool empty = lo >= Lk || (causal && lo > q0w + 31);
            const bool whole = hi < Lk && (!causal || hi <= q0w);
            st[t] = empty ? 0 : (whole ? 2 : 1);
        }
    }
}

// The online-softmax step of one staged tile for this lane's query row qrow
// (S: element (t, e) is key key0 + 32 t + 16 half + e; c the tile's score
// scale): row max, the O / l rescale when some row's max grew, and
// q = 448 * 2^(x - m) packed as the PV B operand into pf.  Returns the
// tile's sum of q for l (added by the caller).
template <int D, bool MX, bool FULL>
__device__ __forceinline__ float tile_softmax(const SAccT<D, MX> (&S)[kNT], const int (&st)[kNT], int key0,
                                              int half, int Lk, bool causal, int qrow, float c, float& m,
                                              float& l, v16f (&O)[D / 32], v8i& pf) {
    auto visible = [&](int t, int e) {
        const int key = key0 + 32 * t + 16 * half + e;
        return key < Lk && (!causal || key <= qrow);
    };
    // row max (on the integer scores for INT8: rounding is monotone, and
    // c > 0, so the max of the scaled scores is the scaled max score)
    float tmax = -INFINITY;
    if constexpr (FULL) {
        auto mx = S[0][0];
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int e = t == 0 ? 1 : 0; e < 16; ++e) mx = vmax(mx, S[t][e]);
        tmax = score_f(mx) * c;
    } else {
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            if (st[t] == 2) {
                auto mx = S[t][0];
#pragma unroll
                for (int e = 1; e < 16; ++e) mx = vmax(mx, S[t][e]);
                tmax = fmaxf(tmax, score_f(mx) * c);
            } else if (st[t] == 1) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    tmax = fmaxf(tmax, visible(t, e) ? score_f(S[t][e]) * c : -INFINITY);
            }
        }
    }
    const float m_new = fmaxf(m, half_pair_max(tmax));
    // online-softmax rescale, skipped when no row's max moved; a row that
    // has seen no key yet (m = -inf) holds O = 0 and l = 0, which the
    // rescale by 0 leaves as they are, so its first max does not count
    if (__any(m_new > m && m != -INFINITY)) {
        const float sc = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
        l *= sc;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) O[i] *= sc;
    }
    m = m_new;
    const float mb = (FULL || m_new != -INFINITY ? m_new : 0.0f) - kLog2Fp8Max;

    // q = 448 * 2^(x - m) evaluated as 2^(fma(S, c, -(m - log2 448))); l
    // accumulates q (so l = 448 * sum p).  Packed as the PV B operand:
    // byte 16 t + e = key 32 t + 16 half + e of the tile.  The low-word
    // conversion keeps the high word of its third operand, which the
    // high-word conversion overwrites: the word's stale value is passed, so
    // no register has to be zeroed first.
    float ls = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const int t = w / 4, e0 = 4 * (w % 4);
        if (st[t] == 0) {
            pf[w] = 0;
            continue;
        }
        float p[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float xv = __builtin_fmaf(score_f(S[t][e0 + jj]), c, -mb);
            if (st[t] == 1 && !visible(t, e0 + jj)) xv = -INFINITY;
            p[jj] = __builtin_amdgcn_exp2f(xv);
        }
        // (in a full tile the first word's sum starts ls: 0 + x = x for the
        // non-negative x here, so the sum is the same)
        if (FULL && w == 0)
            ls = (p[0] + p[1]) + (p[2] + p[3]);
        else
            ls += (p[0] + p[1]) + (p[2] + p[3]);
        uint32_t pk = cvt_pk_fp8<false>(p[0], p[1], (uint32_t)pf[w]);
        pk = cvt_pk_fp8<true>(p[2], p[3], pk);
        pf[w] = (int)pk;
    }
    return ls;
}

// Epilogue: out = (O * v_scale) / l (times the reciprocal of l, one division
// per row) for this lane's query row, written with the caller's strides.  vs:
// the KV head's V scales in LDS.
template <int D>
__device__ __forceinline__ void store_rows(const AttnKernelArgs& a, const v16f (&O)[D / 32], float l,
                                           const float* vs, int b, int h, int qrow, int half) {
    const float lt = l + __shfl_xor(l, 32);
    const float inv_l = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qrow >= a.Lq) return;
    const int64_t ooff = (int64_t)b * a.out.sB + (int64_t)qrow * a.out.sL + (int64_t)h * a.out.sH;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * db + 8 * i + 4 * half;
            float o[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[jj] = (O[db][4 * i + jj] * vs[d0 + jj]) * inv_l;
            if (a.out.dtype == kOutF32) {
                *(float4*)((float*)a.out.ptr + ooff + d0) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                uint32_t w[2];
#pragma unroll
                for (int jj = 0; jj < 4; jj += 2) {
                    uint32_t h0, h1;
                    if (a.out.dtype == kOutBF16) {
                        h0 = __builtin_bit_cast(uint16_t, (__bf16)o[jj]);
                        h1 = __builtin_bit_cast(uint16_t, (__bf16)o[jj + 1]);
                    } else {
                        h0 = __builtin_bit_cast(uint16_t, (_Float16)o[jj]);
                        h1 = __builtin_bit_cast(uint16_t, (_Float16)o[jj + 1]);
                    }
                    w[jj / 2] = h0 | (h1 << 16);
                }
                *(uint2*)((uint16_t*)a.out.ptr + ooff + d0) = make_uint2(w[0], w[1]);
            }
        }
}

// QF: Q quantized in the prologue from the fp16/bf16 view qh (INT8 per
// 128-row block, or MXFP4 with the Hadamard rotation).
template <int D, bool MX, bool QF = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd))) void k_attn_fwd(
    AttnKernelArgs a, float alpha, HalfView qh) {
    using G = Geo<D, MX>;
    using SAcc = SAccT<D, MX>;
    constexpr int kDB = D / 32;         // 32-row blocks of O^T
    // the KV ring, this KV head's V scales (fp32 [D], D <= 128), the waves'
    // Q amax (fused Q quantization)
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * G::kStageBytes + 512 + 16];
    static_assert(D * 4 <= 512, "V scales fit their LDS slot");

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

    // KV tiles this block visits (causal: up to its last query row).  Tiles
    // past the real keys of the padded length are never visited.
    int ntiles = (a.Lk + kBN - 1) / kBN;
    if (a.causal) ntiles = min(ntiles, (qb * kBM + kBM - 1) / kBN + 1);

    using Dma = TileDma<D, MX, 4>;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)Lkp * G::kRowBytes);
    const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(MX ? ksc : kbase, MX ? (int64_t)Lkp * (D / 32) : 16);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (int64_t)D * Lkp);
    auto stage_of = [&](int kt) { return smem + (kt % kStages) * G::kStageBytes; };
    // DMA instructions one tile costs every wave (wave 0 of MXFP4 issues one
    // more, for the K scales; counting without it only waits longer)
    constexpr int kDma = Dma::kKRegions / 4 + Dma::kVRegions / 4;

    // The V scales go to LDS ahead of tile 0 (wave 0, one instruction; they
    // have landed once step 0's barrier is passed), so that the epilogue reads
    // them without a global load: that would wait in the vector memory
    // counter, which on this architecture also counts the output stores.
    uint8_t* const vs_lds = smem + kStages * G::kStageBytes;
    // fused Q: this lane's fp16/bf16 Q loads go out ahead of the copies, so
    // that the Q block's amax does not wait for the first two KV tiles
    uint4 qraw[QF && !MX ? D / 16 : 1];
    if constexpr (QF && !MX) load_q_rows<D>(qraw, qh, b, h, a.Lq, qrow, half);
    if (wave == 0 && lane < D / 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a.v_scale + (int64_t)bhk * D, D * 4), vs_lds, 16,
                                                 16 * lane, 0, 0, 0);
    QFrag<D, MX> qf;
    // Fused MXFP4 Q: the block's 128 rows are rotated and quantized with the
    // MXFP4 quantizer's own arithmetic (mx_rotate_rows / mx_quant_rows), so the
    // codes are its codes bit for bit.  The Hadamard matrix is staged in the
    // KV ring before any tile is copied there (32 KB of the ring's 36.75 KB).
    if constexpr (QF && MX) mx_fused_qfrag(qf, a, qh, b, h, qrow, smem);
    // tiles 0 and 1 in flight before the loop; tile j + 2 is issued in step j
    const typename Dma::LaneOffsets dma_lane = Dma::lane_offsets(Lkp, wave, lane);
    Dma::issue4(stage_of(0), krs, ksrs, vrs, Lkp, 0, wave, lane, dma_lane);
    if (ntiles > 1) Dma::issue4(stage_of(1), krs, ksrs, vrs, Lkp, 1, wave, lane, dma_lane);

    float q_s = 0.0f;
    if constexpr (QF && MX) {
        // done above
    } else if constexpr (QF) {
        q_s = qh.bf16 ? quant_qfrag<D, true>(qf, qraw, (float*)(vs_lds + 512), wave)
                      : quant_qfrag<D, false>(qf, qraw, (float*)(vs_lds + 512), wave);
        q_s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, q_s)));
    } else {
        load_qfrag<D, MX>(qf, qbase, qsc, qrow, lane);
    }
    // Score scale of tile kt: c = fp32(fp32(q_s k_s) alpha) for INT8 (a 64-key
    // tile lies inside one K scale block), alpha for MXFP4.  (Read through the
    // constant address space: a scalar load, which does not queue behind the
    // LDS DMA in the vector memory counter.)
    if (!MX && !QF) q_s = ((const float*)a.q_scale)[(int64_t)bh * (Lqp / a.q_block) + qb * kBM / a.q_block];
    const float* kscale_f = MX ? nullptr : (const float*)a.k_scale + (int64_t)bhk * (Lkp / a.k_block);
    const __attribute__((address_space(4))) float* kscale_c =
        (const __attribute__((address_space(4))) float*)kscale_f;
    // K scale block of tile kt: kt * kBN / k_block, a shift (k_block is 64 or
    // 128; a division here cost ~20 scalar instructions per tile)
    const int kshift = __builtin_amdgcn_readfirstlane(a.k_block == 2 * kBN ? 1 : 0);
    auto tile_c = [&](int kt) -> float {
        if constexpr (MX) return alpha;
        else return (q_s * kscale_c[kt >> kshift]) * alpha;
    };

    v16f O[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) O[i] = v16f{0};
    float m = -INFINITY, l = 0.0f;
    v8i pf = {0, 0, 0, 0, 0, 0, 0, 0};

    // One KV tile.  FULL steps (no key of the tile masked for any row of the
    // block) have no per-key tests; the others mask per 32-key sub-tile, which
    // is wave-uniformly empty, crossing (keys tested one by one) or full for
    // this wave's rows.
    // STG: the LDS stage of tile j (= j % kStages) as a compile-time constant,
    // so that every LDS operand address is a per-lane offset plus an
    // immediate; kStages means "compute it".
    auto step = [&](int j, auto full_tag, auto stage_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr int STG = decltype(stage_tag)::value;
        uint8_t* stage = STG < kStages ? smem + STG * G::kStageBytes : stage_of(j);
        uint8_t* stage2 = STG < kStages ? smem + ((STG + 2) % kStages) * G::kStageBytes : stage_of(j + 2);
        // every wave's part of tile j has landed (tile j+1 may be in flight)
        // and all waves finished step j-1, whose stage tile j+2 reuses
        if (j + 1 < ntiles)
            dma_barrier<kDma>();
        else
            dma_barrier<0>();
        if (j + 2 < ntiles) Dma::issue4(stage2, krs, ksrs, vrs, Lkp, j + 2, wave, lane, dma_lane);
        const float c = tile_c(j);
        const int key0 = j * kBN;

        int st[kNT];
        tile_states<FULL>(st, key0, a.Lk, a.causal, q0w);
        // S: element (t, e) is key key0 + 32 t + 16 half + e of query qrow
        SAcc S[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) S[t] = qk_subtile<D, MX>(stage, qf, t, lane);
        const float ls = tile_softmax<D, MX, FULL>(S, st, key0, half, a.Lk, a.causal, qrow, c, m, l, O, pf);
        pv_tile<D, MX>(stage, pf, lane, O);
        l += ls;
    };

    // Tiles [0, n_full) are full for every wave of the block.
    int n_full = a.Lk / kBN;
    if (a.causal) n_full = min(n_full, qb * (kBM / kBN));
    n_full = min(n_full, ntiles);
    int j = 0;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using SR = std::integral_constant<int, kStages>;
    static_assert(kStages == 3, "the full-tile loop is unrolled once per stage");
    for (; j + 3 <= n_full; j += 3) {
        step(j, std::true_type{}, S0{});
        step(j + 1, std::true_type{}, S1{});
        step(j + 2, std::true_type{}, S2{});
    }
    for (; j < n_full; ++j) step(j, std::true_type{}, SR{});
    for (; j < ntiles; ++j) step(j, std::false_type{}, SR{});

    store_rows<D>(a, O, l, (const float*)vs_lds, b, h, qrow, half);
}

// ---- Wave-pair ping-pong schedule -------------------------------------------
// The "Sage2 SM89 Temporal Pair Experiment" README (Candidate section) pairs
// warps so that one pair runs QK and the softmax while the other runs PV of
// the previous tile, then they swap.  Here: a workgroup of 8 waves = two
// groups of four, each owning one 128-row Q block (two consecutive Q blocks of
// one head), so every SIMD holds one wave of each group.  A wave alternates
// two phases separated by workgroup barriers: X(j) = PV of tile j - 1 and QK
// of tile j (MFMA work), Y(j) = the softmax of tile j (VALU work).  Group 1
// passes one barrier more at the start, so whenever one group is in X the
// other is in Y.  The K/V tiles are shared by the two groups (copied once per
// 256 query rows) in a ring of four stages: tile j is read until X(j + 1) of
// group 1, which ends at the barrier after which tile j + 4 is issued.  Per
// row the arithmetic is the interleaved kernel's (the same helpers in the
// same order), so the outputs are equal bit for bit.  INT8 QK, D = 128.
constexpr int kPPWaves = 8;
constexpr int kPPStages = 4;

template <bool QF>
__device__ __forceinline__ void attn_fwd_pp(const AttnKernelArgs& a, float alpha, const HalfView& qh) {
    constexpr int D = 128;
    constexpr bool MX = false;
    using G = Geo<D, MX>;
    using Dma = TileDma<D, MX, kPPWaves>;
    using SAcc = SAccT<D, MX>;
    constexpr int kDB = D / 32;
    // DMA instructions one tile costs every wave
    constexpr int kDma = Dma::kKRegions / kPPWaves + Dma::kVRegions / kPPWaves;
    // the KV ring, the KV head's V scales (fp32 [D]), the waves' Q amax (QF)
    __shared__ __attribute__((aligned(16))) uint8_t smem[kPPStages * G::kStageBytes + 512 + (QF ? 4 * kPPWaves : 0)];

    const int Lqp = pad128(a.Lq), Lkp = pad128(a.Lk);
    const int nqb = Lqp / kBM, npr = (nqb + 1) / 2;   // Q blocks, pairs of them
    const int BH = a.B * a.H;
    // causal: longest pairs first, heads fastest; otherwise head-major
    int pr, bh;
    if (a.causal) {
        pr = npr - 1 - (int)(blockIdx.x / BH);
        bh = (int)(blockIdx.x % BH);
    } else {
        bh = (int)(blockIdx.x / npr);
        pr = (int)(blockIdx.x % npr);
    }
    const int b = bh / a.H, h = bh % a.H;
    const int hk = h / (a.H / a.Hkv);
    const int bhk = b * a.Hkv + hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wq = wave & 3;
    const int half = lane >> 5, col = lane & 31;
    // this group's Q block; qb == nqb (no rows) for the second group of the
    // last pair when nqb is odd
    const int qb = 2 * pr + grp;
    const bool live = qb < nqb;
    const int q0w = qb * kBM + wq * 32;
    const int qrow = q0w + col;

    // tiles this group visits, and the workgroup's (the later block's)
    const int nkt = (a.Lk + kBN - 1) / kBN;
    int my_nt = live ? nkt : 0;
    if (a.causal && live) my_nt = min(my_nt, (qb * kBM + kBM - 1) / kBN + 1);
    int nt = nkt;
    if (a.causal) nt = min(nt, (min(2 * pr + 1, nqb - 1) * kBM + kBM - 1) / kBN + 1);
    // tiles [0, n_full) are full for every row of this group
    int n_full = a.Lk / kBN;
    if (a.causal) n_full = min(n_full, qb * (kBM / kBN));

    const uint8_t* kbase = (const uint8_t*)a.k + (int64_t)bhk * Lkp * G::kRowBytes;
    const uint8_t* vbase = a.v + (int64_t)bhk * D * Lkp;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)Lkp * G::kRowBytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, (int64_t)D * Lkp);
    auto stage_of = [&](int kt) { return smem + (kt % kPPStages) * G::kStageBytes; };

    uint8_t* const vs_lds = smem + kPPStages * G::kStageBytes;
    uint4 qraw[QF ? D / 16 : 1];
    if constexpr (QF) load_q_rows<D>(qraw, qh, b, h, a.Lq, qrow, half);   // rows past Lq read as zeros
    if (wave == 0 && lane < D / 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a.v_scale + (int64_t)bhk * D, D * 4), vs_lds, 16,
                                                 16 * lane, 0, 0, 0);
    Dma::issue(stage_of(0), krs, krs, vrs, Lkp, 0, wave, lane);
    if (nt > 1) Dma::issue(stage_of(1), krs, krs, vrs, Lkp, 1, wave, lane);

    QFrag<D, MX> qf;
    float q_s;
    if constexpr (QF) {
        float* red = (float*)(vs_lds + 512);
        q_s = qh.bf16 ? quant_qfrag<D, true>(qf, qraw, red, wave, 4 * grp)
                      : quant_qfrag<D, false>(qf, qraw, red, wave, 4 * grp);
        q_s = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, q_s)));
    } else {
        // a group without rows reads row 0 (in bounds) and computes nothing
        const uint8_t* qbase = (const uint8_t*)a.q + (int64_t)bh * Lqp * G::kRowBytes;
        load_qfrag<D, MX>(qf, qbase, nullptr, live ? qrow : 0, lane);
        q_s = ((const float*)a.q_scale)[(int64_t)bh * (Lqp / a.q_block) + (live ? qb : 0) * kBM / a.q_block];
    }
    const __attribute__((address_space(4))) float* kscale_c =
        (const __attribute__((address_space(4))) float*)((const float*)a.k_scale + (int64_t)bhk * (Lkp / a.k_block));
    const int kshift = __builtin_amdgcn_readfirstlane(a.k_block == 2 * kBN ? 1 : 0);

    v16f O[kDB];
#pragma unroll
    for (int i = 0; i < kDB; ++i) O[i] = v16f{0};
    float m = -INFINITY, l = 0.0f;
    v8i pf = {0, 0, 0, 0, 0, 0, 0, 0};

    // Tile j is first read in X(j) of group 0, so before the barrier that
    // starts it every wave waits for its own copies of tile j: group 0 at its
    // X(j) barrier, group 1 at the same barrier, which for it starts Y(j - 1)
    // (or is its extra first barrier).  At either point a wave's most recent
    // copies (tile j + 1) may still be in flight.
    auto dma_wait_barrier = [&](int t) {   // every tile up to t landed
        if (t + 1 < nt)
            dma_barrier<kDma>();
        else
            dma_barrier<0>();
    };
    if (grp == 1) dma_wait_barrier(0);   // the second group runs one phase behind
    for (int j = 0; j <= nt; ++j) {
        // ---- X(j).  Every wave has finished X(j - 1), the last reader of the
        // stage tile j + 2 reuses.
        if (grp == 0)
            dma_wait_barrier(j);
        else
            lds_barrier();
        if (j + 2 < nt) Dma::issue(stage_of(j + 2), krs, krs, vrs, Lkp, j + 2, wave, lane);
        if (j >= 1 && j - 1 < my_nt) pv_tile<D, MX>(stage_of(j - 1), pf, lane, O);
        const bool qk = j < my_nt;
        SAcc S[kNT];
        if (qk) {
#pragma unroll
            for (int t = 0; t < kNT; ++t) S[t] = qk_subtile<D, MX>(stage_of(j), qf, t, lane);
        }
        // ---- Y(j): the softmax of tile j (for group 1 this barrier starts X(j + 1) of group 0)
        if (grp == 1)
            dma_wait_barrier(j + 1);
        else
            lds_barrier();
        if (qk) {
            const float c = (q_s * kscale_c[j >> kshift]) * alpha;
            const int key0 = j * kBN;
            int st[kNT];
            float ls;
            if (j < n_full) {
                tile_states<true>(st, key0, a.Lk, a.causal, q0w);
                ls = tile_softmax<D, MX, true>(S, st, key0, half, a.Lk, a.causal, qrow, c, m, l, O, pf);
            } else {
                tile_states<false>(st, key0, a.Lk, a.causal, q0w);
                ls = tile_softmax<D, MX, false>(S, st, key0, half, a.Lk, a.causal, qrow, c, m, l, O, pf);
            }
            l += ls;
        }
    }
    if (grp == 0) lds_barrier();   // both groups pass the same number of barriers

    if (live) store_rows<D>(a, O, l, (const float*)vs_lds, b, h, qrow, half);
}

// (Two kernels around one template body: with a kernel template here this
// compiler emitted the host launch stub of only the first instantiation.)
__global__ __launch_bounds__(64 * kPPWaves) void k_attn_fwd_pp_fused_q(AttnKernelArgs a, float alpha, HalfView qh) {
    attn_fwd_pp<true>(a, alpha, qh);
}
__global__ __launch_bounds__(64 * kPPWaves) void k_attn_fwd_pp(AttnKernelArgs a, float alpha, HalfView qh) {
    attn_fwd_pp<false>(a, alpha, qh);
}

// Test hook: int32 S = Q8 K8^T through the same staging and qk_subtile_i8 as
// the attention kernel.  One wave per (32 queries, one KV tile of keys, b*h).
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk(const int8_t* q, const int8_t* k, int Lqp, int Lkp,
                                                 int q0, int k0, int nq, int nk, int32_t* out) {
    using G = Geo<D, false>;
    __shared__ __attribute__((aligned(16))) uint8_t stage[G::kStageBytes];
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    const int qg = blockIdx.x, kg = blockIdx.y, bh = blockIdx.z;
    const uint8_t* qbase = (const uint8_t*)q + (int64_t)bh * Lqp * D;
    const uint8_t* kbase = (const uint8_t*)k + (int64_t)bh * Lkp * D + (int64_t)k0 * D;
    // stage K rows [k0 + kBN kg, +kBN); the V part of the stage is not used
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)nk * D);
    TileDma<D, false, 1>::issue(stage, krs, krs, krs, 0, kg, 0, lane, false);
    wait_dma();
    __syncthreads();
    QFrag<D, false> qf;
    load_qfrag<D, false>(qf, qbase, nullptr, q0 + 32 * qg + col, lane);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        const v16i s = qk_subtile_i8<D>(stage, qf, t, lane);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kBN * kg + 32 * t + 16 * half + e;   // relative to k0
            const int qq = 32 * qg + col;                         // relative to q0
            out[((int64_t)bh * nq + qq) * nk + key] = s[e];
        }
    }
}

// Test hook: fp32 S = Q K^T of MXFP4 codes (E2M1 with E8M0 block scales),
// through the same staging and qk_subtile_mx as the attention kernel.
template <int D>
__global__ __launch_bounds__(64) void k_debug_qk_mx(const uint8_t* q, const uint8_t* qs, const uint8_t* k,
                                                    const uint8_t* ks, int Lqp, int Lkp, int q0, int k0,
                                                    int nq, int nk, float* out) {
    using G = Geo<D, true>;
    __shared__ __attribute__((aligned(16))) uint8_t stage[G::kStageBytes];
    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    const int qg = blockIdx.x, kg = blockIdx.y, bh = blockIdx.z;
    const uint8_t* qbase = q + (int64_t)bh * Lqp * G::kRowBytes;
    const uint8_t* qsc = qs + (int64_t)bh * Lqp * (D / 32);
    const uint8_t* kbase = k + ((int64_t)bh * Lkp + k0) * G::kRowBytes;
    const uint8_t* ksc = ks + ((int64_t)bh * Lkp + k0) * (D / 32);
    // stage K rows [k0 + kBN kg, +kBN) and their scales; the V part is not used
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (int64_t)nk * G::kRowBytes);
    const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(ksc, (int64_t)nk * (D / 32));
    TileDma<D, true, 1>::issue(stage, krs, ksrs, krs, 0, kg, 0, lane, false);
    wait_dma();
    __syncthreads();
    QFrag<D, true> qf;
    load_qfrag<D, true>(qf, qbase, qsc, q0 + 32 * qg + col, lane);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        const v16f s = qk_subtile_mx<D>(stage, qf, t, lane);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kBN * kg + 32 * t + 16 * half + e;   // relative to k0
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
    const AttnKernelArgs k{a.q, a.q_scale, a.k, a.k_scale, a.v, a.v_scale, a.out, a.B, a.H, a.Hkv,
                           a.Lq, a.Lk, a.D, a.q_block, a.k_block, a.causal,
                           a.q_fused ? (a.qh.bf16 ? a.hmat_bf16 : a.hmat_f16) : nullptr, a.inv_sqrt_r};
    if (a.pingpong) {   // INT8, D 128 (checked by the caller)
        dim3 pgrid((unsigned)((nqb + 1) / 2 * a.B * a.H));
        if (a.q_fused)
            k_attn_fwd_pp_fused_q<<<pgrid, 64 * kPPWaves, 0, stream>>>(k, alpha, a.qh);
        else
            k_attn_fwd_pp<<<pgrid, 64 * kPPWaves, 0, stream>>>(k, alpha, a.qh);
        return hipGetLastError();
    }
    if (a.mxfp4) {
        if (a.q_fused)
            k_attn_fwd<128, true, true><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
        else
            k_attn_fwd<128, true><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
    } else if (a.D == 128) {
        if (a.q_fused)
            k_attn_fwd<128, false, true><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
        else
            k_attn_fwd<128, false><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
    } else {
        if (a.q_fused)
            k_attn_fwd<64, false, true><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
        else
            k_attn_fwd<64, false><<<grid, kThreads, 0, stream>>>(k, alpha, a.qh);
    }
    return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q, const int8_t* k, int B, int H, int Lqp, int Lkp,
                           int D, int q0, int nq, int k0, int nk, int32_t* out,
                           hipStream_t stream) {
    dim3 grid(nq / 32, nk / kBN, B * H);
    if (D == 128)
        k_debug_qk<128><<<grid, 64, 0, stream>>>(q, k, Lqp, Lkp, q0, k0, nq, nk, out);
    else
        k_debug_qk<64><<<grid, 64, 0, stream>>>(q, k, Lqp, Lkp, q0, k0, nq, nk, out);
    return hipGetLastError();
}

hipError_t launch_debug_qk_mx(const uint8_t* q, const uint8_t* q_scale, const uint8_t* k,
                              const uint8_t* k_scale, int B, int H, int Lqp, int Lkp, int q0, int nq,
                              int k0, int nk, float* out, hipStream_t stream) {
    dim3 grid(nq / 32, nk / kBN, B * H);
    k_debug_qk_mx<128><<<grid, 64, 0, stream>>>(q, q_scale, k, k_scale, Lqp, Lkp, q0, k0, nq, nk, out);
    return hipGetLastError();
}

}  // namespace sage

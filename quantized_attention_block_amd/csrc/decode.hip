// Paged decode over an FP8 e4m3 KV cache with split-KV partials and a merge,
// for gfx950.
//
// Source: ROCm/aiter pull request 7388 (FlyDSL pa_decode), sections Changes
// and "Batch-first plan grid removal": paged attention decode with an FP8 KV
// cache and per-token scales, MTP query tokens, GQA, sliding windows; the work
// is cut into 256-token window tiles, one task per tile; a reduce
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
// The block copies the tile's K rows and V^T rows global -> LDS with 16-byte
// buffer_load ... lds instructions whose buffer descriptor is the page (one
// page per instruction), right after two scalar round trips (context length,
// page ids), so the whole tile is in flight at once.  Wave w then owns query
// rows [16 w, +16) of the KV head for the whole tile: S^T on
// v_mfma_f32_16x16x128 (e4m3 x e4m3; the Q row is quantized in registers and
// is the B operand), with K rows fed in an order that leaves each lane 32
// consecutive keys of one query row per 128-key group, which is exactly the
// B operand layout of the PV product O^T = V^T P^T.  Row max and sum need
// only lane shuffles: no LDS round trip and one block barrier in total.
// Partials (m, l, O) go to the workspace; a second kernel merges them.
#include "sage_device.hpp"
#include "sage_launch.hpp"

#include <mutex>
#include <type_traits>

namespace sage {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;            // query rows per KV head (padded): 16 per wave
constexpr int kTile = kDecodeTile;   // 256 keys per split
constexpr int kD = 128;
constexpr float kLog2Fp8Max = 8.807354922057604f;   // log2(448)
// Partial row of one (sequence, KV head, split, query row): h[DD] as fp16,
// then m, l and vmax as fp32, then 4 pad bytes (DD = 128 for D <= 128, else
// 256).  h = O8 / (448 l) with O8 = sum P8 V8 (e4m3 codes): P8 <= 448 p and
// |V8| <= 448 give |h| <= 448, so the fp16 rounding is relative (2^-11)
// whatever the cache's scales; the split's output is h vmax.
__host__ __device__ constexpr int part_bytes(int DD) { return 2 * DD + 16; }

// Keeps the first n bytes of v (all for n >= 16, none for n <= 0), zeroes the rest.
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

// two fp32 -> fp16 (round to nearest even), x in the low half
__device__ __forceinline__ uint32_t pack_h2(float x, float y) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y) << 16);
}
__device__ __forceinline__ float2 unpack_h2(uint32_t w) {
    return make_float2((float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)),
                       (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)));
}

// LDS K tile [256 keys][128 B]: chunk c of key k is stored at chunk
// c ^ dk_swz(k).  One 16-lane read pass fetches keys {32 a + 4 m + b} (a, b in
// 0..3) at one chunk; the XOR puts the 8 keys of each parity on 8 distinct
// chunks, so the pass touches 16 distinct 16-byte bank groups.
__device__ __forceinline__ int dk_swz(int key) { return ((key >> 5) & 3) | (((key >> 1) & 1) << 2); }

// MX K tile [256 keys][64 B]: one read pass fetches keys {16 a + 4 m + b}
// (a, b in 0..3, see kx) at one of the 4 chunks; 4 rows share a bank sweep,
// and the XOR with key bits 4-5 (= a) separates the 4 sweeps.
__device__ __forceinline__ int dk_swz_mx(int key) { return (key >> 4) & 3; }

// Key (within a 128-key group) of element i of S^T MFMA m in lane group q4,
// which is also byte 4 m + i of that lane group's PV B operand.  e4m3:
// 32 q4 + 4 m + i.  MX: the block-scaled MFMA pairs nibble j of an E2M1
// operand's lane group G with byte b of an e4m3 operand's lane group G' where
// 32 G' + b = 64 (G & 1) + 32 (j / 16) + 16 (G >> 1) + j % 16 (measured on
// gfx950); for the E2M1 lane group q4 to hold the 32 consecutive keys (or
// channels) [32 q4, +32) of one MX block, e4m3 byte b of lane group q4 must
// hold 16 q4 + b (b < 16) or 64 + 16 q4 + b - 16 (b >= 16).
template <bool MX>
__device__ __forceinline__ int kx(int q4, int m, int i) {
    if constexpr (MX) return (m < 4 ? 16 * q4 + 4 * m : 64 + 16 * q4 + 4 * (m - 4)) + i;
    else return 32 * q4 + 4 * m + i;
}

// LDS V^T tile [page-block][128 d][PW keys], PW = min(page, 256), n = PW / 16
// chunks per row (n = 2^LGN): chunk c of row d is stored at c ^ dv_swz(d).
// One read pass fetches 16 consecutive rows at one chunk; 16 / n rows share a
// 256-byte bank sweep and the XOR separates the sweeps.
template <int LGN>
__device__ __forceinline__ int dv_swz(int d) { return (d >> (4 - LGN)) & ((1 << LGN) - 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* scalar_ptr(const T* p) {
    return (const __attribute__((address_space(4))) T*)p;
}

// Plain (not transposed) V tile [256 keys][128 B] per plane: chunk c of key
// k is stored at c ^ pv_swz(k).  PV reads it with ds_read_b64_tr_b8: in each
// 16-lane group, source lane 2 j + h points at key kb + j, channels
// [16 db + 8 h, +8); the transposing read hands output lane 8 h + i the
// bytes of channel 16 db + 8 h + i for keys kb .. kb + 7 (lane layout
// measured on gfx950), the A operand of O^T = V^T P^T.  A half-wave then
// reads 16 rows (two lane groups, 8 rows each) at one chunk; the XOR puts the
// 8 rows of each row parity on 8 distinct chunks.
__device__ __forceinline__ int pv_swz(int key) { return ((key >> 1) & 3) | (((key >> 5) & 1) << 2); }

__device__ __forceinline__ uint2 keep_bytes8(uint2 v, int n) {
    const uint32_t m0 = n >= 4 ? 0xFFFFFFFFu : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
    const int n1 = n - 4;
    const uint32_t m1 = n1 >= 4 ? 0xFFFFFFFFu : (n1 <= 0 ? 0u : (1u << (8 * n1)) - 1u);
    return make_uint2(v.x & m0, v.y & m1);
}

// PW: keys per page-block, min(page, 256) (a page of at most 256 keys divides
// 256; a larger page holds the whole tile at offset t0 % page).
// MX: MXFP4 cache (E2M1 codes two per byte, E8M0 scales per 32 channels of
// each K row and per 32 keys of each V^T row), QK and PV on the block-scaled
// MFMA with the cache's scales; otherwise e4m3 with per-token fp32 scales.
// DD: 128 (D 64 runs as 128 with zero channels) or 256 (e4m3 only): the
// channels are held as DD / 128 planes of 128, each with the D = 128 tile
// layouts, QK accumulating over the planes.
// VT: V cache transposed [P, Hkv, D, page] (the tile's V^T rows are copied as
// they are); otherwise plain [P, Hkv, page, D] (e4m3 only), copied like K and
// transposed by the LDS reads of PV.
template <int PW, bool MX, int DD, bool VT>
__global__ __launch_bounds__(kThreads) void k_paged_decode(DecodeArgs a, float alpha) {
    static_assert(!MX || PW >= 64, "MXFP4 pages of 64 keys or more");
    static_assert(!MX || (DD == 128 && VT), "MXFP4: D 128 and transposed V");
    constexpr int kPlanes = DD / 128;
    constexpr int kNpb = kTile / PW;                 // page-blocks per tile
    constexpr int kLgn = PW == 16 ? 0 : PW == 32 ? 1 : PW == 64 ? 2 : PW == 128 ? 3 : 4;   // log2(PW / 16)
    constexpr int kRowB = MX ? kD / 2 : kD;          // bytes of one K row (per plane)
    constexpr int kVLgn = MX ? kLgn - 1 : kLgn;      // log2 of 16-byte chunks per V^T row of a page-block
    constexpr int kPlaneB = kTile * kD;              // bytes of one plane of a tile
    // Every kernel argument the block uses is read at entry, in one batch:
    // left to itself the compiler loads the pointers only after the context
    // length has arrived, one more round trip before the tile copies start.
    asm volatile("" ::"s"(a.q), "s"(a.q_sB), "s"(a.q_sM), "s"(a.q_sH), "s"(a.k_cache), "s"(a.v_cache),
                 "s"(a.k_scale), "s"(a.v_scale), "s"(a.partials));
    // (split, sequence x KV head): the splits of a sequence are dispatched
    // together (numbering the blocks split-major, or the window's first tile
    // last, measured 1.4 us slower per call)
    const int s = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv, hk = bk % a.Hkv;
    // A page table of at most 64 pages per sequence is read whole, one entry
    // per lane, in flight together with the context length (the tile's pages
    // depend on it); longer tables are read after it.
    const bool row_in_lanes = a.max_pages <= 64;
    int prow = 0;
    if (row_in_lanes) {
        const int l = (int)(threadIdx.x & 63);
        prow = a.page_table[(int64_t)b * a.pt_stride + (l < a.max_pages ? l : 0)];
    }
    const int G = a.Hq / a.Hkv, R = a.MTP * G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15, q4 = lane >> 4;

    // ---- 1. this lane's Q slice of each plane: row r = 16 wave + c16,
    // channels [32 q4, +32); MX: [16 q4, +16) and [64 + 16 q4, +16) (the e4m3
    // operand's byte order that meets the E2M1 operand's, see kx).  In
    // flight with the context length; rows past R read row 0 of the head, in
    // bounds, and are zeroed below.  bf16 / fp16: 64 bytes per plane; e4m3:
    // the 32 code bytes in qraw[p][0..1].
    const int r = 16 * wave + c16;
    const int mt = (r < R ? r : 0) / G, gq = (r < R ? r : 0) % G;
    // the context length's scalar load goes out first: issued after the Q
    // loads, it waited for them, two memory latencies in a row
    const int ctx_raw = scalar_ptr(a.ctx_lens)[b];
    const int64_t qrow_idx = (int64_t)b * a.q_sB + (int64_t)mt * a.q_sM + (int64_t)(hk * G + gq) * a.q_sH;
    uint4 qraw[kPlanes][4];
    {
        const int c0 = MX ? 16 * q4 : 32 * q4, c1 = MX ? 64 + 16 * q4 : 32 * q4 + 16;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) {
            const int o0 = 128 * p + c0, o1 = 128 * p + c1;
            if (a.q_kind == kQueryE4M3) {
                const uint8_t* qp = (const uint8_t*)a.q + qrow_idx;
                const bool in = MX || o0 < a.D;
                qraw[p][0] = in ? *(const uint4*)(qp + o0) : make_uint4(0, 0, 0, 0);
                qraw[p][1] = in ? *(const uint4*)(qp + o1) : make_uint4(0, 0, 0, 0);
                qraw[p][2] = qraw[p][3] = make_uint4(0, 0, 0, 0);
            } else if (MX || o0 < a.D) {
                const uint16_t* qp = (const uint16_t*)a.q + qrow_idx;
                qraw[p][0] = *(const uint4*)(qp + o0);
                qraw[p][1] = *(const uint4*)(qp + o0 + 8);
                qraw[p][2] = *(const uint4*)(qp + o1);
                qraw[p][3] = *(const uint4*)(qp + o1 + 8);
            } else {   // D = 64: channels [64, 128) are zero
                qraw[p][0] = qraw[p][1] = qraw[p][2] = qraw[p][3] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    // e4m3 queries: the row's scale (one per tensor, or per (token, head) row)
    float qs_given = 0.0f;
    if (a.q_kind == kQueryE4M3) qs_given = a.q_scale[a.q_scale_per_tensor ? 0 : (int64_t)(b * a.MTP + mt) * a.Hq + hk * G + gq];
    // Both are awaited here, so the Q loads cannot be moved below the early
    // exits (after the length arrives).
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asm volatile("" : "+v"(qraw[p][i].x), "+v"(qraw[p][i].y), "+v"(qraw[p][i].z), "+v"(qraw[p][i].w)
                         : "s"(ctx_raw));

    // context lengths beyond max_ctx (which sizes the split plan) or beyond
    // what the page table covers are clamped to them
    const int ctx = min(min(ctx_raw, a.max_ctx), a.max_pages * a.page);
    if (ctx <= 0) return;
    const int lo_b = a.window > 0 ? max(0, ctx - a.MTP - a.window + 1) : 0;
    const int T = lo_b / kTile + s;
    if (T > (ctx - 1) / kTile) return;            // this sequence has fewer splits
    const int t0 = T * kTile, last = ctx - 1;
    // A 128-key half of the tile with no key in [lo_b, ctx) (the first tile
    // of a window, the last of a context) is not read from memory: its copies
    // take offsets past the page's resource, which land zeros in LDS (every
    // key of it is masked, and zero V codes keep P V finite).
    const bool live[2] = {t0 + kTile / 2 > lo_b, t0 + kTile / 2 < ctx};

    // K tile and V tile, kPlanes planes of [256 keys][128 B] (V^T: [page-block]
    // [128 d][PW keys]); MX uses the first half of each plane.  (Declared
    // with literal sizes in the branch of each plane count: a __shared__ size
    // that depends on the template arguments leaves this compiler's host-side
    // launch stubs undefined.)
    uint8_t* kt_s;
    uint8_t* vt_s;
    if constexpr (kPlanes == 2) {
        __shared__ __attribute__((aligned(16))) uint8_t kt2[2 * kTile * kD], vt2[2 * kTile * kD];
        kt_s = kt2;
        vt_s = vt2;
    } else {
        __shared__ __attribute__((aligned(16))) uint8_t kt1[kTile * kD], vt1[kTile * kD];
        kt_s = kt1;
        vt_s = vt1;
    }
    // per-token fp32 scales; MX: the E8M0 bytes ([key][D/32] and [page-block][d][PW/32])
    __shared__ __attribute__((aligned(16))) float kss[kTile], vss[kTile];

    // ---- 2. page ids of the tile's page-blocks (scalar loads, all in flight
    // at once).  Page-block i is page t0 / page + i; a block that starts past
    // the context uses the last token's page, so every copy below reads inside
    // a real page; page ids outside [0, num_pages) read page 0.
    const int koff = a.page > kTile ? t0 % a.page : 0;   // tile offset inside a large page
    const auto* ptab = scalar_ptr(a.page_table + (int64_t)b * a.pt_stride);
    const int p0 = __builtin_amdgcn_readfirstlane(t0 / a.page);
    const int pl = __builtin_amdgcn_readfirstlane(last / a.page);
    int pid[kNpb];
#pragma unroll
    for (int i = 0; i < kNpb; ++i)
        pid[i] = row_in_lanes ? __builtin_amdgcn_readlane(prow, min(p0 + i, pl)) : ptab[min(p0 + i, pl)];
#pragma unroll
    for (int i = 0; i < kNpb; ++i) pid[i] = (unsigned)pid[i] < (unsigned)a.num_pages ? pid[i] : 0;

    // per-token scales of key t0 + tid (issued before the copies); MX: the
    // four E8M0 bytes of K row t0 + tid, and dword tid of the tile's V^T
    // scale bytes laid out [page-block][d][PW / 32]
    float ks, vs;
    {
        const int pbs = tid / PW;
        int pg = pid[0];
#pragma unroll
        for (int i = 1; i < kNpb; ++i) pg = pbs == i ? pid[i] : pg;
        const int64_t ph = (int64_t)pg * a.Hkv + hk;
        const int64_t o = ph * a.page + (koff + tid % PW);
        if constexpr (MX) {
            ks = __builtin_bit_cast(float, ((const uint32_t*)a.k_scale)[o]);
            const int wb = 4 * (tid % PW);                     // byte of the page-block's [d][PW / 32]
            const int d = wb / (PW / 32), col = wb % (PW / 32);
            const uint8_t* vsb = (const uint8_t*)a.v_scale + ph * kD * (a.page / 32);
            vs = __builtin_bit_cast(float, *(const uint32_t*)(vsb + d * (a.page / 32) + koff / 32 + col));
        } else {
            ks = a.k_scale[a.scale_per_tensor ? 0 : o];   // one scale for the whole cache, or per token
            vs = a.v_scale[a.scale_per_tensor ? 0 : o];
        }
    }

    // ---- 3. tile copies, per plane 8 K and 8 V instructions per wave, 1 KB
    // each (MX: 4 and 4).  Instruction i = wave + 4 j fills LDS chunks
    // [64 i, +64) of a plane; the K plane (and a plain V plane) holds keys
    // [8 i, +8), in page-block 8 i / PW: a constant for PW >= 32, and
    // 2 j + wave / 2 for 16-key pages (a wave-uniform choice between two page
    // ids).  A V^T plane holds 128 n chunks per page-block (n = PW / 16 chunks
    // per row; MX: PW / 32).  Channels at or past D (D = 64, and for every
    // copy whose plane lies past D) get offsets past the page's resource,
    // which reads as zeros.
    const int kpage = a.page * (MX ? kRowB : a.D);   // bytes of one page of one KV head
    if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = wave + 4 * j;
            // K keys [16 i, +16) (and a V^T page-block of at most 128 keys)
            // lie in half j / 2; a 256-key V^T page-block spans both
            const bool k_live = live[j >> 1], v_live = PW == 256 ? (live[0] || live[1]) : k_live;
            const int pg = pid[j >> (kLgn - 2)];   // page-block 16 i / PW (PW >= 64)
            // K: keys [16 i, +16) of the tile, 4 chunks each
            const __amdgpu_buffer_rsrc_t kr = page_rsrc(a.k_cache + ((int64_t)pg * a.Hkv + hk) * kpage, kpage);
            const int key = 16 * i + (lane >> 2);
            const int kc = (lane & 3) ^ dk_swz_mx(key);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kt_s + 1024 * i, 16,
                                                     k_live ? (koff + key % PW) * kRowB + 16 * kc : kpage, 0, 0, 0);
            // V^T: rows d of page-block (i >> (log2 n + 1)), chunks c
            const int within = ((64 * i) & ((128 << kVLgn) - 1)) + lane;
            const int d = within >> kVLgn, c = (within & ((1 << kVLgn) - 1)) ^ dv_swz<kVLgn>(d);
            const __amdgpu_buffer_rsrc_t vr = page_rsrc(a.v_cache + ((int64_t)pg * a.Hkv + hk) * kpage, kpage);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vt_s + 1024 * i, 16,
                                                     v_live ? d * (a.page / 2) + koff / 2 + 16 * c : kpage, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = wave + 4 * j;
            // keys [8 i, +8) of K (and of a plain V, and of a V^T page-block of
            // at most 128 keys) lie in half j / 4; a 256-key V^T page-block
            // spans both, copied when either is live
            const bool k_live = live[j >> 2], v_live = PW == 256 ? (live[0] || live[1]) : k_live;
            int pg;
            if constexpr (PW == 16) pg = (wave & 2) ? pid[2 * j + 1] : pid[2 * j];
            else pg = pid[j >> (kLgn - 1)];
            // K: keys [8 i, +8) of the tile, channels [128 p, +128)
            const __amdgpu_buffer_rsrc_t kr = page_rsrc(a.k_cache + ((int64_t)pg * a.Hkv + hk) * kpage, kpage);
            const int key = 8 * i + (lane >> 3);
            const int kc = (lane & 7) ^ dk_swz(key);
            const int kch = 128 * p + 16 * kc;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kt_s + p * kPlaneB + 1024 * i, 16,
                                                     k_live && kch < a.D ? (koff + key % PW) * a.D + kch : kpage,
                                                     0, 0, 0);
            const __amdgpu_buffer_rsrc_t vr = page_rsrc(a.v_cache + ((int64_t)pg * a.Hkv + hk) * kpage, kpage);
            if constexpr (VT) {
                // V^T: rows d of page-block (j >> kShift), chunks c
                const int within = ((64 * i) & ((128 << kLgn) - 1)) + lane;
                const int d = within >> kLgn, c = (within & ((1 << kLgn) - 1)) ^ dv_swz<kLgn>(d);
                const int dg = 128 * p + d;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vt_s + p * kPlaneB + 1024 * i, 16,
                                                         v_live && dg < a.D ? dg * a.page + koff + 16 * c : kpage,
                                                         0, 0, 0);
            } else {
                // plain V: laid out like K, with the PV read swizzle
                const int vc = (lane & 7) ^ pv_swz(key);
                const int vch = 128 * p + 16 * vc;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vt_s + p * kPlaneB + 1024 * i, 16,
                                                         v_live && vch < a.D ? (koff + key % PW) * a.D + vch : kpage,
                                                         0, 0, 0);
            }
        }
    }
    // keep the Q arithmetic below (which waits for the Q loads) from being
    // scheduled in between the copy instructions
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. Q row -> e4m3 with a per-row scale (the B operand of QK), or the
    // given e4m3 codes and scale.  A negative given scale is moved into the
    // codes' signs, so the row's score factor below is never negative.
    v8i qf[kPlanes];
    float qs;
    if (a.q_kind == kQueryE4M3) {
        const uint32_t flip = r < R && qs_given < 0.0f ? 0x80808080u : 0u;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) {
            const uint4 lo = r < R ? qraw[p][0] : make_uint4(0, 0, 0, 0);
            const uint4 hi = r < R ? qraw[p][1] : make_uint4(0, 0, 0, 0);
            qf[p] = v8i{(int)(lo.x ^ flip), (int)(lo.y ^ flip), (int)(lo.z ^ flip), (int)(lo.w ^ flip),
                        (int)(hi.x ^ flip), (int)(hi.y ^ flip), (int)(hi.z ^ flip), (int)(hi.w ^ flip)};
        }
        qs = r < R ? fabsf(qs_given) : 0.0f;
    } else {
        const bool f16 = a.q_kind == kQueryF16;
        float x[kPlanes][32];
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w[4] = {qraw[p][i].x, qraw[p][i].y, qraw[p][i].z, qraw[p][i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float v0 = f16 ? f16_bits_to_f32(w[k] & 0xFFFF) : bf16_bits_to_f32(w[k] & 0xFFFF);
                    const float v1 = f16 ? f16_bits_to_f32(w[k] >> 16) : bf16_bits_to_f32(w[k] >> 16);
                    x[p][8 * i + 2 * k] = r < R ? v0 : 0.0f;
                    x[p][8 * i + 2 * k + 1] = r < R ? v1 : 0.0f;
                }
            }
        float am = 0.0f;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
            for (int k = 0; k < 32; ++k) am = fmaxf(am, fabsf(x[p][k]));
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        const float inv = am > 0.0f ? kFp8Max / am : 0.0f;
#pragma unroll
        for (int p = 0; p < kPlanes; ++p)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                uint32_t c0 = cvt_pk_fp8<false>(x[p][4 * w] * inv, x[p][4 * w + 1] * inv, 0);
                qf[p][w] = (int)cvt_pk_fp8<true>(x[p][4 * w + 2] * inv, x[p][4 * w + 3] * inv, c0);
            }
        qs = am / kFp8Max;
    }

    const int kpos_s = t0 + tid;
    if constexpr (MX) {   // E8M0 bytes as loaded (K rows past ctx are masked later)
        kss[tid] = ks;
        vss[tid] = vs;
    } else {
        kss[tid] = kpos_s < ctx ? ks * alpha : 0.0f;   // alpha = sm_scale log2(e) folded in
        vss[tid] = kpos_s < ctx ? vs : 0.0f;
    }
    __syncthreads();   // every wave's copies have landed (vmcnt(0)) and the scales are in LDS

    // the tile's largest V scale over keys inside [lo_b, ctx); MX: the largest
    // V^T block exponent em of blocks that start before ctx (it bounds |V|)
    float vmax;
    int em = 0;
    if constexpr (MX) {
        const uint4 w4 = *(const uint4*)((const uint8_t*)vss + 16 * lane);
        const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int bi = 16 * lane + i;                       // byte of [page-block][d][PW / 32]
            const int pb = bi / (kD * (PW / 32)), col = bi % (PW / 32);
            const int e = (int)((wv[i / 4] >> (8 * (i % 4))) & 0xFFu);
            em = t0 + pb * PW + 32 * col < ctx ? max(em, e) : em;
        }
        em = (int)wave_max((float)em);
        vmax = __builtin_ldexpf(1.0f, em - 127);
    } else {
        const float4 v4 = *(const float4*)&vss[4 * lane];
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
        float vm = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kp = t0 + 4 * lane + i;
            vm = fmaxf(vm, (kp >= lo_b && kp < ctx) ? vv[i] : 0.0f);
        }
        vmax = wave_max(vm);
    }

    // ---- 5. S^T for 256 keys x this wave's 16 rows: MFMA (g, m) holds, in
    // element i of lane l, key 128 g + 32 (l / 16) + 4 m + i of query row r
    // (summed over the planes).
    v4f S[2][8];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int key = 128 * g + kx<MX>(c16 >> 2, m, c16 & 3);   // A row c16
            if constexpr (MX) {
                // channels [32 q4, +32) of K row key: 16 bytes of E2M1 and the
                // row's E8M0 byte for that block
                const v4i k4 = *(const v4i*)(kt_s + key * kRowB + 16 * (q4 ^ dk_swz_mx(key)));
                const int sk = (int)((const uint8_t*)kss)[4 * key + q4];
                S[g][m] = mfma_f4f8_16x16x128(__builtin_shufflevector(k4, k4, 0, 1, 2, 3, -1, -1, -1, -1), qf[0],
                                              v4f{0.0f, 0.0f, 0.0f, 0.0f}, sk);
            } else {
                const int sw = dk_swz(key);
                v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int p = 0; p < kPlanes; ++p) {
                    const uint8_t* krow = kt_s + p * kPlaneB + key * kD;
                    const v4i lo = *(const v4i*)(krow + 16 * ((2 * q4) ^ sw));
                    const v4i hi = *(const v4i*)(krow + 16 * ((2 * q4 + 1) ^ sw));
                    acc = mfma_f8_16x16x128(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qf[p], acc);
                }
                S[g][m] = acc;
            }
        }

    // ---- 6. scores x = t c with t = S k_scale alpha (the K scale and alpha
    // are in kss; MX: t = S, the K scale is inside S) and the row factor
    // c = q_scale (MX: q_scale alpha), kept positive, so the row max of x is
    // c times that of t; masked keys get t = -inf.  Row max and sum over the
    // 4 lanes of the row.
    const int pos = ctx - a.MTP + mt;
    const int lo = a.window > 0 ? pos - a.window + 1 : 0;
    // (a zero row has t = 0 on every key: any c > 0 gives it x = 0, and
    // -inf * c stays -inf)
    const float cr = fmaxf(MX ? qs * alpha : qs, 1.0e-30f);
    // A tile whose every key is visible to every query row (all but the first
    // and last tiles of a window) skips the per-key mask; rows past R are
    // padding whose results are never stored.
    const bool all_vis = t0 + kTile - 1 <= ctx - a.MTP && (a.window <= 0 || t0 >= ctx - a.window);
    float rmax = -INFINITY;
    auto scores = [&](auto all_tag) {
        constexpr bool ALL = decltype(all_tag)::value;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int kl0 = 128 * g + 32 * q4;         // e4m3: key of element (m, i) = kl0 + 4 m + i
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                float kk[4] = {1.0f, 1.0f, 1.0f, 1.0f};   // MX: the K scale is inside S
                if constexpr (!MX) {
                    const float4 k4 = *(const float4*)&kss[kl0 + 4 * m];
                    kk[0] = k4.x, kk[1] = k4.y, kk[2] = k4.z, kk[3] = k4.w;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv = MX ? S[g][m][i] : S[g][m][i] * kk[i];
                    if constexpr (ALL) {
                        S[g][m][i] = xv;
                    } else {
                        const int key = t0 + 128 * g + kx<MX>(q4, m, i);
                        const bool ok = r < R && key < ctx && key <= pos && key >= lo;
                        S[g][m][i] = ok ? xv : -INFINITY;
                    }
                    rmax = fmaxf(rmax, S[g][m][i]);
                }
            }
        }
    };
    if (all_vis)
        scores(std::true_type{});
    else
        scores(std::false_type{});
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    // the row max of x (-inf: no visible key in this tile)
    const float M = rmax == -INFINITY ? -INFINITY : rmax * cr;
    // p = 2^(x - M) and P' = p v_scale 448 / vmax -> e4m3 (MX: 448 p), packed
    // as the B operand of PV (byte 4 m + i of group g = key kl0 + 4 m + i).
    // The constant factor 448 / vmax is folded into the exponent, u =
    // 2^(fma(t, c, -(M - log2(448 / vmax)))) = p 448 / vmax, so l = sum u
    // vmax / 448 (with vmax = 0 every P' is 0 and u = p).
    const float lp = MX ? kLog2Fp8Max : (vmax > 0.0f ? kLog2Fp8Max - __builtin_amdgcn_logf(vmax) : 0.0f);
    const float Mo = (rmax == -INFINITY ? 0.0f : M) - lp;
    float ls = 0.0f;
    v8i pf[2];
    auto probs = [&](int g) {
        const int kl0 = 128 * g + 32 * q4;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            float vv[4] = {1.0f, 1.0f, 1.0f, 1.0f};   // MX: V's scales are in the MFMA
            if constexpr (!MX) {
                const float4 v4 = *(const float4*)&vss[kl0 + 4 * m];
                vv[0] = v4.x, vv[1] = v4.y, vv[2] = v4.z, vv[3] = v4.w;
            }
            float pp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = __builtin_amdgcn_exp2f(__builtin_fmaf(S[g][m][i], cr, -Mo));
                ls += u;
                pp[i] = MX ? u : u * vv[i];
            }
            const uint32_t c0 = cvt_pk_fp8<false>(pp[0], pp[1], 0);
            pf[g][m] = (int)cvt_pk_fp8<true>(pp[2], pp[3], c0);
        }
    };
    // ---- 7. O^T = V^T P^T: element i of lane l of d-block db is channel
    // 16 db + 4 (l / 16) + i of query row r
    constexpr int kDB = 8 * kPlanes;
    const bool all_in = t0 + kTile <= ctx;   // no page slot past the context in this tile
    v4f O[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) O[db] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto pv = [&](int g) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int p = db / 8, dl = 16 * (db % 8) + c16;   // plane, channel within the plane
            const uint8_t* vplane = vt_s + p * kPlaneB;
            const int k0 = 128 * g + 32 * q4;                // tile-relative first key of this lane's 32
            if constexpr (MX) {
                // 16 bytes of V^T row d (keys [k0, +32), E2M1; any finite
                // value past ctx meets P = 0) and that block's E8M0 byte; a
                // block wholly past ctx may hold an unwritten scale (E8M0 255
                // is NaN), so it gets 2^0
                const int d = dl;
                const int pb = k0 / PW, c = (k0 % PW) / 32;
                const uint8_t* vrow = vt_s + (pb * 128 + d) * (PW / 2);
                const v4i v4 = *(const v4i*)(vrow + 16 * (c ^ dv_swz<kVLgn>(d)));
                int sv = (int)((const uint8_t*)vss)[(pb * 128 + d) * (PW / 32) + c];
                if (!all_in && t0 + k0 >= ctx) sv = 127;
                O[db] = mfma_f4f8_16x16x128(__builtin_shufflevector(v4, v4, 0, 1, 2, 3, -1, -1, -1, -1), pf[g],
                                            O[db], sv);
                continue;
            }
            // keys at or beyond ctx may hold any bytes (e4m3 NaN codes
            // included) and 0 * NaN would poison the product: zero them
            v8i av;
            if constexpr (VT) {
                const int d = dl;
                const int sw = dv_swz<kLgn>(d);
                const int pb = k0 / PW, c = (k0 % PW) / 16;
                const uint8_t* vrow = vplane + (pb * 128 + d) * PW;
                // keys [k0 + 16, +16): the next chunk of the row, or with 16-key
                // pages the row of the next page-block
                const uint8_t* vrow_hi = PW == 16 ? vrow + 128 * PW : vrow;
                const int c_hi = PW == 16 ? 0 : c + 1;
                uint4 lo4 = *(const uint4*)(vrow + 16 * (c ^ sw));
                uint4 hi4 = *(const uint4*)(vrow_hi + 16 * (c_hi ^ sw));
                if (!all_in) {
                    const int nv = ctx - (t0 + k0);
                    lo4 = keep_bytes(lo4, nv);
                    hi4 = keep_bytes(hi4, nv - 16);
                }
                av = v8i{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                         (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
            } else {
                // four transposing reads of 8 keys each (see pv_swz)
                const int sl = lane & 15;
                const int cb = 16 * (db % 8) + 8 * (sl & 1);   // channels of this source lane
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = k0 + 8 * rr + (sl >> 1);
                    const uint8_t* src = vplane + key * kD + 16 * ((cb >> 4) ^ pv_swz(key)) + (cb & 8);
                    const auto t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i*)(src));
                    uint2 u = make_uint2((uint32_t)t[0], (uint32_t)t[1]);
                    if (!all_in) u = keep_bytes8(u, ctx - (t0 + k0 + 8 * rr));
                    av[2 * rr] = (int)u.x;
                    av[2 * rr + 1] = (int)u.y;
                }
            }
            O[db] = mfma_f8_16x16x128(av, pf[g], O[db]);
        }
    };
    // The probabilities of key group g, then its PV products: group 1's exp2
    // work is issued after group 0's MFMAs, so the two overlap (the same
    // operations, and the same accumulation orders, as all probabilities
    // first; -0.5 % per call).
    probs(0);
    pv(0);
    probs(1);
    pv(1);
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    ls = MX ? ls / kFp8Max : (vmax > 0.0f ? (ls * vmax) / kFp8Max : ls);

    // An MFMA reads its operands from every lane, whatever the exec mask: the
    // PV products (and the P packing and V reads feeding them) must not be
    // moved into the r < R branch below, where the padding rows' lanes would
    // feed stale registers into the valid rows' channels.
#pragma unroll
    for (int db = 0; db < kDB; ++db) asm volatile("" : "+v"(O[db]));
    if (r < R) {
        const float hs = ls > 0.0f ? 1.0f / (kFp8Max * ls) : 0.0f;
        constexpr int kPB = 2 * DD + 16;
        uint8_t* prow = (uint8_t*)a.partials + (((int64_t)bk * a.num_splits + s) * kRows + r) * kPB;
        // MX: h = O / (448 l vmax) with vmax = 2^(em - 127) (|h| <= 6)
        auto hv = [&](float o) { return MX ? __builtin_ldexpf(o * hs, 127 - em) : o * hs; };
#pragma unroll
        for (int db = 0; db < kDB; ++db)
            if (16 * db < a.D)
                *(uint2*)(prow + 2 * (16 * db + 4 * q4)) =
                    make_uint2(pack_h2(hv(O[db][0]), hv(O[db][1])), pack_h2(hv(O[db][2]), hv(O[db][3])));
        if (q4 == 0) *(float4*)(prow + 2 * DD) = make_float4(M, ls, vmax, 0.0f);
    }
}

// Merge of the split partials of one (sequence, KV head, row): m* = max m_s,
// out = sum 2^(m_s - m*) l_s (h_s vmax_s) / sum 2^(m_s - m*) l_s (fp32, split
// order), bf16 or fp16; l_s h_s vmax_s is the split's O_s.
// One wave per row; the weights are broadcast and every lane merges DD / 64
// output channels over all splits with coalesced loads.
constexpr int kMergeRowsPerBlock = 4;
constexpr int kMergeBatch = 32;

template <int DD>
__global__ __launch_bounds__(64 * kMergeRowsPerBlock) void k_decode_merge(DecodeArgs a) {
    constexpr int kCh = DD / 64;                  // channels per lane: 2 or 4
    using Word = typename std::conditional<kCh == 2, uint32_t, uint2>::type;
    constexpr int kPB = part_bytes(DD);
    const int lane = threadIdx.x & 63;
    // (the row is the wave's: read into a scalar register, the split count
    // and every per-split condition below are scalar too)
    const int rowg = __builtin_amdgcn_readfirstlane(blockIdx.x * kMergeRowsPerBlock + (threadIdx.x >> 6));
    const int R = a.MTP * (a.Hq / a.Hkv);
    const int bk = rowg / kRows, r = rowg % kRows;
    if (bk >= a.B * a.Hkv || r >= R) return;
    const int b = bk / a.Hkv, hk = bk % a.Hkv;
    const int ctx_raw = a.ctx_lens[b];
    const int G = a.Hq / a.Hkv;
    const uint8_t* base = (const uint8_t*)a.partials + ((int64_t)bk * a.num_splits * kRows + r) * kPB;
    const int64_t sstride = (int64_t)kRows * kPB;
    // The first batch's loads go out together with the context length's,
    // for every allocated split (rows of splits this sequence does not have
    // are read but never used), instead of waiting for the split count.
    // (Split indexes are clamped to the allocated ones rather than guarded:
    // guarded loads become branches that the compiler waits on one by one.)
    const int na = min(kMergeBatch, a.num_splits);
    const float4 ml_first = *(const float4*)(base + min(lane, na - 1) * sstride + 2 * DD);
    Word o_first[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
        o_first[u] = *(const Word*)(base + min(u, na - 1) * sstride + sizeof(Word) * lane);
    const int ctx = min(min(ctx_raw, a.max_ctx), a.max_pages * a.page);   // as in k_paged_decode
    const int lo_b = a.window > 0 ? max(0, ctx - a.MTP - a.window + 1) : 0;
    const int nsp = ctx > 0 ? (ctx - 1) / kTile - lo_b / kTile + 1 : 0;
    // Splits are taken kMergeBatch at a time with every load of a batch in
    // flight at once: lane s holds split s's (m, l), every lane kCh output
    // channels of each split.  With at most kMergeBatch splits this is the
    // plain two-step merge; longer contexts carry a running max across
    // batches and rescale the running sums.
    float M = -INFINITY, L = 0.0f, o[kCh] = {};
    for (int s0 = 0; s0 < nsp; s0 += kMergeBatch) {
        const int n = min(kMergeBatch, nsp - s0);
        float4 ml = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);   // m, l, vmax
        Word w[kMergeBatch];
        if (s0 == 0) {
            if (lane < n) ml = ml_first;
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) w[u] = o_first[u];
        } else {
            if (lane < n) ml = *(const float4*)(base + (s0 + lane) * sstride + 2 * DD);
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u)
                w[u] = u < n ? *(const Word*)(base + (s0 + u) * sstride + sizeof(Word) * lane) : Word{};
        }
        const float Mn = fmaxf(M, wave_max(ml.x));
        if (Mn == -INFINITY) continue;               // no visible key so far
        if (M != -INFINITY && M != Mn) {
            const float sc = __builtin_amdgcn_exp2f(M - Mn);
            L *= sc;
#pragma unroll
            for (int c = 0; c < kCh; ++c) o[c] *= sc;
        }
        M = Mn;
        const float wgt = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);
        const float lw = wgt * ml.y;
        const float ow = lw * ml.z;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (u < n) {
                // lane u's weights, read into scalar registers (u is a
                // constant once unrolled: no LDS round trip per split)
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ow), u));
                L = L + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lw), u));
                const uint32_t* hw = (const uint32_t*)&w[u];
#pragma unroll
                for (int c = 0; c < kCh / 2; ++c) {
                    const float2 h = unpack_h2(hw[c]);
                    o[2 * c] = o[2 * c] + wj * h.x;
                    o[2 * c + 1] = o[2 * c + 1] + wj * h.y;
                }
            }
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int mt = r / G, g = r % G;
    uint16_t* op = (uint16_t*)a.out + (int64_t)b * a.o_sB + (int64_t)mt * a.o_sM +
                   (int64_t)(hk * G + g) * a.o_sH + kCh * lane;
    if (kCh * lane < a.D) {
        uint32_t ow[kCh / 2];
#pragma unroll
        for (int c = 0; c < kCh / 2; ++c)
            ow[c] = a.out_f16 ? pack_h2(o[2 * c] * inv, o[2 * c + 1] * inv)
                              : (uint32_t)f32_to_bf16_bits(o[2 * c] * inv) |
                                    ((uint32_t)f32_to_bf16_bits(o[2 * c + 1] * inv) << 16);
        if constexpr (kCh == 2)
            *(uint32_t*)op = ow[0];
        else
            *(uint2*)op = make_uint2(ow[0], ow[1]);
    }
}

}  // namespace

// Scratch of the no-allocation decode entry point: the split partials, which
// the allocating entry point keeps in the caller's workspace.  One copy per
// device, held until the process ends; every call on a device shares it.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    // Device address of this device's copy of `scratch`, looked up once per
    // device (with that device current) and kept; the array's name in host
    // code is only a host-side stand-in and is never passed to a kernel.
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    const float alpha = a.sm_scale * kLog2e;
    const dim3 grid(a.num_splits, a.B * a.Hkv);
    const int pw = a.page < kTile ? a.page : kTile;
    if (a.mx) {
        switch (pw) {
            case 64: k_paged_decode<64, true, 128, true><<<grid, kThreads, 0, stream>>>(a, alpha); break;
            case 128: k_paged_decode<128, true, 128, true><<<grid, kThreads, 0, stream>>>(a, alpha); break;
            default: k_paged_decode<256, true, 128, true><<<grid, kThreads, 0, stream>>>(a, alpha); break;
        }
    } else {
        // e4m3 cache: page-block width x head dim (128, or 256) x V layout
        auto go = [&](auto pw_tag) {
            constexpr int PW = decltype(pw_tag)::value;
            if (a.D > 128) {
                if (a.v_transposed) k_paged_decode<PW, false, 256, true><<<grid, kThreads, 0, stream>>>(a, alpha);
                else k_paged_decode<PW, false, 256, false><<<grid, kThreads, 0, stream>>>(a, alpha);
            } else {
                if (a.v_transposed) k_paged_decode<PW, false, 128, true><<<grid, kThreads, 0, stream>>>(a, alpha);
                else k_paged_decode<PW, false, 128, false><<<grid, kThreads, 0, stream>>>(a, alpha);
            }
        };
        switch (pw) {
            case 16: go(std::integral_constant<int, 16>{}); break;
            case 32: go(std::integral_constant<int, 32>{}); break;
            case 64: go(std::integral_constant<int, 64>{}); break;
            case 128: go(std::integral_constant<int, 128>{}); break;
            default: go(std::integral_constant<int, 256>{}); break;
        }
    }
    const int rows = a.B * a.Hkv * kRows;
    const int mblocks = (rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock;
    if (a.D > 128)
        k_decode_merge<256><<<mblocks, 64 * kMergeRowsPerBlock, 0, stream>>>(a);
    else
        k_decode_merge<128><<<mblocks, 64 * kMergeRowsPerBlock, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace sage

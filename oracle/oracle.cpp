// CPU oracle for SageAttention2-style quantized attention and FP8 paged decode.
//
// TEST INFRASTRUCTURE ONLY: the slow, plain reference the HIP path is checked
// against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
// load it; it shares nothing with the HIP library.  Build: plain C++17, -O2,
// -ffp-contract=off, no fast-math (every float operation below is one IEEE
// binary32 or binary64 operation, rounded to nearest even).
//
// Sources (the pages give names and hints, not formulas; every place where they
// leave a step open is marked READING and listed with the design notes):
//   [Sage2 README]  "Sage2 SM89 Temporal Pair Experiment" README, section
//                   Candidate: per-warp state RS / RS_f8 / RO / m / d and the
//                   per-KV-tile order QK -> update_mdo -> accumulate_d ->
//                   RS_32_to_8 -> PV; the kernel name says INT8 QK, FP8 "SV"
//                   and a fused V scale.
//   [aiter #7388]   ROCm/aiter pull request 7388 (FlyDSL pa_decode), sections
//                   Changes (FP8_MAX is the finfo max of the format Q and P are
//                   quantized to; the epilogue applies 1/FP8_MAX; OCP e4m3 on
//                   gfx950) and "Batch-first plan grid removal" (window tiles
//                   (window + 4 - 2 + 256 - 1)//256 + 1, one task per tile,
//                   decode and reduce timed together).
//   [xDiT #665]     xDiT pull request 665 "Sage v2 improvements": the Sage v2
//                   MXFP4 path applies a Hadamard matrix with BLOCK_R = 128,
//                   built once.
//   [OCP MX]        OCP Microscaling Formats v1.0 (E2M1, E8M0, shared exponent
//                   floor(log2 amax) - emax_elem) and OCP 8-bit floating point
//                   (E4M3: bias 7, max 448, no infinities) - public standards
//                   the pages name by their type names only.
//
// Parity pins live in tests/test_oracle_*.py; functions without an independent
// pin say "parity unpinned" below.

#include "oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

const double kLog2e = 1.4426950408889634073599246810019;  // log2(e)

// ---------------------------------------------------------------------------
// Rounding to a small binary floating-point format, from its definition.
//
// A format with `mant` explicit mantissa bits and smallest normal exponent
// `emin` represents, around |x| in [2^e, 2^(e+1)), multiples of the quantum
// 2^(max(e, emin) - mant).  Round-to-nearest-even picks the nearest multiple
// and, on a tie, the even multiple.  Values whose rounded magnitude exceeds
// `maxv` either saturate to maxv or become infinity.
// x must be finite.  All steps are exact in binary64 for the formats used
// (inputs are binary32).
double round_to_format(double x, int mant, int emin, double maxv, bool saturate) {
    if (x == 0.0) return x;
    double ax = std::fabs(x);
    int e2;
    std::frexp(ax, &e2);          // ax = f * 2^e2, f in [0.5, 1)
    int e = e2 - 1;               // ax in [2^e, 2^(e+1))
    int eq = std::max(e, emin) - mant;
    double r = std::ldexp(ax, -eq);          // exact scaling by a power of two
    double n = std::nearbyint(r);            // default mode: nearest, ties to even
    double v = std::ldexp(n, eq);
    if (v > maxv) v = saturate ? maxv : INFINITY;
    return std::copysign(v, x);
}

// OCP E4M3 ("float8_e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
// normals (1 + m/8) * 2^(e-7) for e = 1..15, subnormals (m/8) * 2^-6, largest
// finite value 448 (code 0x7E), 0x7F/0xFF are NaN, no infinities.
const int kE4M3Mant = 3, kE4M3Emin = -6;
const double kE4M3Max = 448.0;   // FP8_MAX of the OCP flavour [aiter #7388]
const float kFp8Max = 448.0f;     // the same value, the static scale of P

uint8_t e4m3_bits_of_value(double v) {   // v exactly representable, finite
    uint8_t s = std::signbit(v) ? 0x80 : 0x00;
    double a = std::fabs(v);
    if (a == 0.0) return s;
    if (a < std::ldexp(1.0, kE4M3Emin)) {               // subnormal: m * 2^-9
        return s | (uint8_t)std::lrint(std::ldexp(a, 9));
    }
    int e2;
    std::frexp(a, &e2);
    int e = e2 - 1;
    int m = (int)std::lrint((std::ldexp(a, -e) - 1.0) * 8.0);
    return s | (uint8_t)(((e + 7) << 3) | m);
}

// E2M1 (OCP MX FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; values
// 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
const int kE2M1Mant = 1, kE2M1Emin = 0;
const double kE2M1Max = 6.0;

uint8_t e2m1_bits_of_value(double v) {
    uint8_t s = std::signbit(v) ? 0x8 : 0x0;
    double a = std::fabs(v);
    if (a == 0.0) return s;
    if (a < 1.0) return s | (uint8_t)std::lrint(a * 2.0);  // subnormal 0.5
    int e2;
    std::frexp(a, &e2);
    int e = e2 - 1;
    int m = (int)std::lrint((std::ldexp(a, -e) - 1.0) * 2.0);
    return s | (uint8_t)(((e + 1) << 1) | m);
}

inline float f32(double x) { return (float)x; }

// exp2 evaluated in binary64 and rounded once to binary32.
inline float exp2_f32(float t) { return (float)std::exp2((double)t); }

template <class F>
void parallel_for(int64_t n, int nthreads, F&& body) {
    if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
    nthreads = (int)std::min<int64_t>(nthreads, std::max<int64_t>(n, 1));
    if (nthreads <= 1) {
        for (int64_t i = 0; i < n; ++i) body(i);
        return;
    }
    std::atomic<int64_t> next{0};
    std::vector<std::thread> ts;
    for (int t = 0; t < nthreads; ++t)
        ts.emplace_back([&] {
            for (int64_t i; (i = next.fetch_add(1)) < n;) body(i);
        });
    for (auto& t : ts) t.join();
}

inline int64_t idx4(int b, int h, int l, int d, int H, int L, int D) {
    return (((int64_t)b * H + h) * L + l) * D + d;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Number formats [OCP MX], [aiter #7388].  Pinned: exhaustive code round trip,
// ties-to-even on every midpoint, torch's float8_e4m3fn cast for |x| <= 464,
// brute-force nearest search for E2M1.
// READING (saturation): values beyond 448 (E4M3) or 6 (E2M1) saturate; the
// pages never overflow these formats on purpose (P <= 1 is scaled by 448).

uint8_t orc_e4m3_encode(float x) {
    if (std::isnan(x)) return 0x7F;
    if (std::isinf(x)) return x > 0 ? 0x7E : 0xFE;
    double v = round_to_format((double)x, kE4M3Mant, kE4M3Emin, kE4M3Max, true);
    return e4m3_bits_of_value(v);
}

float orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double a = (e == 0) ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -a : a);
}

uint8_t orc_e2m1_encode(float x) {
    if (std::isnan(x)) return 0x7;   // no NaN in E2M1: treat as +max (never produced)
    if (std::isinf(x)) return x > 0 ? 0x7 : 0xF;
    double v = round_to_format((double)x, kE2M1Mant, kE2M1Emin, kE2M1Max, true);
    return e2m1_bits_of_value(v);
}

float orc_e2m1_decode(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double a = (e == 0) ? 0.5 * m : std::ldexp(1.0 + m / 2.0, e - 1);
    return (float)(s ? -a : a);
}

// E8M0: 2^(code - 127), code 255 is NaN [OCP MX].
float orc_e8m0_decode(uint8_t c) {
    if (c == 0xFF) return NAN;
    return (float)std::ldexp(1.0, (int)c - 127);
}

// Shared MX block exponent: floor(log2(amax)) - 2, where 2 is the exponent of
// E2M1's largest normal (6 = 1.5 * 2^2) [OCP MX].  Read from the binary32 bits
// so that subnormal amax is exact; clamped to the E8M0 range [-127, 127].
// amax == 0 gives -127 (code 0).
int orc_mx_shared_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    uint32_t bits;
    std::memcpy(&bits, &amax, 4);
    int ef = (int)((bits >> 23) & 0xFF);
    int flog2;
    if (ef != 0) {
        flog2 = ef - 127;
    } else {                                  // subnormal: 2^-149 * mantissa
        uint32_t m = bits & 0x7FFFFF;
        int hb = 31 - __builtin_clz(m);
        flog2 = hb - 149;
    }
    int e = flog2 - 2;
    return std::min(127, std::max(-127, e));
}

// Round-to-nearest-even to bfloat16 (8 exponent, 7 mantissa bits) and to IEEE
// binary16, returned as bit patterns.  Overflow becomes infinity.
uint16_t orc_bf16_round(float x) {
    if (std::isnan(x)) return 0x7FC0;
    double v = std::isinf(x) ? (double)x
                             : round_to_format((double)x, 7, -126, 3.3895313892515355e38, false);
    float fv = (float)v;
    uint32_t bits;
    std::memcpy(&bits, &fv, 4);
    return (uint16_t)(bits >> 16);
}

uint16_t orc_fp16_round(float x) {
    if (std::isnan(x)) return 0x7E00;
    double v = std::isinf(x) ? (double)x : round_to_format((double)x, 10, -14, 65504.0, false);
    uint16_t s = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (std::isinf(a)) return s | 0x7C00;
    if (a == 0.0) return s;
    if (a < std::ldexp(1.0, -14)) return s | (uint16_t)std::lrint(std::ldexp(a, 24));
    int e2;
    std::frexp(a, &e2);
    int e = e2 - 1;
    int m = (int)std::lrint((std::ldexp(a, -e) - 1.0) * 1024.0);
    return s | (uint16_t)(((e + 15) << 10) | m);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}
void orc_e4m3_decode_array(const uint8_t* c, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

// ---------------------------------------------------------------------------
// Sylvester Hadamard matrix of order R (a power of two): H[i][j] =
// (-1)^popcount(i & j), entries +-1 [xDiT #665: BLOCK_R = 128, built once].
// Pinned: equals scipy.linalg.hadamard(R); H H^T = R I.
void orc_hadamard(int R, float* H) {
    for (int i = 0; i < R; ++i)
        for (int j = 0; j < R; ++j)
            H[(int64_t)i * R + j] = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------------------
// K smoothing (SageAttention2 method named on the pages; the pages do not spell
// it out).  READING: mu[b,h,d] is the mean of K over ALL Lk tokens, summed in
// binary64 in ascending token order, divided by Lk in binary64 and rounded once
// to binary32; K_s = fp32(K - mu).  Softmax is invariant to subtracting q.mu
// from every score of a row, so the reading does not change exact attention.
// Pinned: exact attention with K and with K - mu agree to 1e-12.
void orc_k_mean(const float* k, int B, int H, int L, int D, float* mu) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < D; ++d) {
                double s = 0.0;
                for (int j = 0; j < L; ++j) s += (double)k[idx4(b, h, j, d, H, L, D)];
                mu[((int64_t)b * H + h) * D + d] = L > 0 ? (float)(s / (double)L) : 0.0f;
            }
}

void orc_smooth_k(const float* k, const float* mu, int B, int H, int L, int D, float* ks) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int j = 0; j < L; ++j)
                for (int d = 0; d < D; ++d) {
                    int64_t o = idx4(b, h, j, d, H, L, D);
                    ks[o] = k[o] - mu[((int64_t)b * H + h) * D + d];
                }
}

// Symmetric INT8 block quantization (Q: 128-token blocks, K_s: 64-token blocks).
// READING: per (b, h, block of `block` tokens; the last block holds only the
// valid tokens): amax = max |x|; amax == 0 -> scale 0 and all codes 0; else
// inv = fp32(127 / amax), scale = fp32(amax / 127), code = clamp(rne(fp32(x *
// inv)), -127, 127).  Pinned: max |code| = 127 in every non-zero block,
// |x - code*scale| <= scale/2 (+ rounding slack), brute force on tiny blocks.
void orc_quant_int8(const float* x, int B, int H, int L, int D, int block,
                    int8_t* codes, float* scales) {
    int nb = (L + block - 1) / block;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int bi = 0; bi < nb; ++bi) {
                int j0 = bi * block, j1 = std::min(L, j0 + block);
                float amax = 0.0f;
                for (int j = j0; j < j1; ++j)
                    for (int d = 0; d < D; ++d)
                        amax = std::max(amax, std::fabs(x[idx4(b, h, j, d, H, L, D)]));
                float scale = 0.0f, inv = 0.0f;
                if (amax > 0.0f) {
                    inv = 127.0f / amax;
                    scale = amax / 127.0f;
                }
                scales[((int64_t)b * H + h) * nb + bi] = scale;
                for (int j = j0; j < j1; ++j)
                    for (int d = 0; d < D; ++d) {
                        int64_t o = idx4(b, h, j, d, H, L, D);
                        float y = x[o] * inv;
                        float r = std::nearbyint(y);
                        r = std::min(127.0f, std::max(-127.0f, r));
                        codes[o] = (int8_t)r;
                    }
            }
}

// V to FP8 e4m3 with a per-channel scale (the "fuse_v_scale" kernel of
// [Sage2 README] applies one scale per V channel in its epilogue).  READING:
// per (b, h, d): amax over all tokens; inv = fp32(448 / amax), scale =
// fp32(amax / 448), code = e4m3_rne_sat(fp32(v * inv)); amax == 0 -> scale 0,
// codes 0.  Pinned: codes decode within 2^-4 relative of v/scale (normals),
// max |decoded| = 448 per non-zero channel.
void orc_quant_v_fp8(const float* v, int B, int H, int L, int D, uint8_t* codes, float* scales) {
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < D; ++d) {
                float amax = 0.0f;
                for (int j = 0; j < L; ++j)
                    amax = std::max(amax, std::fabs(v[idx4(b, h, j, d, H, L, D)]));
                float inv = 0.0f, scale = 0.0f;
                if (amax > 0.0f) {
                    inv = 448.0f / amax;
                    scale = amax / 448.0f;
                }
                scales[((int64_t)b * H + h) * D + d] = scale;
                for (int j = 0; j < L; ++j) {
                    int64_t o = idx4(b, h, j, d, H, L, D);
                    codes[o] = orc_e4m3_encode(v[o] * inv);
                }
            }
}

// Hadamard rotation per R-channel block [xDiT #665].  READING: for every row
// and every block of R channels, y_j = sum_d x_d * H[d][j] computed exactly
// (binary64; the +-1 products are exact) and rounded once to binary32, then
// x'_j = fp32(y_j * r) with r = fp32(1 / sqrt(R)).  Pinned: H H^T = R I,
// rotation preserves norms and dot products within binary32 rounding, and
// rotating twice returns the input.
void orc_rotate(const float* x, int B, int H, int L, int D, int R, float* out) {
    std::vector<float> Hm((size_t)R * R);
    orc_hadamard(R, Hm.data());
    const float r = (float)(1.0 / std::sqrt((double)R));
    int64_t rows = (int64_t)B * H * L;
    for (int64_t row = 0; row < rows; ++row) {
        const float* xr = x + row * D;
        float* orow = out + row * D;
        for (int c0 = 0; c0 < D; c0 += R)
            for (int j = 0; j < R; ++j) {
                double y = 0.0;
                for (int d = 0; d < R; ++d) y += (double)xr[c0 + d] * (double)Hm[(size_t)d * R + j];
                orow[c0 + j] = (float)y * r;
            }
    }
}

// MXFP4 quantization of rows (OCP MX, block of 32 along D) [OCP MX],
// [xDiT #665: the Sage v2 MXFP4 path].  For each block: e = shared exponent of
// amax (orc_mx_shared_exponent), E8M0 code = e + 127, element codes =
// e2m1_rne_sat(x * 2^-e) (exact power-of-two scaling).
// Codes are returned one per byte; packing puts element 2i in the low nibble.
// Pinned: amax * 2^-e in [4, 8); brute force on tiny inputs.
// One element's code in a block whose shared exponent is e: E2M1 of x * 2^-e
// [OCP MX] (the scaling is exact in binary64; taking the value to binary32
// is exact too, except for magnitudes below 2^-126, which code to 0 either
// way).
uint8_t orc_e2m1_code_scaled(float x, int e) {
    double scaled = std::ldexp((double)x, -e);
    return orc_e2m1_encode((float)scaled);
}

void orc_e2m1_code_scaled_array(const float* x, int64_t n, int e, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_code_scaled(x[i], e);
}

void orc_quant_mxfp4(const float* x, int B, int H, int L, int D, uint8_t* codes, uint8_t* e8m0) {
    int64_t rows = (int64_t)B * H * L;
    int nblk = D / 32;
    for (int64_t row = 0; row < rows; ++row)
        for (int bl = 0; bl < nblk; ++bl) {
            const float* xb = x + row * D + bl * 32;
            float amax = 0.0f;
            for (int d = 0; d < 32; ++d) amax = std::max(amax, std::fabs(xb[d]));
            int e = orc_mx_shared_exponent(amax);
            e8m0[row * nblk + bl] = (uint8_t)(e + 127);
            for (int d = 0; d < 32; ++d) codes[row * D + bl * 32 + d] = orc_e2m1_code_scaled(xb[d], e);
        }
}

// Exact integer QK^T of INT8 codes over D channels.
int64_t orc_qk_int8_exact(const int8_t* q8, const int8_t* k8, int D) {
    int64_t s = 0;
    for (int d = 0; d < D; ++d) s += (int64_t)q8[d] * (int64_t)k8[d];
    return s;
}

// ---------------------------------------------------------------------------
// Quantized attention, emulated step by step.
//
// Per query row, KV tiles of BN keys are visited in ascending order; tiles whose
// every key is causally masked are skipped.  Per tile, in the order of
// [Sage2 README] (QK -> update_mdo -> accumulate_d -> RS_32_to_8 -> PV):
//   (a) S = exact integer q8 . k8 (INT8) or the MXFP4 block sum rounded once
//       to fp32;
//   (b) c = fp32(fp32(q_scale * k_scale) * alpha) (INT8) or c = alpha (MXFP4),
//       alpha = fp32(sm_scale * log2 e); the score x = fp32(float(S) * c);
//       masked keys get x = -inf;
//   (c) m_new = max(m, max_j x_j); a = exp2(m - m_new) (0 while m = -inf);
//       l = a * l; O = a * O (update_mdo);
//   (d) p_j = exp2(x_j - m_new); l += p_j in key order (accumulate_d, from the
//       fp32 probabilities, before their conversion);
//   (e) P8_j = e4m3(fp32(448 * p_j)) (RS_32_to_8: 448 = FP8_MAX, the largest
//       e4m3 value, scales P as in [aiter #7388] Changes; valid because
//       p_j <= 1);
//   (f) O[d] += fp32(sum_j dec(P8_j) * dec(V8[j, d])) with the tile's sum exact.
// Epilogue: out[d] = fp32(fp32(O[d] * v_scale[d]) / fp32(448 * l)) (the fused
// V scale, and the epilogue's 1/FP8_MAX of [aiter #7388]); l == 0 -> 0.
// READINGS: exp2 with log2(e) folded into alpha; exp2 is evaluated in binary64
// and rounded once; the tile length BN and the ascending order are part of the
// numeric definition (the running max decides how P is rounded), so the
// caller passes the kernel's BN.
// Pins: with quantization off (ORC_QK_FLOAT, quant_pv = 0: P and V stay fp32,
// out = O / l) it equals exact attention within 1e-6 and is invariant to BN;
// with V = 1 the output is the row sum of P8 / (448 l), which lies within the
// e4m3 rounding bound of 1; on inputs where every rounding step is exact
// (integer scores in log2 units within 15 of the row max, power-of-two or
// unit scales, codes equal to the values, K mean exactly 0) the quantized INT8
// and MXFP4 results equal base-2 attention on those scores, computed
// independently in float64 (a dropped rescale, 448 factor, scale, mask or V
// index each break it).

namespace {

struct EmulRow {
    const orc_attn_params& p;
    const orc_attn_inputs& in;
    float alpha;
    int nqb, nkb;
    const float* dec;   // e4m3 code -> value, tabulated from orc_e4m3_decode

    // Returns float(S) for key j of row i and sets *c to its scale (INT8:
    // fp32(q_scale * k_scale) * alpha; MXFP4: alpha; float mode: 1 with S
    // already scaled by sm_scale * log2 e).
    float score(int b, int h, int i, int j, float* c) const {
        const int D = p.D;
        if (p.qk_mode == ORC_QK_INT8) {
            const int8_t* qr = in.q8 + idx4(b, h, i, 0, p.H, p.Lq, D);
            const int8_t* kr = in.k8 + idx4(b, h, j, 0, p.H, p.Lk, D);
            int64_t S = orc_qk_int8_exact(qr, kr, D);
            float qs = in.q_scale[((int64_t)b * p.H + h) * nqb + i / p.q_block];
            float ks = in.k_scale[((int64_t)b * p.H + h) * nkb + j / p.k_block];
            *c = (qs * ks) * alpha;
            return (float)S;
        }
        if (p.qk_mode == ORC_QK_MXFP4) {
            const uint8_t* qr = in.q4 + idx4(b, h, i, 0, p.H, p.Lq, D);
            const uint8_t* kr = in.k4 + idx4(b, h, j, 0, p.H, p.Lk, D);
            const uint8_t* qe = in.q_e8 + idx4(b, h, i, 0, p.H, p.Lq, D / 32);
            const uint8_t* ke = in.k_e8 + idx4(b, h, j, 0, p.H, p.Lk, D / 32);
            double S = 0.0;
            for (int bl = 0; bl < D / 32; ++bl) {
                int64_t isum = 0;   // sum of (2 q)(2 k): E2M1 values are multiples of 0.5
                for (int d = bl * 32; d < bl * 32 + 32; ++d) {
                    int64_t a = (int64_t)std::lrint(2.0 * orc_e2m1_decode(qr[d]));
                    int64_t c2 = (int64_t)std::lrint(2.0 * orc_e2m1_decode(kr[d]));
                    isum += a * c2;
                }
                int ex = ((int)qe[bl] - 127) + ((int)ke[bl] - 127) - 2;
                S += std::ldexp((double)isum, ex);
            }
            *c = alpha;
            return (float)S;
        }
        const float* qr = in.qf + idx4(b, h, i, 0, p.H, p.Lq, D);
        const float* kr = in.kf + idx4(b, h, j, 0, p.H, p.Lk, D);
        double S = 0.0;
        for (int d = 0; d < D; ++d) S += (double)qr[d] * (double)kr[d];
        *c = 1.0f;
        return (float)(S * p.sm_scale * kLog2e);
    }

    void run(int b, int h, int i, float* out) const {
        const int D = p.D, BN = p.BN;
        float m = -INFINITY, l = 0.0f;
        std::vector<float> O(D, 0.0f), Sf(BN), cs(BN), pr(BN);
        std::vector<uint8_t> p8(BN), vis(BN);
        std::vector<double> acc(D);
        const int kend = p.causal ? std::min(p.Lk, i + 1) : p.Lk;
        for (int n0 = 0; n0 < kend; n0 += BN) {
            const int n1 = std::min(n0 + BN, p.Lk);
            const int nt = n1 - n0;
            float mt = -INFINITY;
            for (int t = 0; t < nt; ++t) {
                int j = n0 + t;
                vis[t] = !(p.causal && j > i);
                if (!vis[t]) continue;
                Sf[t] = score(b, h, i, j, &cs[t]);
                mt = std::max(mt, Sf[t] * cs[t]);          // x = fp32(S c)
            }
            const float m_new = std::max(m, mt);
            const float a = (m == -INFINITY) ? 0.0f : exp2_f32(m - m_new);
            l = a * l;
            for (int d = 0; d < D; ++d) O[d] = a * O[d];
            for (int t = 0; t < nt; ++t) {
                pr[t] = vis[t] ? exp2_f32(Sf[t] * cs[t] - m_new) : 0.0f;
                l = l + pr[t];
            }
            std::fill(acc.begin(), acc.end(), 0.0);
            if (p.quant_pv) {
                for (int t = 0; t < nt; ++t) p8[t] = orc_e4m3_encode(kFp8Max * pr[t]);
                for (int t = 0; t < nt; ++t) {
                    double pv = dec[p8[t]];
                    if (pv == 0.0) continue;
                    const uint8_t* vr = in.v8 + idx4(b, h, n0 + t, 0, p.H, p.Lk, D);
                    for (int d = 0; d < D; ++d) acc[d] += pv * (double)dec[vr[d]];
                }
            } else {
                for (int t = 0; t < nt; ++t) {
                    if (pr[t] == 0.0f) continue;
                    const float* vr = in.vf + idx4(b, h, n0 + t, 0, p.H, p.Lk, D);
                    for (int d = 0; d < D; ++d) acc[d] += (double)pr[t] * (double)vr[d];
                }
            }
            for (int d = 0; d < D; ++d) O[d] = O[d] + (float)acc[d];
            m = m_new;
        }
        for (int d = 0; d < D; ++d) {
            if (l == 0.0f) {
                out[d] = 0.0f;
            } else if (p.quant_pv) {
                float vs = in.v_scale[((int64_t)b * p.H + h) * D + d];
                out[d] = (O[d] * vs) / (kFp8Max * l);
            } else {
                out[d] = O[d] / l;
            }
        }
    }
};

}  // namespace

int orc_attn_emulated(const orc_attn_params* p, const orc_attn_inputs* in,
                      const int32_t* rows, int64_t nrows, float* out) {
    if (!p || !in || p->BN <= 0 || p->D <= 0) return -1;
    if (p->qk_mode == ORC_QK_MXFP4 && p->D % 32) return -1;
    float dec[256];
    for (int c = 0; c < 256; ++c) dec[c] = orc_e4m3_decode((uint8_t)c);
    EmulRow er{*p, *in, (float)(p->sm_scale * kLog2e),
               (p->Lq + p->q_block - 1) / std::max(1, p->q_block),
               (p->Lk + p->k_block - 1) / std::max(1, p->k_block), dec};
    int64_t n = rows ? nrows : (int64_t)p->B * p->H * p->Lq;
    parallel_for(n, p->nthreads, [&](int64_t r) {
        int b, h, i;
        if (rows) {
            b = rows[3 * r]; h = rows[3 * r + 1]; i = rows[3 * r + 2];
        } else {
            i = (int)(r % p->Lq); h = (int)((r / p->Lq) % p->H); b = (int)(r / ((int64_t)p->Lq * p->H));
        }
        er.run(b, h, i, out + r * p->D);
    });
    return 0;
}

// Exact softmax attention in binary64: out_i = sum_j w_ij v_j / sum_j w_ij,
// w_ij = exp(sm_scale * q_i . k_j - max_j), causal keeps j <= i.  This is the
// plain definition of the attention that the quantized method approximates.
// Pinned: torch scaled_dot_product_attention in float64; Lk = 1 -> V; Q = 0 ->
// (prefix) mean of V.
int orc_attn_exact(const float* q, const float* k, const float* v,
                   int B, int H, int Lq, int Lk, int D, int causal, double sm_scale,
                   const int32_t* rows, int64_t nrows, int nthreads, double* out) {
    int64_t n = rows ? nrows : (int64_t)B * H * Lq;
    parallel_for(n, nthreads, [&](int64_t r) {
        int b, h, i;
        if (rows) {
            b = rows[3 * r]; h = rows[3 * r + 1]; i = rows[3 * r + 2];
        } else {
            i = (int)(r % Lq); h = (int)((r / Lq) % H); b = (int)(r / ((int64_t)Lq * H));
        }
        const int kend = causal ? std::min(Lk, i + 1) : Lk;
        std::vector<double> s(std::max(kend, 1));
        double mx = -INFINITY;
        const float* qr = q + idx4(b, h, i, 0, H, Lq, D);
        for (int j = 0; j < kend; ++j) {
            const float* kr = k + idx4(b, h, j, 0, H, Lk, D);
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += (double)qr[d] * (double)kr[d];
            s[j] = acc * sm_scale;
            mx = std::max(mx, s[j]);
        }
        double den = 0.0;
        for (int j = 0; j < kend; ++j) { s[j] = std::exp(s[j] - mx); den += s[j]; }
        double* o = out + r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < kend; ++j) {
            const float* vr = v + idx4(b, h, j, 0, H, Lk, D);
            for (int d = 0; d < D; ++d) o[d] += s[j] * (double)vr[d];
        }
        for (int d = 0; d < D; ++d) o[d] = den > 0 ? o[d] / den : 0.0;
    });
    return 0;
}

// ---------------------------------------------------------------------------
// Paged decode with split-KV partials and a merge [aiter #7388].
//
// Query token m (0 .. MTP-1) of sequence b sits at position pos = ctx - MTP + m
// (READING: the MTP query tokens are the last positions of the context, causal
// among themselves).  With a sliding window W it sees keys [pos - W + 1, pos]
// (READING, consistent with the page's tile count: the union over the MTP
// tokens spans W + MTP - 1 keys, and (W + MTP - 1 - 1 + 255)//256 + 1 gives the
// page's 18 / 25 / 34 tiles for W = 4096 / 6000 / 8192).  Key t of sequence b
// lives in page page_table[b][t / page_size], slot t % page_size; query head
// hq reads KV head hq / (Hq / Hkv).
// Splits are `tile`-token windows aligned to absolute positions, one split per
// tile the sequence's window union touches (one task per window tile, as the
// "Batch-first plan grid removal" section describes the plan).
// Per split and query row:
//   quant: Q row -> e4m3 with a dynamic scale (quant_query_row), or the
//          e4m3 query as given (p->q8: codes and a per-row or per-tensor
//          scale; the page lists e4m3 queries beside bf16 ones);
//          x = fp32(fp32(fp32(dot * q_scale) * k_scale[t]) * alpha) where dot
//          is the exact e4m3 dot product rounded once;
//   float: x = fp32(sum_d q * k_cache * k_scale[t] in binary64 * sm_scale *
//          log2 e);
//   m_s = max x, p = exp2(x - m_s), l_s = sum p (fp32, key order);
//   quant: READING for the per-token V scale inside an FP8 PV: vmax = max of
//          v_scale over the split's keys inside [lo, ctx) (lo = first key of the
//          union window), p' = fp32(p * v_scale[t]), P8 = e4m3(fp32(p' *
//          fp32(448 / vmax))), O_s = fp32(fp32(sum P8 * V8 exact) *
//          fp32(vmax / 448));
//   float: O_s = fp32(sum p * v_cache * v_scale[t] in binary64).
// Merge: m* = max_s m_s, w_s = exp2(m_s - m*), out = sum w_s O_s / sum w_s l_s
// (fp32, split order); l == 0 -> 0.
// Pins: float mode equals exact attention of the last MTP rows; page
// permutation and split length do not change the float result; the split
// count formula reproduces the page's 18 / 25 / 34.  Quant mode: on inputs
// where every rounding is exact (integer scores, power-of-two token scales,
// e4m3-exact Q rows with a 448 and cache values) it equals base-2 attention
// over each query's window with the per-token V scale applied, computed
// independently in float64 (a wrong window bound, fold, score scale, merge
// weight or query position each break it).

namespace {
// The e4m3 query row r: given codes and scale (p->q8), or the float row
// quantized with a dynamic scale (READING: per (token, head) row, scale =
// fp32(amax / 448), codes e4m3(fp32(q * fp32(448 / amax))); the page says Q
// is quantized to the cache's FP8 format).
void quant_query_row(const orc_decode_params* p, const float* qr, int64_t r, uint8_t* q8, float* q_s) {
    const int D = p->D;
    if (p->q8) {
        for (int d = 0; d < D; ++d) q8[d] = p->q8[r * D + d];
        *q_s = p->q8_scale[p->q8_scale_per_tensor ? 0 : r];
        return;
    }
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) amax = std::max(amax, std::fabs(qr[d]));
    float inv = 0.0f;
    *q_s = 0.0f;
    if (amax > 0.0f) { inv = 448.0f / amax; *q_s = amax / 448.0f; }
    for (int d = 0; d < D; ++d) q8[d] = orc_e4m3_encode(qr[d] * inv);
}
}  // namespace

int orc_decode_num_splits(int window, int mtp, int tile) {
    // Largest number of tile-aligned windows that W + MTP - 1 consecutive keys
    // can touch.
    int span = window + mtp - 1;
    return (span - 1 + tile - 1) / tile + 1;
}

int orc_paged_decode(const orc_decode_params* p, const float* q,
                     const void* k_cache, const void* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* page_table, const int32_t* ctx_lens, float* out) {
    if (!p || p->Hkv <= 0 || p->Hq % p->Hkv || p->tile <= 0) return -1;
    const int D = p->D, PS = p->page_size;
    const float alpha = (float)(p->sm_scale * kLog2e);
    const int group = p->Hq / p->Hkv;
    int64_t nrows = (int64_t)p->B * p->MTP * p->Hq;
    float dec[256];
    for (int c = 0; c < 256; ++c) dec[c] = orc_e4m3_decode((uint8_t)c);
    std::atomic<int> bad{0};
    parallel_for(nrows, p->nthreads, [&](int64_t r) {
        const int hq = (int)(r % p->Hq);
        const int m = (int)((r / p->Hq) % p->MTP);
        const int b = (int)(r / ((int64_t)p->Hq * p->MTP));
        const int hk = hq / group;
        const int ctx = ctx_lens[b];
        const int pos = ctx - p->MTP + m;
        const int lo_row = p->window > 0 ? std::max(0, pos - p->window + 1) : 0;
        const int lo_b = p->window > 0 ? std::max(0, ctx - p->MTP - p->window + 1) : 0;
        const float* qr = q + r * D;
        float* o = out + r * D;

        auto slot = [&](int t, int64_t* base_row) -> bool {
            int pg = page_table[(int64_t)b * p->max_pages + t / PS];
            if (pg < 0 || pg >= p->num_pages) return false;
            *base_row = ((int64_t)pg * p->Hkv + hk) * PS + (t % PS);
            return true;
        };

        std::vector<uint8_t> q8(D);
        float q_s = 0.0f;
        if (p->quant) quant_query_row(p, qr, r, q8.data(), &q_s);

        std::vector<float> ms, ls;
        std::vector<std::vector<float>> Os;
        if (ctx > 0) {
            const int t_first = lo_b / p->tile, t_last = (ctx - 1) / p->tile;
            for (int T = t_first; T <= t_last; ++T) {
                const int k0 = std::max(T * p->tile, lo_b), k1 = std::min((T + 1) * p->tile, ctx);
                const int r0 = std::max(k0, lo_row), r1 = std::min(k1, pos + 1);
                std::vector<float> Osp(D, 0.0f);
                if (r0 >= r1) { ms.push_back(-INFINITY); ls.push_back(0.0f); Os.push_back(Osp); continue; }
                std::vector<float> x(r1 - r0), pr(r1 - r0);
                float mx = -INFINITY;
                for (int t = r0; t < r1; ++t) {
                    int64_t row;
                    if (!slot(t, &row)) { bad = 1; return; }
                    float xv;
                    if (p->quant) {
                        const uint8_t* kr = (const uint8_t*)k_cache + row * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += (double)dec[q8[d]] * (double)dec[kr[d]];
                        xv = (((float)dot * q_s) * k_scale[row]) * alpha;
                    } else {
                        const float* kr = (const float*)k_cache + row * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += (double)qr[d] * (double)kr[d] * (double)k_scale[row];
                        xv = (float)(dot * p->sm_scale * kLog2e);
                    }
                    x[t - r0] = xv;
                    mx = std::max(mx, xv);
                }
                float l = 0.0f;
                for (int t = r0; t < r1; ++t) {
                    pr[t - r0] = exp2_f32(x[t - r0] - mx);
                    l = l + pr[t - r0];
                }
                std::vector<double> acc(D, 0.0);
                if (p->quant) {
                    float vmax = 0.0f;
                    for (int t = k0; t < k1; ++t) {
                        int64_t row;
                        if (!slot(t, &row)) { bad = 1; return; }
                        vmax = std::max(vmax, v_scale[row]);
                    }
                    const float inv_v = vmax > 0.0f ? 448.0f / vmax : 0.0f;
                    const float back_v = vmax / 448.0f;
                    for (int t = r0; t < r1; ++t) {
                        int64_t row = 0;
                        slot(t, &row);
                        float pp = pr[t - r0] * v_scale[row];
                        double pv = dec[orc_e4m3_encode(pp * inv_v)];
                        if (pv == 0.0) continue;
                        const uint8_t* vr = (const uint8_t*)v_cache + row * D;
                        for (int d = 0; d < D; ++d) acc[d] += pv * (double)dec[vr[d]];
                    }
                    for (int d = 0; d < D; ++d) Osp[d] = (float)acc[d] * back_v;
                } else {
                    for (int t = r0; t < r1; ++t) {
                        int64_t row = 0;
                        slot(t, &row);
                        const float* vr = (const float*)v_cache + row * D;
                        for (int d = 0; d < D; ++d)
                            acc[d] += (double)pr[t - r0] * (double)vr[d] * (double)v_scale[row];
                    }
                    for (int d = 0; d < D; ++d) Osp[d] = (float)acc[d];
                }
                ms.push_back(mx); ls.push_back(l); Os.push_back(Osp);
            }
        }
        float mstar = -INFINITY;
        for (float v : ms) mstar = std::max(mstar, v);
        float L = 0.0f;
        std::vector<float> acc(D, 0.0f);
        for (size_t s = 0; s < ms.size(); ++s) {
            float w = (ms[s] == -INFINITY) ? 0.0f : exp2_f32(ms[s] - mstar);
            L = L + w * ls[s];
            for (int d = 0; d < D; ++d) acc[d] = acc[d] + w * Os[s][d];
        }
        for (int d = 0; d < D; ++d) o[d] = L > 0.0f ? acc[d] / L : 0.0f;
    });
    return bad ? -2 : 0;
}

// Paged decode over an MXFP4 KV cache ([aiter #7388] names pa_decode_mxfp4:
// E2M1 KV with E8M0 scales, e4m3 queries and P, FP8_MAX of E4M3).
// READING (the page fixes no layout): K keeps one E8M0 scale per 32 channels
// of each token (the QK reduction axis); V is stored transposed with one
// scale per 32 consecutive keys of each channel (the PV reduction axis), so
// each block scale multiplies a whole 32-term partial sum.  Per split and
// query row, with the fp8 path's window, split and merge:
//   Q -> e4m3 per (token, head) row as in orc_paged_decode;
//   dot = sum over 32-channel blocks of 2^(e_k - 127) * sum dec(Q8) e2m1(K)
//         (exact), x = fp32(fp32(fp32(dot) * q_scale) * alpha);
//   m_s = max x, p = exp2(x - m_s), l_s = sum p (fp32, key order);
//   P8 = e4m3(fp32(448 p));
//   O_s[d] = fp32(fp32(sum_t dec(P8_t) e2m1(V[d, t]) 2^(e_v[d, t/32] - 127))
//            * fp32(1/448)) with the split's sum exact.
// Pin: on caches whose dequantized values are e4m3 values, with unit
// per-token scales, it equals orc_paged_decode's quantized mode bit for bit.
int orc_paged_decode_mx(const orc_decode_params* p, const float* q,
                        const uint8_t* k_codes, const uint8_t* k_e8,
                        const uint8_t* v_codes, const uint8_t* v_e8,
                        const int32_t* page_table, const int32_t* ctx_lens, float* out) {
    if (!p || p->Hkv <= 0 || p->Hq % p->Hkv || p->tile <= 0 || p->D % 32 || p->page_size % 32) return -1;
    const int D = p->D, PS = p->page_size;
    const float alpha = (float)(p->sm_scale * kLog2e);
    const float inv448 = 1.0f / 448.0f;
    const int group = p->Hq / p->Hkv;
    const int64_t nrows = (int64_t)p->B * p->MTP * p->Hq;
    float dec[256];
    for (int c = 0; c < 256; ++c) dec[c] = orc_e4m3_decode((uint8_t)c);
    std::atomic<int> bad{0};
    parallel_for(nrows, p->nthreads, [&](int64_t r) {
        const int hq = (int)(r % p->Hq);
        const int m = (int)((r / p->Hq) % p->MTP);
        const int b = (int)(r / ((int64_t)p->Hq * p->MTP));
        const int hk = hq / group;
        const int ctx = ctx_lens[b];
        const int pos = ctx - p->MTP + m;
        const int lo_row = p->window > 0 ? std::max(0, pos - p->window + 1) : 0;
        const int lo_b = p->window > 0 ? std::max(0, ctx - p->MTP - p->window + 1) : 0;
        const float* qr = q + r * D;
        float* o = out + r * D;

        // (page, KV head) of key t, or -1 for an invalid page id
        auto page_of = [&](int t) -> int64_t {
            int pg = page_table[(int64_t)b * p->max_pages + t / PS];
            if (pg < 0 || pg >= p->num_pages) return -1;
            return (int64_t)pg * p->Hkv + hk;
        };

        std::vector<uint8_t> q8(D);
        float q_s = 0.0f;
        quant_query_row(p, qr, r, q8.data(), &q_s);

        std::vector<float> ms, ls;
        std::vector<std::vector<float>> Os;
        if (ctx > 0) {
            const int t_first = lo_b / p->tile, t_last = (ctx - 1) / p->tile;
            for (int T = t_first; T <= t_last; ++T) {
                const int k0 = std::max(T * p->tile, lo_b), k1 = std::min((T + 1) * p->tile, ctx);
                const int r0 = std::max(k0, lo_row), r1 = std::min(k1, pos + 1);
                std::vector<float> Osp(D, 0.0f);
                if (r0 >= r1) { ms.push_back(-INFINITY); ls.push_back(0.0f); Os.push_back(Osp); continue; }
                std::vector<float> x(r1 - r0), pr(r1 - r0);
                float mx = -INFINITY;
                for (int t = r0; t < r1; ++t) {
                    const int64_t ph = page_of(t);
                    if (ph < 0) { bad = 1; return; }
                    const int64_t row = ph * PS + t % PS;
                    const uint8_t* kr = k_codes + row * D;
                    const uint8_t* ke = k_e8 + row * (D / 32);
                    double dot = 0.0;
                    for (int bl = 0; bl < D / 32; ++bl) {
                        double part = 0.0;
                        for (int d = 32 * bl; d < 32 * bl + 32; ++d)
                            part += (double)dec[q8[d]] * (double)orc_e2m1_decode(kr[d]);
                        dot += std::ldexp(part, (int)ke[bl] - 127);
                    }
                    const float xv = ((float)dot * q_s) * alpha;
                    x[t - r0] = xv;
                    mx = std::max(mx, xv);
                }
                float l = 0.0f;
                for (int t = r0; t < r1; ++t) {
                    pr[t - r0] = exp2_f32(x[t - r0] - mx);
                    l = l + pr[t - r0];
                }
                std::vector<double> acc(D, 0.0);
                for (int t = r0; t < r1; ++t) {
                    const double pv = dec[orc_e4m3_encode(448.0f * pr[t - r0])];
                    if (pv == 0.0) continue;
                    const int64_t ph = page_of(t);
                    const int s = t % PS;
                    for (int d = 0; d < D; ++d) {
                        const int64_t vrow = ph * D + d;
                        const double v = std::ldexp((double)orc_e2m1_decode(v_codes[vrow * PS + s]),
                                                    (int)v_e8[vrow * (PS / 32) + s / 32] - 127);
                        acc[d] += pv * v;
                    }
                }
                for (int d = 0; d < D; ++d) Osp[d] = (float)acc[d] * inv448;
                ms.push_back(mx); ls.push_back(l); Os.push_back(Osp);
            }
        }
        float mstar = -INFINITY;
        for (float v : ms) mstar = std::max(mstar, v);
        float L = 0.0f;
        std::vector<float> acc(D, 0.0f);
        for (size_t s = 0; s < ms.size(); ++s) {
            float w = (ms[s] == -INFINITY) ? 0.0f : exp2_f32(ms[s] - mstar);
            L = L + w * ls[s];
            for (int d = 0; d < D; ++d) acc[d] = acc[d] + w * Os[s][d];
        }
        for (int d = 0; d < D; ++d) o[d] = L > 0.0f ? acc[d] / L : 0.0f;
    });
    return bad ? -2 : 0;
}

}  // extern "C"

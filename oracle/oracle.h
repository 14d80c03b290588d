/*
 * CPU oracle for SageAttention2-style quantized attention and FP8 paged decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * Canonical layouts (all contiguous, row-major):
 *   prefill Q/K/V values        float  [B, H, L, D]
 *   INT8 codes                  int8   [B, H, L, D]
 *   INT8 block scales           float  [B, H, ceil(L / block)]
 *   FP8 e4m3 codes              uint8  [B, H, L, D]
 *   V per-channel scale         float  [B, H, D]
 *   MXFP4 codes (one per byte)  uint8  [B, H, L, D]   (low nibble used)
 *   MXFP4 E8M0 scales           uint8  [B, H, L, D/32]
 *   decode query                float  [B, MTP, Hq, D]
 *   decode caches               uint8/float [P, Hkv, page, D]
 *   decode per-token scales     float  [P, Hkv, page]
 *
 * Parity status of every function is listed in oracle.cpp next to it.
 */
#ifndef SAGE_ORACLE_H
#define SAGE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
uint8_t orc_e4m3_encode(float x);
float   orc_e4m3_decode(uint8_t code);
uint8_t orc_e2m1_encode(float x);
float   orc_e2m1_decode(uint8_t nibble);
float   orc_e8m0_decode(uint8_t code);
int     orc_mx_shared_exponent(float amax);
uint16_t orc_bf16_round(float x);
uint16_t orc_fp16_round(float x);
void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out);
void orc_e4m3_decode_array(const uint8_t* c, int64_t n, float* out);
/* E2M1 code of x * 2^-e: an element of an MX block with shared exponent e */
uint8_t orc_e2m1_code_scaled(float x, int e);
void orc_e2m1_code_scaled_array(const float* x, int64_t n, int e, uint8_t* out);

/* ---- Hadamard ---------------------------------------------------------- */
void orc_hadamard(int R, float* H);

/* ---- quantizers --------------------------------------------------------- */
void orc_k_mean(const float* k, int B, int H, int L, int D, float* mu);
void orc_smooth_k(const float* k, const float* mu, int B, int H, int L, int D, float* ks);
void orc_quant_int8(const float* x, int B, int H, int L, int D, int block,
                    int8_t* codes, float* scales);
void orc_quant_v_fp8(const float* v, int B, int H, int L, int D,
                     uint8_t* codes, float* scales);
void orc_rotate(const float* x, int B, int H, int L, int D, int R, float* out);
void orc_quant_mxfp4(const float* x, int B, int H, int L, int D,
                     uint8_t* codes, uint8_t* e8m0);

/* ---- attention ---------------------------------------------------------- */
enum { ORC_QK_INT8 = 0, ORC_QK_MXFP4 = 1, ORC_QK_FLOAT = 2 };

typedef struct {
    int B, H, Lq, Lk, D;
    int causal;
    double sm_scale;
    int BN;            /* KV tile length of the online softmax */
    int qk_mode;       /* ORC_QK_* */
    int q_block, k_block;
    int quant_pv;      /* 1: P -> e4m3 and V e4m3 codes; 0: fp32 P, float V */
    int nthreads;      /* 0: all hardware threads */
} orc_attn_params;

typedef struct {
    /* ORC_QK_INT8 */
    const int8_t* q8; const float* q_scale;
    const int8_t* k8; const float* k_scale;
    /* ORC_QK_MXFP4 (codes one per byte) */
    const uint8_t* q4; const uint8_t* q_e8;
    const uint8_t* k4; const uint8_t* k_e8;
    /* ORC_QK_FLOAT */
    const float* qf; const float* kf;
    /* V: codes + per-channel scales when quant_pv, else float values */
    const uint8_t* v8; const float* v_scale;
    const float* vf;
} orc_attn_inputs;

int  orc_attn_emulated(const orc_attn_params* p, const orc_attn_inputs* in,
                       const int32_t* rows, int64_t nrows, float* out);
int  orc_attn_exact(const float* q, const float* k, const float* v,
                    int B, int H, int Lq, int Lk, int D, int causal, double sm_scale,
                    const int32_t* rows, int64_t nrows, int nthreads, double* out);
int64_t orc_qk_int8_exact(const int8_t* q8, const int8_t* k8, int D);

/* ---- paged decode ------------------------------------------------------- */
typedef struct {
    int B, MTP, Hq, Hkv, D;
    int page_size, max_pages, num_pages;
    int window;        /* 0: no window */
    int tile;          /* split length in tokens, aligned to absolute positions */
    double sm_scale;
    int quant;         /* 1: e4m3 caches + per-row e4m3 query + e4m3 P; 0: float */
    int nthreads;
    /* Optional query given already in e4m3 (quant modes only): codes
     * [B, MTP, Hq, D] and fp32 scales, one per (token, head) row or (per
     * tensor) one for all; NULL: the float q is quantized per row. */
    const uint8_t* q8;
    const float* q8_scale;
    int q8_scale_per_tensor;
} orc_decode_params;

int orc_decode_num_splits(int window, int mtp, int tile);
int orc_paged_decode(const orc_decode_params* p, const float* q,
                     const void* k_cache, const void* v_cache,
                     const float* k_scale, const float* v_scale,
                     const int32_t* page_table, const int32_t* ctx_lens, float* out);
/* MXFP4 KV cache (E2M1 codes, one per byte, and E8M0 block scales):
 * k_codes [P, Hkv, page, D], k_e8 [P, Hkv, page, D/32] (blocks along D);
 * v_codes [P, Hkv, D, page], v_e8 [P, Hkv, D, page/32] (V transposed, blocks
 * along the keys).  p->quant is ignored (Q and P are always e4m3). */
int orc_paged_decode_mx(const orc_decode_params* p, const float* q,
                        const uint8_t* k_codes, const uint8_t* k_e8,
                        const uint8_t* v_codes, const uint8_t* v_e8,
                        const int32_t* page_table, const int32_t* ctx_lens, float* out);

#ifdef __cplusplus
}
#endif
#endif

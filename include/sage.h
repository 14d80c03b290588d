/*
 * sage.h - C ABI of the MI355X (gfx950) quantized-attention library.
 *
 * SageAttention2-style quantized scaled-dot-product attention and an FP8
 * paged-KV decode, as discussed on these pages (cited by title and section):
 *   [xDiT #665]    xDiT pull request 665 "Sage v2 improvements" - the Sage v2
 *                  MXFP4 attention is fed strided tensors without contiguity
 *                  copies, and its Hadamard matrix (BLOCK_R = 128) is built
 *                  once and reused by every call.
 *   [FastVideo]    FastVideo API page "sage_attn3" (SageAttention3Impl) -
 *                  constructor arguments causal / softmax_scale /
 *                  num_kv_heads; its pre/post-processing copies QKV into
 *                  [B,H,L,D] and back, the copies this library avoids.
 *   [aiter #7388]  ROCm/aiter pull request 7388 (FlyDSL pa_decode) - paged
 *                  decode with an FP8 KV cache, per-token scales, sliding
 *                  window, split-KV partitions merged by a reduce step; FP8
 *                  flavour must match the architecture (OCP e4m3fn on gfx950,
 *                  FNUZ refused); FP8_MAX = 448 scales Q and P.
 *   [Sage2 README] "Sage2 SM89 Temporal Pair Experiment" README, section
 *                  Candidate - INT8 QK, FP8 PV, fused V scale, per-tile order
 *                  QK -> online-softmax update -> row sum -> FP8 P -> PV.
 *
 * Conventions
 *  - Tensors are described by sage_tensor: a device pointer, a dtype, and a
 *    LOGICAL shape with element strides.  Q/K/V/out are logical [B, L, H, D];
 *    any non-negative B/L/H strides are accepted (so [B,L,H,D], [B,H,L,D] and
 *    views into a stacked QKV buffer all work) but stride[D] must be 1; a
 *    negative stride is refused with SAGE_ERR_LAYOUT.  The library never
 *    copies an input to make it contiguous.  The kernels read one (b, h) slice
 *    of an fp16/bf16 Q, K or V with 32-bit byte offsets, so a slice may span
 *    at most 0x7FFFFF00 bytes, ((L - 1) stride[L] + D) * 2; a longer one is
 *    refused with SAGE_ERR_UNSUPPORTED (for the stacked video-DiT layout,
 *    stride[L] = 3 H D = 15360, that is L <= 69906).
 *  - Alignment: every pointer handed to the library must be 16-byte aligned;
 *    for strided Q/K/V/out, every row start (each B/L/H stride in bytes) must
 *    be a multiple of 16 bytes.
 *  - Quantized tensors use the library layouts documented per function; they
 *    must be contiguous with exactly the stated shape.  Padded lengths:
 *    SAGE_PAD(L) = ceil(L / 128) * 128.
 *  - Ownership: the caller owns every tensor and every workspace.  The only
 *    device memory the library allocates is inside sage_hadamard_create.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream).  Every
 *    call only enqueues work on that stream: no allocation, no
 *    synchronisation, no host blocking.
 *  - Errors: every function returns a sage_status.  All argument validation
 *    runs before any HIP call (so it can be exercised without a GPU) and is
 *    O(1).  On failure nothing is enqueued and sage_last_error() returns a
 *    thread-local message.  Launch failures are reported as SAGE_ERR_HIP;
 *    faults inside a kernel surface at the caller's next synchronisation.
 *    No C++ exception crosses this interface.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_VERSION_MAJOR 0
#define SAGE_VERSION_MINOR 4
#define SAGE_PAD(L) ((((L) + 127) / 128) * 128)

typedef enum {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARG = 1,  /* null pointer, bad enum, inconsistent sizes  */
    SAGE_ERR_DTYPE = 2,        /* unsupported dtype or combination (incl. FNUZ FP8) */
    SAGE_ERR_SHAPE = 3,        /* shape mismatch, unsupported head dim, R != 128  */
    SAGE_ERR_LAYOUT = 4,       /* stride[D] != 1, negative stride, non-contiguous library tensor */
    SAGE_ERR_ALIGNMENT = 5,    /* pointer or row stride not 16-byte aligned      */
    SAGE_ERR_WORKSPACE = 6,    /* workspace missing or too small                 */
    SAGE_ERR_ARCH = 7,         /* current device is not gfx950                   */
    SAGE_ERR_HIP = 8,          /* a HIP runtime call or launch failed            */
    SAGE_ERR_UNSUPPORTED = 9   /* valid request outside what is implemented      */
} sage_status;

typedef enum {
    SAGE_F16 = 1,
    SAGE_BF16 = 2,
    SAGE_F32 = 3,
    SAGE_I8 = 4,
    SAGE_I32 = 5,
    SAGE_U8 = 6,
    SAGE_FP8_E4M3FN = 7,    /* OCP e4m3 (gfx950's MFMA format), max 448            */
    SAGE_FP8_E4M3FNUZ = 8,  /* gfx94x flavour: always refused (SAGE_ERR_DTYPE)    */
    SAGE_FP4X2_E2M1 = 9,    /* two E2M1 codes per byte, element 2i in low nibble  */
    SAGE_E8M0 = 10          /* MX shared exponent, value 2^(code-127)             */
} sage_dtype;

typedef struct {
    void* data;          /* device pointer, 16-byte aligned                     */
    int32_t dtype;       /* sage_dtype                                          */
    int32_t ndim;        /* 1..5                                                */
    int64_t shape[5];
    int64_t stride[5];   /* in elements (for FP4X2: in bytes, i.e. code pairs)  */
} sage_tensor;

typedef enum { SAGE_QK_INT8 = 0, SAGE_QK_MXFP4 = 1 } sage_qk_mode;

/* Immutable Hadamard rotation (Sylvester order R, scaled by 1/sqrt(R)) kept on
 * one device and shared by every call and thread ([xDiT #665]: built once). */
typedef struct sage_hadamard sage_hadamard;

/* ------------------------------------------------------------------------- */
/* Q/K quantization.                                                          */
/*
 * Method (SageAttention2 as named on the pages; step details are the
 * library's documented reading):
 *  - smooth_k: mu[b,h,d] = mean of K over all Lk tokens (fp64 sum, rounded
 *    once to fp32); K_s = fp32(K - mu).
 *  - SAGE_QK_INT8: Q in q_block-token blocks and K_s in k_block-token blocks
 *    per (b,h): scale = fp32(amax / 127), code = clamp(rne(fp32(x *
 *    fp32(127 / amax))), -127, 127); amax == 0 -> scale 0, codes 0.
 *      q_out   I8   [B, H, SAGE_PAD(Lq), D]    (rows >= Lq are 0)
 *      q_scale F32  [B, H, SAGE_PAD(Lq) / q_block]
 *      k_out   I8   [B, H, SAGE_PAD(Lk), D]
 *      k_scale F32  [B, H, SAGE_PAD(Lk) / k_block]
 *    q_block must be 128; k_block must be 64 or 128.
 *  - SAGE_QK_MXFP4 ([xDiT #665]): rows of Q and K_s are rotated per 128-channel
 *    block by the Hadamard handle (NULL: no rotation), then quantized per 32
 *    channels: E8M0 exponent e = floor(log2 amax) - 2, codes
 *    e2m1_rne_sat(x * 2^-e).
 *      q_out   FP4X2 [B, H, SAGE_PAD(Lq), D/2]   q_scale E8M0 [B, H, SAGE_PAD(Lq), D/32]
 *      k_out   FP4X2 [B, H, SAGE_PAD(Lk), D/2]   k_scale E8M0 [B, H, SAGE_PAD(Lk), D/32]
 *  q, k: F16 or BF16 logical [B, L, H, D], D in {64, 128}, any B/L/H strides.
 *    q NULL: K alone, with q_out and q_scale NULL; Q is then quantized inside
 *    sage_attn_fwd (q_scale NULL there; MXFP4: with the same hadamard).
 *  k_mean: optional F32 [B, H, D] output of mu (NULL: kept in the workspace).
 *  workspace: sage_quantize_qk_workspace_size bytes, 16-byte aligned.  Its
 *    contents need no initialization and may be anything between calls; the
 *    blocks of one call exchange per-chunk K statistics and arrival flags
 *    through it, so calls that share a workspace must not overlap in time.
 */
typedef struct {
    int32_t mode;       /* sage_qk_mode                              */
    int32_t q_block;    /* INT8: tokens per Q scale (128)            */
    int32_t k_block;    /* INT8: tokens per K scale (64 or 128)      */
    int32_t smooth_k;   /* 1: subtract the per-channel K mean        */
} sage_qk_params;

sage_status sage_quantize_qk_workspace_size(const sage_tensor* q, const sage_tensor* k,
                                            const sage_qk_params* params, size_t* bytes);
sage_status sage_quantize_qk(const sage_tensor* q, const sage_tensor* k,
                             const sage_qk_params* params,
                             const sage_tensor* q_out, const sage_tensor* q_scale,
                             const sage_tensor* k_out, const sage_tensor* k_scale,
                             const sage_tensor* k_mean, const sage_hadamard* hadamard,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* V quantization to FP8 e4m3 with one scale per channel ([Sage2 README]: the
 * kernel fuses a per-channel V scale).  Per (b,h,d): amax over all Lk tokens,
 * scale = fp32(amax / 448), code = e4m3_rne(fp32(v * fp32(448 / amax))).
 *   v       F16/BF16 logical [B, Lk, H, D], any B/L/H strides
 *   v_out   FP8_E4M3FN [B, H, D, SAGE_PAD(Lk)]  ("transposed V": keys contiguous;
 *           keys >= Lk are 0)
 *   v_scale F32 [B, H, D]
 *   workspace: sage_quantize_v_workspace_size bytes, 16-byte aligned; as for
 *           sage_quantize_qk it needs no initialization, and calls sharing it
 *           must not overlap in time.
 */
sage_status sage_quantize_v_workspace_size(const sage_tensor* v, size_t* bytes);
sage_status sage_quantize_v(const sage_tensor* v, const sage_tensor* v_out,
                            const sage_tensor* v_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* How the attention kernel's waves share a SIMD.  Both give the same output
 * bits; they differ in speed only.
 *   SAGE_SCHED_INTERLEAVED  workgroups of 4 waves (128 query rows), three per
 *     CU: the hardware interleaves the waves' MFMA and softmax phases.
 *   SAGE_SCHED_PINGPONG  workgroups of 8 waves (two 128-row query blocks of
 *     one head, sharing every K/V tile), two waves per SIMD alternating an
 *     MFMA phase (PV of the previous tile, QK of this one) and a softmax phase
 *     between workgroup barriers, the two groups offset by one phase: the
 *     wave-pair schedule of the "Sage2 SM89 Temporal Pair Experiment" README
 *     (Candidate section).  INT8 QK with head dim 128 only
 *     (SAGE_ERR_UNSUPPORTED otherwise).
 * Any other value is refused with SAGE_ERR_INVALID_ARG. */
typedef enum { SAGE_SCHED_INTERLEAVED = 0, SAGE_SCHED_PINGPONG = 1 } sage_attn_schedule;

/* Quantized attention forward.  For each query row, KV tiles of
 * sage_attn_kv_tile() keys in ascending order (the online-softmax block size,
 * so part of the numeric result): S = QK^T on INT8 (or scaled MXFP4) MFMA with int32 (fp32)
 * accumulation; x = S * q_scale * k_scale * sm_scale * log2(e); online
 * softmax with fp32 running max m and row sum l (l summed from the fp32
 * probabilities, before conversion); P = e4m3(448 p) (the kernel evaluates
 * 448 p as exp2(fma(S, c, -(m - log2 448))), the same value up to the
 * rounding of the exponent); O += P V on FP8 MFMA with fp32
 * accumulation; out = O * v_scale[d] / (448 l), rounded to out's dtype,
 * written with out's strides ([Sage2 README], [aiter #7388]: 448 = FP8_MAX
 * of OCP e4m3).  Causal masks keep key j <= query i (Lq == Lk);
 * fully masked tiles are skipped.
 *   q_q, q_scale, k_q, k_scale: sage_quantize_qk outputs (mode = qk_mode)
 *   q_scale NULL: q_q is the F16/BF16 Q, logical [B, Lq, H, D] with any
 *     B/L/H strides (token stride >= D, one head within 2^31 bytes),
 *     quantized in the kernel's prologue with sage_quantize_qk's arithmetic:
 *     INT8 per 128-query block, or (SAGE_QK_MXFP4) rotated by
 *     params.hadamard and quantized to MXFP4.  The codes and scales, hence
 *     the output, are those of the unfused path bit for bit; Q's quantized
 *     copy is neither written nor read.
 *   v_q, v_scale: sage_quantize_v outputs
 *   out: F16, BF16 or F32 logical [B, Lq, H, D], any B/L/H strides
 * num_kv_heads: K/V heads (H % num_kv_heads == 0; query head h reads KV head
 * h / (H / num_kv_heads)); 0 means H.  No workspace is needed (pass NULL, 0).
 */

typedef struct {
    float sm_scale;        /* <= 0: 1/sqrt(D)                                  */
    int32_t causal;
    int32_t qk_mode;       /* sage_qk_mode                                     */
    int32_t batch, heads, seqlen_q, seqlen_k, head_dim;
    int32_t num_kv_heads;  /* 0: heads                                         */
    int32_t q_block, k_block;  /* INT8 scale granularities used by quantize_qk */
    /* SAGE_QK_MXFP4 with q_scale NULL only (else NULL): the rotation applied to
     * Q in the prologue; NULL there means no rotation */
    const sage_hadamard* hadamard;
    int32_t schedule;      /* sage_attn_schedule (0: interleaved)              */
} sage_attn_params;

sage_status sage_attn_fwd(const sage_tensor* q_q, const sage_tensor* q_scale,
                          const sage_tensor* k_q, const sage_tensor* k_scale,
                          const sage_tensor* v_q, const sage_tensor* v_scale,
                          const sage_attn_params* params, const sage_tensor* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Keys per KV tile of sage_attn_fwd's online softmax (64). */
int32_t sage_attn_kv_tile(void);

/* ------------------------------------------------------------------------- */
/* Paged decode over an FP8 e4m3 KV cache ([aiter #7388]; its shape matrix
 * covers D 64 / 128 / 256, bf16, fp16 and e4m3 queries, per-tensor and
 * per-token scales, transposed and plain V).
 *   q          BF16 or F16 [B, MTP, Hq, D], or FP8_E4M3FN with the scales
 *              params.q_scale (any B/MTP/Hq strides, rows 16-byte aligned);
 *              query token m sits at position ctx_lens[b] - MTP + m
 *   k_cache    FP8_E4M3FN [P, Hkv, page, D] contiguous
 *   v_cache    FP8_E4M3FN [P, Hkv, D, page] contiguous when v_transposed = 1,
 *              [P, Hkv, page, D] ("plain") when v_transposed = 0
 *   k_scale, v_scale  F32 [P, Hkv, page] (per-token scales), or F32 [1] each
 *              (one scale per cache tensor)
 *   page_table I32 [B, max_pages]: page of token t is page_table[b][t / page]
 *   ctx_lens   I32 [B]
 *   out        BF16 or F16 [B, MTP, Hq, D] (any B/MTP/Hq strides)
 * With window W > 0 query position p sees keys [p - W + 1, p]; otherwise
 * [0, p].  The work is split into 256-token tiles aligned to absolute
 * positions, one split per tile ([aiter #7388], "Batch-first plan grid
 * removal": one task per 256-token window tile); splits
 * write (m, l, O) partials to the workspace and a merge step combines them
 * (O is kept normalized, O / l, in fp16 scaled into [-448, 448]: the merge's
 * inputs carry a relative rounding of 2^-11, below the bf16 output's 2^-9).
 * bf16 / fp16 Q rows are quantized to e4m3 with a per-(token, head) scale
 * (an e4m3 q is used as given, with its scale); scores use FP8 MFMA; P is
 * requantized per tile with the tile's largest per-token V scale.  D must be
 * 64, 128 or 256 (MXFP4 cache: 128); the page size must be a multiple of 16
 * that divides 256 or is a multiple of 256; MTP * (Hq / Hkv) <= 64.  Page-table entries of tokens
 * below ctx_lens[b] must be valid page indices, and ctx_lens[b] <=
 * params.max_ctx; device data is not validated, but a page id outside
 * [0, P) reads page 0 and a length above max_ctx is treated as max_ctx, so
 * bad device data gives wrong numbers, never a fault.
 * MXFP4 cache ([aiter #7388] names pa_decode_mxfp4: E2M1 KV, E8M0 scales;
 * the layout is this library's reading), chosen by k_cache's dtype:
 *   k_cache FP4X2_E2M1 [P, Hkv, page, D/2], k_scale E8M0 [P, Hkv, page, D/32]
 *           (one scale per 32 channels of a token: the QK reduction axis)
 *   v_cache FP4X2_E2M1 [P, Hkv, D, page/2] (transposed; key 2i in the low
 *           nibble), v_scale E8M0 [P, Hkv, D, page/32] (one scale per 32 keys
 *           of a channel: the PV reduction axis)
 * QK and PV run on the block-scaled MFMA with these scales, P8 =
 * e4m3(448 p); the page size must be a multiple of 64, V must be transposed
 * (the only layout whose blocks run along the keys), and the V scale of
 * every 32-key block that holds a key below ctx_lens[b] must be set (blocks
 * wholly past it are ignored).
 */
typedef struct {
    float sm_scale;        /* <= 0: 1/sqrt(D)                  */
    int32_t window;        /* 0: no sliding window             */
    int32_t v_transposed;  /* layout flag of v_cache (1 transposed, 0 plain) */
    int32_t max_ctx;       /* upper bound of ctx_lens (sizes the split plan) */
    /* FP8_E4M3FN q only (NULL otherwise): F32 [1] (one scale for q) or
     * [B, MTP, Hq] (one per (token, head) row), contiguous; q's value is
     * code * scale */
    const sage_tensor* q_scale;
    /* splits per sequence: 0 takes the plan, one split per 256-token tile
     * (sage_decode_num_splits(window, MTP, max_ctx)); any other value must
     * equal the plan's count (other split lengths are not built:
     * SAGE_ERR_UNSUPPORTED; negative: SAGE_ERR_INVALID_ARG) */
    int32_t num_splits;
} sage_decode_params;

sage_status sage_paged_decode_workspace_size(const sage_tensor* q, const sage_tensor* k_cache,
                                             const sage_tensor* page_table,
                                             const sage_decode_params* params, size_t* bytes);
sage_status sage_paged_decode(const sage_tensor* q, const sage_tensor* k_cache,
                              const sage_tensor* v_cache, const sage_tensor* k_scale,
                              const sage_tensor* v_scale, const sage_tensor* page_table,
                              const sage_tensor* ctx_lens, const sage_decode_params* params,
                              const sage_tensor* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* sage_paged_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and kernels, with the split partials kept in a fixed device
 * scratch array of SAGE_DECODE_SCRATCH_BYTES per device instead of a
 * workspace.  The caller still owns q, the caches, scales, page table,
 * lengths and out.  The call allocates nothing (no hipMalloc or allocating
 * library routine); its first call on a device looks the array's address up
 * once (hipGetSymbolAddress).  A decode whose partials need more than
 * SAGE_DECODE_SCRATCH_BYTES (sage_paged_decode_workspace_size) is refused
 * with SAGE_ERR_WORKSPACE before anything is enqueued.  Every call on a
 * device shares that device's scratch, which keeps the last call's contents
 * (nothing in it needs clearing between calls): calls that overlap in time
 * on one device -- on different streams or threads -- race and give wrong
 * results; calls enqueued on one stream are ordered and safe. */
#define SAGE_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
sage_status sage_paged_decode_noalloc(const sage_tensor* q, const sage_tensor* k_cache,
                                      const sage_tensor* v_cache, const sage_tensor* k_scale,
                                      const sage_tensor* v_scale, const sage_tensor* page_table,
                                      const sage_tensor* ctx_lens, const sage_decode_params* params,
                                      const sage_tensor* out, void* stream);

/* Number of splits per sequence the plan uses for a window:
 * (window + mtp - 1 - 1 + 255) / 256 + 1 when window > 0, else
 * ceil(max_ctx / 256) ([aiter #7388] window tiles). */
int32_t sage_decode_num_splits(int32_t window, int32_t mtp, int32_t max_ctx);

/* ------------------------------------------------------------------------- */
/* Helpers.                                                                   */

/* Builds the order-R Sylvester Hadamard matrix scaled by 1/sqrt(R) on
 * `device` (R must be 128).  The handle is immutable and may be shared by
 * threads and calls; destroy it once no enqueued work uses it. */
sage_status sage_hadamard_create(int32_t R, int32_t device, void* stream, sage_hadamard** out);
sage_status sage_hadamard_destroy(sage_hadamard* h);

/* Bound on the wait inside sage_quantize_qk (INT8 with smooth_k) and
 * sage_quantize_v.  When the whole grid fits on the device at once, each
 * block holds one 256-token chunk of a head and waits for the other chunks'
 * statistics (channel sums of K, channel amax of V), so the inputs are read
 * from HBM once.  A block that has not seen every chunk of its head after
 * `us` microseconds (other streams' kernels may hold part of the device)
 * computes the head's statistic itself from the inputs, in the same order:
 * the outputs are identical, only slower.  Default 2000; 0 is allowed (tests
 * use it to take that path).  Process-wide; affects launches made after the
 * call.  Returns SAGE_ERR_INVALID_ARG outside [0, 1000000]. */
sage_status sage_set_quant_wait_us(int32_t us);

/* Test hook: int32 S = Q8 K8^T for query rows [q0, q0 + nq) and keys
 * [k0, k0 + nk) of every (b, h), computed by the attention kernel's own QK
 * step (same MFMA shape, operand layout and reduction order).  q0 and nq must
 * be multiples of 32, k0 and nk multiples of 128, inside the padded lengths
 * of the INT8 q_q [B, H, Lqp, D] and k_q [B, H, Lkp, D].
 *   out I32 [B, H, nq, nk] contiguous. */
sage_status sage_debug_qk_tile(const sage_tensor* q_q, const sage_tensor* k_q,
                               int32_t q0, int32_t nq, int32_t k0, int32_t nk,
                               const sage_tensor* out, void* stream);

/* Test hook: fp32 S = Q K^T of MXFP4 codes, for query rows [q0, q0 + nq)
 * and keys [k0, k0 + nk) of every (b, h), computed by sage_attn_fwd's own
 * MXFP4 QK step (the block-scaled MFMA, same operand layout and order): per
 * 32-channel block the E2M1 products scaled by 2^(e_q + e_k), summed in fp32
 * ([xDiT #665]: the Sage v2 MXFP4 path).  Ranges as for sage_debug_qk_tile.
 *   q_q FP4X2_E2M1 [B, H, Lqp, 64], q_scale E8M0 [B, H, Lqp, 4] (D = 128),
 *   k_q, k_scale likewise with Lkp; out F32 [B, H, nq, nk] contiguous. */
sage_status sage_debug_qk_tile_mx(const sage_tensor* q_q, const sage_tensor* q_scale,
                                  const sage_tensor* k_q, const sage_tensor* k_scale, int32_t q0,
                                  int32_t nq, int32_t k0, int32_t nk, const sage_tensor* out,
                                  void* stream);

/* Test hook: codes[i] = the OCP e4m3 code (OCP 8-bit floating point, E4M3:
 * round to nearest even) that the kernels give x[i] -- the conversion that
 * codes P8 = e4m3(448 p) in attention and decode, the V quantizers' codes and
 * the decode's query codes ([aiter #7388], Changes: Q and P in FP8_MAX's
 * format).  The kernels never convert a value of magnitude above 448 by more
 * than rounding slack; beyond 464 the code is whatever the hardware gives.
 *   x F32 [n] contiguous (device), codes U8 [n] contiguous (device); n = 0
 *   does nothing.  Errors: DTYPE / SHAPE / LAYOUT / ALIGNMENT for the
 *   descriptors, before any HIP call. */
sage_status sage_debug_cvt_e4m3(const sage_tensor* x, const sage_tensor* codes, void* stream);

/* Test hook: codes[i] = the E2M1 code (low nibble; OCP MX v1.0 FP4: round to
 * nearest even, saturating at 6) of x[i] * 2^-exponent as the MXFP4 quantizer
 * and the fused-Q attention prologue code an element of a block whose shared
 * exponent is `exponent` ([xDiT #665]: the Sage v2 MXFP4 path).
 *   x F32 [n], codes U8 [n] as above; exponent in [-127, 127], else
 *   SAGE_ERR_INVALID_ARG. */
sage_status sage_debug_cvt_e2m1(const sage_tensor* x, int32_t exponent, const sage_tensor* codes,
                                void* stream);

/* Thread-local message of the last failure on this thread ("" if none). */
const char* sage_last_error(void);
/* (major << 16) | minor */
int32_t sage_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H */

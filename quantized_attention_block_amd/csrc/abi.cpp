// C ABI of the quantized-attention library: argument validation, workspace
// sizing and dispatch to the gfx950 kernels.  Every check runs before the
// first HIP call, so refusals can be exercised without a GPU.  Refusal rules
// follow ROCm/aiter pull request 7388 (Changes): unsupported dtypes are
// refused, and an FP8 tensor that is not the architecture's MFMA format (FNUZ
// on gfx950) is refused.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/sage.h"
#include "sage_launch.hpp"

static_assert(SAGE_DECODE_SCRATCH_BYTES == sage::kDecodeScratchBytes, "scratch size in sage.h");

struct sage_hadamard {
    int32_t R;
    int32_t device;
    void* bf16_mat;   // R x R, +-1
    void* f16_mat;    // R x R, +-1
    float inv_sqrt_r; // fp32(1 / sqrt(R))
};

namespace {

thread_local char g_err[512] = "";

sage_status fail(sage_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

sage_status ok() {
    g_err[0] = 0;
    return SAGE_OK;
}

size_t elem_bytes(int32_t dt) {
    switch (dt) {
        case SAGE_F16: case SAGE_BF16: return 2;
        case SAGE_F32: case SAGE_I32: return 4;
        case SAGE_I8: case SAGE_U8: case SAGE_FP8_E4M3FN: case SAGE_FP8_E4M3FNUZ:
        case SAGE_FP4X2_E2M1: case SAGE_E8M0: return 1;
        default: return 0;
    }
}

const char* dtype_name(int32_t dt) {
    switch (dt) {
        case SAGE_F16: return "f16";
        case SAGE_BF16: return "bf16";
        case SAGE_F32: return "f32";
        case SAGE_I8: return "i8";
        case SAGE_I32: return "i32";
        case SAGE_U8: return "u8";
        case SAGE_FP8_E4M3FN: return "fp8_e4m3fn";
        case SAGE_FP8_E4M3FNUZ: return "fp8_e4m3fnuz";
        case SAGE_FP4X2_E2M1: return "fp4x2_e2m1";
        case SAGE_E8M0: return "e8m0";
        default: return "unknown";
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

sage_status check_basic(const sage_tensor* t, const char* name, int ndim) {
    if (!t) return fail(SAGE_ERR_INVALID_ARG, "%s: null descriptor", name);
    if (!t->data) return fail(SAGE_ERR_INVALID_ARG, "%s: null data pointer", name);
    if (elem_bytes(t->dtype) == 0) return fail(SAGE_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
    if (t->ndim != ndim)
        return fail(SAGE_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] < 0) return fail(SAGE_ERR_SHAPE, "%s: negative extent", name);
    if (!aligned16(t->data)) return fail(SAGE_ERR_ALIGNMENT, "%s: data pointer not 16-byte aligned", name);
    return SAGE_OK;
}

sage_status check_fp8(const sage_tensor* t, const char* name) {
    if (t->dtype == SAGE_FP8_E4M3FNUZ)
        return fail(SAGE_ERR_DTYPE,
                    "%s: FP8 tensor is e4m3fnuz, but gfx950 MFMAs read OCP e4m3fn", name);
    if (t->dtype != SAGE_FP8_E4M3FN)
        return fail(SAGE_ERR_DTYPE, "%s: expected fp8_e4m3fn, got %s", name, dtype_name(t->dtype));
    return SAGE_OK;
}

// Library-layout tensor: exact shape, contiguous, given dtype.
sage_status check_exact(const sage_tensor* t, const char* name, int32_t dtype, int ndim,
                        const int64_t* shape) {
    sage_status st = check_basic(t, name, ndim);
    if (st) return st;
    if (dtype == SAGE_FP8_E4M3FN) {
        if ((st = check_fp8(t, name))) return st;
    } else if (t->dtype != dtype) {
        return fail(SAGE_ERR_DTYPE, "%s: expected %s, got %s", name, dtype_name(dtype),
                    dtype_name(t->dtype));
    }
    int64_t expect = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        if (t->shape[i] != shape[i])
            return fail(SAGE_ERR_SHAPE, "%s: dim %d is %lld, expected %lld", name, i,
                        (long long)t->shape[i], (long long)shape[i]);
        if (t->shape[i] > 1 && t->stride[i] != expect)
            return fail(SAGE_ERR_LAYOUT, "%s: library tensors must be contiguous (dim %d stride %lld)",
                        name, i, (long long)t->stride[i]);
        expect *= shape[i];
    }
    return SAGE_OK;
}

// A caller's view: no negative stride (it would address memory before the
// view's base pointer, which the kernels' buffer resources start at).
sage_status check_strides(const sage_tensor* t, const char* name) {
    for (int i = 0; i < t->ndim; ++i)
        if (t->stride[i] < 0)
            return fail(SAGE_ERR_LAYOUT, "%s: negative stride %lld in dim %d", name, (long long)t->stride[i], i);
    return SAGE_OK;
}

// Strided half-precision [B, L, H, D] view: stride[D] == 1, 16-byte aligned
// rows, non-negative strides.  The kernels read one (b, h) slice through a
// buffer resource with 32-bit byte offsets, so a slice may span at most
// 0x7FFFFF00 bytes: ((L - 1) stride[L] + D) * 2.
sage_status check_half_view(const sage_tensor* t, const char* name) {
    sage_status st = check_basic(t, name, 4);
    if (st) return st;
    if (t->dtype != SAGE_F16 && t->dtype != SAGE_BF16)
        return fail(SAGE_ERR_DTYPE, "%s: expected f16 or bf16, got %s", name, dtype_name(t->dtype));
    if ((st = check_strides(t, name))) return st;
    for (int i = 0; i < 4; ++i)
        if (t->shape[i] > 0x7FFFFFFF)
            return fail(SAGE_ERR_SHAPE, "%s: dim %d (%lld) exceeds 2^31 - 1", name, i, (long long)t->shape[i]);
    if (t->shape[1] > 0 && ((t->shape[1] - 1) * t->stride[1] + t->shape[3]) * 2 > 0x7FFFFF00LL)
        return fail(SAGE_ERR_UNSUPPORTED, "%s: one (b, h) slice spans more than 2^31 bytes "
                    "(L %lld, token stride %lld elements)", name, (long long)t->shape[1], (long long)t->stride[1]);
    if (t->shape[3] > 1 && t->stride[3] != 1)
        return fail(SAGE_ERR_LAYOUT, "%s: the head-dim stride must be 1 (got %lld)", name,
                    (long long)t->stride[3]);
    for (int i = 0; i < 3; ++i)
        if (t->shape[i] > 1 && ((t->stride[i] * 2) % 16) != 0)
            return fail(SAGE_ERR_ALIGNMENT, "%s: stride of dim %d (%lld elements) is not a multiple of 16 bytes",
                        name, i, (long long)t->stride[i]);
    return SAGE_OK;
}

sage::HalfView half_view(const sage_tensor* t) {
    return sage::HalfView{t->data, t->stride[0], t->stride[1], t->stride[2], t->dtype == SAGE_BF16};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device architecture check, cached per device.
sage_status check_device() {
    static std::mutex mu;
    static int cached[64];   // 0 unknown, 1 gfx950, 2 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SAGE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(SAGE_ERR_ARCH, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (cached[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(SAGE_ERR_HIP, "hipGetDeviceProperties failed");
        cached[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    if (cached[dev] != 1) return fail(SAGE_ERR_ARCH, "device %d is not gfx950", dev);
    return SAGE_OK;
}

sage_status launch_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SAGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- quantize_qk helpers -------------------------------------------------------
struct QkShape {
    int B, H, Lq, Lk, D;
};

sage_status qk_inputs(const sage_tensor* q, const sage_tensor* k, const sage_qk_params* p,
                      QkShape* s) {
    sage_status st;
    if (q && (st = check_half_view(q, "q"))) return st;
    if ((st = check_half_view(k, "k"))) return st;
    if (!p) return fail(SAGE_ERR_INVALID_ARG, "params: null");
    if (q && q->dtype != k->dtype) return fail(SAGE_ERR_DTYPE, "q and k dtypes differ");
    if (q && (q->shape[0] != k->shape[0] || q->shape[2] != k->shape[2] || q->shape[3] != k->shape[3]))
        return fail(SAGE_ERR_SHAPE, "q and k must agree on B, H and D");
    s->B = (int)k->shape[0];
    s->Lq = q ? (int)q->shape[1] : 0;   // q NULL: K only
    s->H = (int)k->shape[2];
    s->D = (int)k->shape[3];
    s->Lk = (int)k->shape[1];
    if (s->B < 1 || s->H < 1 || (q && s->Lq < 1) || s->Lk < 1)
        return fail(SAGE_ERR_SHAPE, "empty q or k (B, H, L must be >= 1)");
    if (p->mode != SAGE_QK_INT8 && p->mode != SAGE_QK_MXFP4)
        return fail(SAGE_ERR_INVALID_ARG, "params.mode: unknown qk mode %d", p->mode);
    if (p->smooth_k != 0 && p->smooth_k != 1)
        return fail(SAGE_ERR_INVALID_ARG, "params.smooth_k must be 0 or 1");
    if (p->mode == SAGE_QK_INT8) {
        if (s->D != 64 && s->D != 128) return fail(SAGE_ERR_SHAPE, "head dim %d not in {64, 128}", s->D);
        if (p->q_block != 128) return fail(SAGE_ERR_UNSUPPORTED, "q_block must be 128");
        if (p->k_block != 64 && p->k_block != 128)
            return fail(SAGE_ERR_UNSUPPORTED, "k_block must be 64 or 128");
    } else if (s->D != 128) {
        return fail(SAGE_ERR_SHAPE, "MXFP4 path needs head dim 128 (BLOCK_R = 128), got %d", s->D);
    }
    return SAGE_OK;
}

size_t qk_ws_bytes(const QkShape& s, const sage_qk_params* p) {
    size_t n = 0;
    if (p->smooth_k) {
        n += align256((size_t)s.B * s.H * sage::mean_chunks(s.Lk) * s.D * sizeof(double));
        n += align256((size_t)s.B * s.H * s.D * sizeof(float));   // mu when k_mean is NULL
        n += align256((size_t)sage::quant_sync_words((int64_t)s.B * s.H, s.Lk) * sizeof(uint64_t));
    }
    if (p->mode == SAGE_QK_MXFP4) n += align256((size_t)s.B * s.H * s.D * sizeof(float));
    return n;
}

// V: channel amax per token chunk (fp32), then the head-synchronization words
size_t v_ws_bytes(int B, int Lk, int H, int D) {
    return align256((size_t)B * H * sage::mean_chunks(Lk) * D * sizeof(float)) +
           align256((size_t)sage::quant_sync_words((int64_t)B * H, Lk) * sizeof(uint64_t));
}

}  // namespace

extern "C" {

const char* sage_last_error(void) { return g_err; }

int32_t sage_version(void) { return (SAGE_VERSION_MAJOR << 16) | SAGE_VERSION_MINOR; }

sage_status sage_set_quant_wait_us(int32_t us) {
    if (us < 0 || us > 1000000) return fail(SAGE_ERR_INVALID_ARG, "wait %d us outside [0, 1e6]", us);
    sage::set_quant_wait_us(us);
    return ok();
}

int32_t sage_attn_kv_tile(void) { return sage::kKvTile; }

int32_t sage_decode_num_splits(int32_t window, int32_t mtp, int32_t max_ctx) {
    const int tile = sage::kDecodeTile;
    if (max_ctx <= 0) return 0;
    const int all = (max_ctx + tile - 1) / tile;
    if (window <= 0) return all;
    const int span = window + mtp - 1;
    const int w = (span - 1 + tile - 1) / tile + 1;
    return w < all ? w : all;
}

sage_status sage_quantize_qk_workspace_size(const sage_tensor* q, const sage_tensor* k,
                                            const sage_qk_params* params, size_t* bytes) {
    QkShape s;
    sage_status st = qk_inputs(q, k, params, &s);
    if (st) return st;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes: null");
    *bytes = qk_ws_bytes(s, params);
    return ok();
}

sage_status sage_quantize_qk(const sage_tensor* q, const sage_tensor* k, const sage_qk_params* params,
                             const sage_tensor* q_out, const sage_tensor* q_scale,
                             const sage_tensor* k_out, const sage_tensor* k_scale,
                             const sage_tensor* k_mean, const sage_hadamard* hadamard,
                             void* workspace, size_t workspace_bytes, void* stream) {
    QkShape s;
    sage_status st = qk_inputs(q, k, params, &s);
    if (st) return st;
    const int64_t Lqp = sage::pad128(s.Lq), Lkp = sage::pad128(s.Lk);
    if (params->mode == SAGE_QK_INT8) {
        const int64_t qs[4] = {s.B, s.H, Lqp, s.D}, ks[4] = {s.B, s.H, Lkp, s.D};
        const int64_t qss[3] = {s.B, s.H, Lqp / params->q_block};
        const int64_t kss[3] = {s.B, s.H, Lkp / params->k_block};
        if (!q) {
            if (q_out || q_scale) return fail(SAGE_ERR_INVALID_ARG, "q is NULL: q_out and q_scale must be NULL");
        } else {
            if ((st = check_exact(q_out, "q_out", SAGE_I8, 4, qs))) return st;
            if ((st = check_exact(q_scale, "q_scale", SAGE_F32, 3, qss))) return st;
        }
        if ((st = check_exact(k_out, "k_out", SAGE_I8, 4, ks))) return st;
        if ((st = check_exact(k_scale, "k_scale", SAGE_F32, 3, kss))) return st;
        if (hadamard) return fail(SAGE_ERR_INVALID_ARG, "hadamard: only used by the MXFP4 mode");
    } else {
        const int64_t qs[4] = {s.B, s.H, Lqp, s.D / 2}, ks[4] = {s.B, s.H, Lkp, s.D / 2};
        const int64_t qe[4] = {s.B, s.H, Lqp, s.D / 32}, ke[4] = {s.B, s.H, Lkp, s.D / 32};
        if (!q) {
            if (q_out || q_scale) return fail(SAGE_ERR_INVALID_ARG, "q is NULL: q_out and q_scale must be NULL");
        } else {
            if ((st = check_exact(q_out, "q_out", SAGE_FP4X2_E2M1, 4, qs))) return st;
            if ((st = check_exact(q_scale, "q_scale", SAGE_E8M0, 4, qe))) return st;
        }
        if ((st = check_exact(k_out, "k_out", SAGE_FP4X2_E2M1, 4, ks))) return st;
        if ((st = check_exact(k_scale, "k_scale", SAGE_E8M0, 4, ke))) return st;
        if (hadamard && (hadamard->R != 128 || s.D % hadamard->R != 0))
            return fail(SAGE_ERR_SHAPE, "hadamard: order %d must be 128 and divide D", hadamard->R);
    }
    if (k_mean) {
        const int64_t ms[3] = {s.B, s.H, s.D};
        if ((st = check_exact(k_mean, "k_mean", SAGE_F32, 3, ms))) return st;
        if (!params->smooth_k) return fail(SAGE_ERR_INVALID_ARG, "k_mean given but smooth_k is 0");
    }
    const size_t need = qk_ws_bytes(s, params);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(SAGE_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (workspace && !aligned16(workspace))
        return fail(SAGE_ERR_ALIGNMENT, "workspace not 16-byte aligned");
    if ((st = check_device())) return st;
    if (hadamard) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (dev != hadamard->device)
            return fail(SAGE_ERR_INVALID_ARG, "hadamard lives on device %d, current device is %d",
                        hadamard->device, dev);
    }

    hipStream_t strm = (hipStream_t)stream;
    char* ws = (char*)workspace;
    // K only: the K view stands in for Q with no Q rows (Lq = 0)
    const sage::HalfView qv = half_view(q ? q : k), kv = half_view(k);
    float* mu = nullptr;
    double* partial = nullptr;
    uint64_t* sync = nullptr;
    size_t off = 0;
    if (params->smooth_k) {
        // K channel sums per token chunk (binary64), the mean, head-sync words
        partial = (double*)(ws + off);
        off += align256((size_t)s.B * s.H * sage::mean_chunks(s.Lk) * s.D * sizeof(double));
        mu = k_mean ? (float*)k_mean->data : (float*)(ws + off);
        off += align256((size_t)s.B * s.H * s.D * sizeof(float));
        sync = (uint64_t*)(ws + off);
        off += align256((size_t)sage::quant_sync_words((int64_t)s.B * s.H, s.Lk) * sizeof(uint64_t));
    }
    hipError_t e;
    if (params->mode == SAGE_QK_INT8) {
        e = sage::launch_quant_qk_int8(qv, kv, s.B, s.H, s.Lq, s.Lk, s.D, params->k_block,
                                       params->smooth_k != 0, partial, sync,
                                       k_mean ? (float*)k_mean->data : nullptr,
                                       q ? (int8_t*)q_out->data : nullptr, q ? (float*)q_scale->data : nullptr,
                                       (int8_t*)k_out->data,
                                       (float*)k_scale->data, strm);
    } else {
        if (partial) {
            e = sage::launch_k_mean_partial(kv, s.B, s.H, s.Lk, s.D, partial, strm);
            if (e != hipSuccess) return launch_status(e, "k mean");
            e = sage::launch_k_mean_final(partial, s.B, s.H, s.Lk, s.D, mu, strm);
            if (e != hipSuccess) return launch_status(e, "k mean");
        }
        float* mu_rot = (float*)(ws + off);
        e = sage::launch_quant_qk_mxfp4(
            qv, kv, s.B, s.H, s.Lq, s.Lk, s.D, mu, hadamard ? hadamard->bf16_mat : nullptr,
            hadamard ? hadamard->f16_mat : nullptr, hadamard ? hadamard->inv_sqrt_r : 1.0f, mu_rot,
            q ? (uint8_t*)q_out->data : nullptr, q ? (uint8_t*)q_scale->data : nullptr,
            (uint8_t*)k_out->data, (uint8_t*)k_scale->data, strm);
    }
    return launch_status(e, "quantize qk");
}

sage_status sage_quantize_v_workspace_size(const sage_tensor* v, size_t* bytes) {
    sage_status st = check_half_view(v, "v");
    if (st) return st;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes: null");
    *bytes = v_ws_bytes((int)v->shape[0], (int)v->shape[1], (int)v->shape[2], (int)v->shape[3]);
    return ok();
}

sage_status sage_quantize_v(const sage_tensor* v, const sage_tensor* v_out, const sage_tensor* v_scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
    sage_status st = check_half_view(v, "v");
    if (st) return st;
    const int B = (int)v->shape[0], Lk = (int)v->shape[1], H = (int)v->shape[2], D = (int)v->shape[3];
    if (B < 1 || Lk < 1 || H < 1) return fail(SAGE_ERR_SHAPE, "empty v");
    if (D != 64 && D != 128) return fail(SAGE_ERR_SHAPE, "head dim %d not in {64, 128}", D);
    const int64_t os[4] = {B, H, D, sage::pad128(Lk)}, ss[3] = {B, H, D};
    if ((st = check_exact(v_out, "v_out", SAGE_FP8_E4M3FN, 4, os))) return st;
    if ((st = check_exact(v_scale, "v_scale", SAGE_F32, 3, ss))) return st;
    const size_t need = v_ws_bytes(B, Lk, H, D);
    if (!workspace || workspace_bytes < need)
        return fail(SAGE_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(SAGE_ERR_ALIGNMENT, "workspace not 16-byte aligned");
    if ((st = check_device())) return st;
    const size_t partial_bytes = align256((size_t)B * H * sage::mean_chunks(Lk) * D * sizeof(float));
    hipError_t e = sage::launch_quant_v(half_view(v), B, H, Lk, D, (float*)workspace,
                                        (uint64_t*)((char*)workspace + partial_bytes),
                                        (uint8_t*)v_out->data, (float*)v_scale->data,
                                        (hipStream_t)stream);
    return launch_status(e, "quantize v");
}

sage_status sage_attn_fwd(const sage_tensor* q_q, const sage_tensor* q_scale, const sage_tensor* k_q,
                          const sage_tensor* k_scale, const sage_tensor* v_q, const sage_tensor* v_scale,
                          const sage_attn_params* p, const sage_tensor* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (!p) return fail(SAGE_ERR_INVALID_ARG, "params: null");
    const int B = p->batch, H = p->heads, Lq = p->seqlen_q, Lk = p->seqlen_k, D = p->head_dim;
    const int Hkv = p->num_kv_heads > 0 ? p->num_kv_heads : H;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1) return fail(SAGE_ERR_SHAPE, "empty problem");
    if (H % Hkv) return fail(SAGE_ERR_SHAPE, "heads %d not a multiple of num_kv_heads %d", H, Hkv);
    if (p->qk_mode != SAGE_QK_INT8 && p->qk_mode != SAGE_QK_MXFP4)
        return fail(SAGE_ERR_INVALID_ARG, "params.qk_mode: unknown mode %d", p->qk_mode);
    if (p->causal != 0 && p->causal != 1) return fail(SAGE_ERR_INVALID_ARG, "params.causal must be 0 or 1");
    if (p->causal && Lq != Lk) return fail(SAGE_ERR_UNSUPPORTED, "causal attention needs seqlen_q == seqlen_k");
    if (p->qk_mode == SAGE_QK_MXFP4 && D != 128)
        return fail(SAGE_ERR_SHAPE, "MXFP4 attention needs head dim 128");
    if (D != 64 && D != 128) return fail(SAGE_ERR_SHAPE, "head dim %d not in {64, 128}", D);
    if (!std::isfinite(p->sm_scale)) return fail(SAGE_ERR_INVALID_ARG, "sm_scale is not finite");
    if (p->schedule != SAGE_SCHED_INTERLEAVED && p->schedule != SAGE_SCHED_PINGPONG)
        return fail(SAGE_ERR_INVALID_ARG, "params.schedule: unknown schedule %d", p->schedule);
    if (p->schedule == SAGE_SCHED_PINGPONG && (p->qk_mode != SAGE_QK_INT8 || D != 128))
        return fail(SAGE_ERR_UNSUPPORTED, "the ping-pong schedule needs INT8 QK and head dim 128");
    const int64_t Lqp = sage::pad128(Lq), Lkp = sage::pad128(Lk);
    sage_status st;
    // q_scale NULL: q_q is the fp16/bf16 Q itself, quantized in the kernel's
    // prologue (MXFP4: rotated by params.hadamard when given)
    const bool q_fused = q_scale == nullptr;
    if (p->hadamard && !(q_fused && p->qk_mode == SAGE_QK_MXFP4))
        return fail(SAGE_ERR_INVALID_ARG,
                    "params.hadamard: only used when the kernel quantizes Q to MXFP4 (q_scale NULL)");
    if (p->hadamard && (p->hadamard->R != 128 || D % p->hadamard->R))
        return fail(SAGE_ERR_SHAPE, "params.hadamard: order %d must be 128 and divide D", p->hadamard->R);
    if (q_fused) {
        if ((st = check_half_view(q_q, "q_q"))) return st;
        if (q_q->shape[0] != B || q_q->shape[1] != Lq || q_q->shape[2] != H || q_q->shape[3] != D)
            return fail(SAGE_ERR_SHAPE, "q_q (fp16/bf16 Q) must be [B, Lq, H, D]");
        if (Lq > 1 && q_q->stride[1] < D)
            return fail(SAGE_ERR_LAYOUT, "q_q: rows of one head overlap (token stride < D)");
        if (((int64_t)(Lq - 1) * q_q->stride[1] + D) * 2 > 0x7FFFFF00LL)
            return fail(SAGE_ERR_UNSUPPORTED, "q_q: one head spans more than 2^31 bytes");
    }
    if (p->qk_mode == SAGE_QK_INT8) {
        if (p->q_block != 128) return fail(SAGE_ERR_UNSUPPORTED, "q_block must be 128");
        if (p->k_block != 64 && p->k_block != 128) return fail(SAGE_ERR_UNSUPPORTED, "k_block must be 64 or 128");
        const int64_t qs[4] = {B, H, Lqp, D}, ks[4] = {B, Hkv, Lkp, D};
        const int64_t qss[3] = {B, H, Lqp / p->q_block}, kss[3] = {B, Hkv, Lkp / p->k_block};
        if (!q_fused && (st = check_exact(q_q, "q_q", SAGE_I8, 4, qs))) {
            return st;
        }
        if ((st = check_exact(k_q, "k_q", SAGE_I8, 4, ks))) return st;
        if (!q_fused && (st = check_exact(q_scale, "q_scale", SAGE_F32, 3, qss))) return st;
        if ((st = check_exact(k_scale, "k_scale", SAGE_F32, 3, kss))) return st;
    } else {
        const int64_t qs[4] = {B, H, Lqp, D / 2}, ks[4] = {B, Hkv, Lkp, D / 2};
        const int64_t qe[4] = {B, H, Lqp, D / 32}, ke[4] = {B, Hkv, Lkp, D / 32};
        if (!q_fused && (st = check_exact(q_q, "q_q", SAGE_FP4X2_E2M1, 4, qs))) return st;
        if ((st = check_exact(k_q, "k_q", SAGE_FP4X2_E2M1, 4, ks))) return st;
        if (!q_fused && (st = check_exact(q_scale, "q_scale", SAGE_E8M0, 4, qe))) return st;
        if ((st = check_exact(k_scale, "k_scale", SAGE_E8M0, 4, ke))) return st;
    }
    const int64_t vs[4] = {B, Hkv, D, Lkp}, vss[3] = {B, Hkv, D};
    if ((st = check_exact(v_q, "v_q", SAGE_FP8_E4M3FN, 4, vs))) return st;
    if ((st = check_exact(v_scale, "v_scale", SAGE_F32, 3, vss))) return st;
    if ((st = check_basic(out, "out", 4))) return st;
    if (out->dtype != SAGE_F16 && out->dtype != SAGE_BF16 && out->dtype != SAGE_F32)
        return fail(SAGE_ERR_DTYPE, "out: expected f16, bf16 or f32, got %s", dtype_name(out->dtype));
    if (out->shape[0] != B || out->shape[1] != Lq || out->shape[2] != H || out->shape[3] != D)
        return fail(SAGE_ERR_SHAPE, "out must be [B, Lq, H, D]");
    if (out->stride[3] != 1) return fail(SAGE_ERR_LAYOUT, "out: the head-dim stride must be 1");
    if ((st = check_strides(out, "out"))) return st;
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] > 1 && (out->stride[i] * (int64_t)elem_bytes(out->dtype)) % 16)
            return fail(SAGE_ERR_ALIGNMENT, "out: stride of dim %d is not a multiple of 16 bytes", i);
    if ((st = check_device())) return st;
    if (p->hadamard) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (dev != p->hadamard->device)
            return fail(SAGE_ERR_INVALID_ARG, "params.hadamard lives on device %d, current device is %d",
                        p->hadamard->device, dev);
    }

    sage::AttnArgs a;
    a.q = q_q->data;
    a.q_scale = q_fused ? nullptr : q_scale->data;
    a.q_fused = q_fused ? 1 : 0;
    a.qh = q_fused ? half_view(q_q) : sage::HalfView{nullptr, 0, 0, 0, 0};
    a.hmat_bf16 = p->hadamard ? p->hadamard->bf16_mat : nullptr;
    a.hmat_f16 = p->hadamard ? p->hadamard->f16_mat : nullptr;
    a.inv_sqrt_r = p->hadamard ? p->hadamard->inv_sqrt_r : 1.0f;
    a.k = k_q->data;
    a.k_scale = k_scale->data;
    a.v = (const uint8_t*)v_q->data;
    a.v_scale = (const float*)v_scale->data;
    a.out = sage::OutView{out->data, out->stride[0], out->stride[1], out->stride[2],
                          out->dtype == SAGE_F32 ? sage::kOutF32
                                                 : (out->dtype == SAGE_BF16 ? sage::kOutBF16 : sage::kOutF16)};
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.Lq = Lq;
    a.Lk = Lk;
    a.D = D;
    a.q_block = p->q_block;
    a.k_block = p->k_block;
    a.causal = p->causal;
    a.mxfp4 = p->qk_mode == SAGE_QK_MXFP4;
    a.pingpong = p->schedule == SAGE_SCHED_PINGPONG;
    a.sm_scale = p->sm_scale > 0.0f ? p->sm_scale : (float)(1.0 / std::sqrt((double)D));
    return launch_status(sage::launch_attn_fwd(a, (hipStream_t)stream), "attention");
}

// ---- paged decode -------------------------------------------------------------
namespace {
struct DecShape {
    int B, MTP, Hq, D, splits, rows_pad;
};
sage_status decode_query(const sage_tensor* q, const sage_tensor* page_table,
                         const sage_decode_params* p, DecShape* s) {
    sage_status st = check_basic(q, "q", 4);
    if (st) return st;
    if (q->dtype == SAGE_FP8_E4M3FN || q->dtype == SAGE_FP8_E4M3FNUZ) {
        if ((st = check_fp8(q, "q"))) return st;
    } else if (q->dtype != SAGE_BF16 && q->dtype != SAGE_F16) {
        return fail(SAGE_ERR_DTYPE, "q: expected bf16, f16 or fp8_e4m3fn, got %s", dtype_name(q->dtype));
    }
    if (q->shape[3] > 1 && q->stride[3] != 1) return fail(SAGE_ERR_LAYOUT, "q: head-dim stride must be 1");
    if ((st = check_strides(q, "q"))) return st;
    const int64_t qeb = (int64_t)elem_bytes(q->dtype);
    for (int i = 0; i < 3; ++i)
        if (q->shape[i] > 1 && (q->stride[i] * qeb) % 16)
            return fail(SAGE_ERR_ALIGNMENT, "q: stride of dim %d is not a multiple of 16 bytes", i);
    if (!p) return fail(SAGE_ERR_INVALID_ARG, "params: null");
    if ((st = check_basic(page_table, "page_table", 2))) return st;
    if (page_table->dtype != SAGE_I32) return fail(SAGE_ERR_DTYPE, "page_table: expected i32");
    s->B = (int)q->shape[0];
    s->MTP = (int)q->shape[1];
    s->Hq = (int)q->shape[2];
    s->D = (int)q->shape[3];
    if (s->B < 1 || s->MTP < 1 || s->Hq < 1) return fail(SAGE_ERR_SHAPE, "empty q");
    if (page_table->shape[0] != s->B) return fail(SAGE_ERR_SHAPE, "page_table must have B rows");
    if (p->max_ctx < 1) return fail(SAGE_ERR_INVALID_ARG, "params.max_ctx must be >= 1");
    if (p->window < 0) return fail(SAGE_ERR_INVALID_ARG, "params.window must be >= 0");
    s->splits = sage_decode_num_splits(p->window, s->MTP, p->max_ctx);
    if (p->num_splits < 0) return fail(SAGE_ERR_INVALID_ARG, "params.num_splits must be >= 0");
    if (p->num_splits != 0 && p->num_splits != s->splits)
        return fail(SAGE_ERR_UNSUPPORTED,
                    "params.num_splits %d: only the plan's %d splits (one per 256-token tile) are built",
                    p->num_splits, s->splits);
    s->rows_pad = 64;
    return SAGE_OK;
}
// partial rows: fp16 h[DD] + fp32 m, l, vmax + pad, DD = 128 (D <= 128) or 256
size_t decode_ws(const DecShape& s, int Hkv) {
    const size_t dd = s.D > 128 ? 256 : 128;
    return align256((size_t)s.B * Hkv * s.splits * s.rows_pad * (2 * dd + 16));
}
}  // namespace

sage_status sage_paged_decode_workspace_size(const sage_tensor* q, const sage_tensor* k_cache,
                                             const sage_tensor* page_table,
                                             const sage_decode_params* params, size_t* bytes) {
    DecShape s;
    sage_status st = decode_query(q, page_table, params, &s);
    if (st) return st;
    if ((st = check_basic(k_cache, "k_cache", 4))) return st;
    if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes: null");
    const int Hkv = (int)k_cache->shape[1];
    if (Hkv < 1) return fail(SAGE_ERR_SHAPE, "k_cache has no KV heads");
    *bytes = decode_ws(s, Hkv);
    return ok();
}

namespace {
// Validation and kernel arguments shared by the two decode entry points
// (everything but the partials' memory); *need = bytes of partials.
sage_status decode_setup(const sage_tensor* q, const sage_tensor* k_cache, const sage_tensor* v_cache,
                         const sage_tensor* k_scale, const sage_tensor* v_scale,
                         const sage_tensor* page_table, const sage_tensor* ctx_lens,
                         const sage_decode_params* p, const sage_tensor* out, sage::DecodeArgs* out_args,
                         size_t* need) {
    DecShape s;
    sage_status st = decode_query(q, page_table, p, &s);
    if (st) return st;
    if ((st = check_basic(k_cache, "k_cache", 4))) return st;
    const bool mx = k_cache->dtype == SAGE_FP4X2_E2M1;   // MXFP4 cache: E2M1 codes + E8M0 scales
    if (!mx && (st = check_fp8(k_cache, "k_cache"))) return st;
    if ((st = check_basic(v_cache, "v_cache", 4))) return st;
    if (!mx && (st = check_fp8(v_cache, "v_cache"))) return st;
    const int P = (int)k_cache->shape[0], Hkv = (int)k_cache->shape[1], page = (int)k_cache->shape[2];
    if (k_cache->shape[3] != (mx ? s.D / 2 : s.D)) return fail(SAGE_ERR_SHAPE, "k_cache head dim differs from q");
    if (mx ? s.D != 128 : (s.D != 64 && s.D != 128 && s.D != 256))
        return fail(SAGE_ERR_UNSUPPORTED, "decode head dim must be 64, 128 or 256 (MXFP4 cache: 128)");
    if (Hkv < 1 || s.Hq % Hkv) return fail(SAGE_ERR_SHAPE, "query heads %d not a multiple of KV heads %d", s.Hq, Hkv);
    const int G = s.Hq / Hkv;
    if (G > 64 || s.MTP * G > 64) return fail(SAGE_ERR_UNSUPPORTED, "MTP x (Hq / Hkv) must be <= 64");
    if (page < 16 || page % 16 || !(256 % page == 0 || page % 256 == 0))
        return fail(SAGE_ERR_UNSUPPORTED, "page size %d: need a multiple of 16 that divides 256 or is a multiple of 256", page);
    if (P < 1) return fail(SAGE_ERR_SHAPE, "empty KV pool");
    if (p->v_transposed != 0 && p->v_transposed != 1)
        return fail(SAGE_ERR_INVALID_ARG, "params.v_transposed must be 0 or 1");
    bool per_tensor = false;
    if (mx) {
        if (!p->v_transposed)
            return fail(SAGE_ERR_UNSUPPORTED, "MXFP4 cache: V must be transposed [P, Hkv, D, page/2] "
                        "(its E8M0 blocks run along the keys)");
        if (page % 64) return fail(SAGE_ERR_UNSUPPORTED, "MXFP4 cache: page size %d is not a multiple of 64", page);
        const int64_t ks[4] = {P, Hkv, page, s.D / 2}, vt[4] = {P, Hkv, s.D, page / 2};
        const int64_t kse[4] = {P, Hkv, page, s.D / 32}, vse[4] = {P, Hkv, s.D, page / 32};
        if ((st = check_exact(k_cache, "k_cache", SAGE_FP4X2_E2M1, 4, ks))) return st;
        if ((st = check_exact(v_cache, "v_cache", SAGE_FP4X2_E2M1, 4, vt))) return st;
        if ((st = check_exact(k_scale, "k_scale", SAGE_E8M0, 4, kse))) return st;
        if ((st = check_exact(v_scale, "v_scale", SAGE_E8M0, 4, vse))) return st;
    } else {
        const int64_t ks[4] = {P, Hkv, page, s.D}, vt[4] = {P, Hkv, s.D, page}, ss[3] = {P, Hkv, page};
        const int64_t one[1] = {1};
        if ((st = check_exact(k_cache, "k_cache", SAGE_FP8_E4M3FN, 4, ks))) return st;
        if ((st = check_exact(v_cache, "v_cache", SAGE_FP8_E4M3FN, 4, p->v_transposed ? vt : ks))) return st;
        // per-token scales [P, Hkv, page], or one per tensor [1] (both K and V)
        per_tensor = k_scale && k_scale->ndim == 1;
        if ((st = check_exact(k_scale, "k_scale", SAGE_F32, per_tensor ? 1 : 3, per_tensor ? one : ss))) return st;
        if ((st = check_exact(v_scale, "v_scale", SAGE_F32, per_tensor ? 1 : 3, per_tensor ? one : ss))) return st;
    }
    if (page_table->shape[1] > 1 && page_table->stride[1] != 1)
        return fail(SAGE_ERR_LAYOUT, "page_table rows must be contiguous");
    if ((st = check_strides(page_table, "page_table"))) return st;
    if ((int64_t)page_table->shape[1] * page < p->max_ctx)
        return fail(SAGE_ERR_SHAPE, "page_table covers %lld tokens < max_ctx %d",
                    (long long)page_table->shape[1] * page, p->max_ctx);
    const int64_t cs[1] = {s.B};
    if ((st = check_exact(ctx_lens, "ctx_lens", SAGE_I32, 1, cs))) return st;
    // e4m3 queries carry their scales: F32 [1] (per tensor) or [B, MTP, Hq]
    const bool q8 = q->dtype == SAGE_FP8_E4M3FN;
    bool q_per_tensor = false;
    if (q8) {
        if (!p->q_scale) return fail(SAGE_ERR_INVALID_ARG, "params.q_scale: required for an fp8_e4m3fn q");
        const int64_t one[1] = {1}, rows[3] = {s.B, s.MTP, s.Hq};
        q_per_tensor = p->q_scale->ndim == 1;
        if ((st = check_exact(p->q_scale, "q_scale", SAGE_F32, q_per_tensor ? 1 : 3, q_per_tensor ? one : rows)))
            return st;
    } else if (p->q_scale) {
        return fail(SAGE_ERR_INVALID_ARG, "params.q_scale: only an fp8_e4m3fn q takes scales");
    }
    if ((st = check_basic(out, "out", 4))) return st;
    if (out->dtype != SAGE_BF16 && out->dtype != SAGE_F16)
        return fail(SAGE_ERR_DTYPE, "out: expected bf16 or f16, got %s", dtype_name(out->dtype));
    for (int i = 0; i < 4; ++i)
        if (out->shape[i] != q->shape[i]) return fail(SAGE_ERR_SHAPE, "out must be shaped like q");
    if (out->shape[3] > 1 && out->stride[3] != 1) return fail(SAGE_ERR_LAYOUT, "out: head-dim stride must be 1");
    if ((st = check_strides(out, "out"))) return st;
    for (int i = 0; i < 3; ++i)
        if (out->shape[i] > 1 && (out->stride[i] * 2) % 16)
            return fail(SAGE_ERR_ALIGNMENT, "out: stride of dim %d is not a multiple of 16 bytes", i);
    if (!std::isfinite(p->sm_scale)) return fail(SAGE_ERR_INVALID_ARG, "sm_scale is not finite");
    *need = decode_ws(s, Hkv);
    sage::DecodeArgs& a = *out_args;
    a.q = q->data;
    a.q_sB = q->stride[0];
    a.q_sM = q->stride[1];
    a.q_sH = q->stride[2];
    a.k_cache = (const uint8_t*)k_cache->data;
    a.v_cache = (const uint8_t*)v_cache->data;
    a.k_scale = (const float*)k_scale->data;
    a.v_scale = (const float*)v_scale->data;
    a.page_table = (const int32_t*)page_table->data;
    a.pt_stride = page_table->stride[0];
    a.ctx_lens = (const int32_t*)ctx_lens->data;
    a.out = out->data;
    a.o_sB = out->stride[0];
    a.o_sM = out->stride[1];
    a.o_sH = out->stride[2];
    a.B = s.B;
    a.MTP = s.MTP;
    a.Hq = s.Hq;
    a.Hkv = Hkv;
    a.D = s.D;
    a.page = page;
    a.num_pages = P;
    a.max_pages = (int)page_table->shape[1];
    a.window = p->window;
    a.v_transposed = p->v_transposed;
    a.num_splits = s.splits;
    a.max_ctx = p->max_ctx;
    a.mx = mx ? 1 : 0;
    a.scale_per_tensor = per_tensor ? 1 : 0;
    a.q_kind = q8 ? sage::kQueryE4M3 : (q->dtype == SAGE_F16 ? sage::kQueryF16 : sage::kQueryBF16);
    a.q_scale = q8 ? (const float*)p->q_scale->data : nullptr;
    a.q_scale_per_tensor = q_per_tensor ? 1 : 0;
    a.out_f16 = out->dtype == SAGE_F16 ? 1 : 0;
    a.sm_scale = p->sm_scale > 0.0f ? p->sm_scale : (float)(1.0 / std::sqrt((double)s.D));
    a.partials = nullptr;
    return SAGE_OK;
}
}  // namespace

sage_status sage_paged_decode(const sage_tensor* q, const sage_tensor* k_cache, const sage_tensor* v_cache,
                              const sage_tensor* k_scale, const sage_tensor* v_scale,
                              const sage_tensor* page_table, const sage_tensor* ctx_lens,
                              const sage_decode_params* p, const sage_tensor* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    sage::DecodeArgs a;
    size_t need = 0;
    sage_status st = decode_setup(q, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, p, out, &a, &need);
    if (st) return st;
    if (!workspace || workspace_bytes < need)
        return fail(SAGE_ERR_WORKSPACE, "workspace: need %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(SAGE_ERR_ALIGNMENT, "workspace not 16-byte aligned");
    if ((st = check_device())) return st;
    a.partials = (float*)workspace;
    return launch_status(sage::launch_paged_decode(a, (hipStream_t)stream), "paged decode");
}

sage_status sage_paged_decode_noalloc(const sage_tensor* q, const sage_tensor* k_cache,
                                      const sage_tensor* v_cache, const sage_tensor* k_scale,
                                      const sage_tensor* v_scale, const sage_tensor* page_table,
                                      const sage_tensor* ctx_lens, const sage_decode_params* p,
                                      const sage_tensor* out, void* stream) {
    sage::DecodeArgs a;
    size_t need = 0;
    sage_status st = decode_setup(q, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, p, out, &a, &need);
    if (st) return st;
    if (need > sage::kDecodeScratchBytes)
        return fail(SAGE_ERR_WORKSPACE,
                    "decode needs %zu bytes of partials, above the fixed scratch of %zu bytes "
                    "(use sage_paged_decode with a workspace)", need, sage::kDecodeScratchBytes);
    if ((st = check_device())) return st;
    void* scratch = nullptr;
    hipError_t e = sage::decode_scratch(&scratch);
    if (e != hipSuccess) return launch_status(e, "decode scratch lookup");
    a.partials = (float*)scratch;
    return launch_status(sage::launch_paged_decode(a, (hipStream_t)stream), "paged decode (no allocation)");
}

// ---- Hadamard handle ------------------------------------------------------------
sage_status sage_hadamard_create(int32_t R, int32_t device, void* stream, sage_hadamard** out) {
    if (!out) return fail(SAGE_ERR_INVALID_ARG, "out: null");
    *out = nullptr;
    if (R != 128) return fail(SAGE_ERR_SHAPE, "Hadamard order must be 128 (got %d)", R);
    if (device < 0) return fail(SAGE_ERR_INVALID_ARG, "device must be >= 0");
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return fail(SAGE_ERR_HIP, "hipGetDevice failed");
    if (hipSetDevice(device) != hipSuccess) return fail(SAGE_ERR_HIP, "hipSetDevice(%d) failed", device);
    sage_status st = check_device();
    if (st) {
        (void)hipSetDevice(prev);
        return st;
    }
    sage_hadamard* h = new (std::nothrow) sage_hadamard();
    if (!h) {
        (void)hipSetDevice(prev);
        return fail(SAGE_ERR_INVALID_ARG, "out of host memory");
    }
    h->R = R;
    h->device = device;
    h->inv_sqrt_r = (float)(1.0 / std::sqrt((double)R));
    const size_t bytes = (size_t)R * R * sizeof(uint16_t);
    hipError_t e = hipMalloc(&h->bf16_mat, bytes);
    if (e == hipSuccess) e = hipMalloc(&h->f16_mat, bytes);
    if (e == hipSuccess) e = sage::launch_hadamard_build(R, h->bf16_mat, h->f16_mat, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        if (h->bf16_mat) (void)hipFree(h->bf16_mat);
        if (h->f16_mat) (void)hipFree(h->f16_mat);
        delete h;
        return fail(SAGE_ERR_HIP, "building the Hadamard matrix: %s", hipGetErrorString(e));
    }
    *out = h;
    return ok();
}

sage_status sage_hadamard_destroy(sage_hadamard* h) {
    if (!h) return ok();
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    (void)hipFree(h->bf16_mat);
    (void)hipFree(h->f16_mat);
    (void)hipSetDevice(prev);
    delete h;
    return ok();
}

// ---- test hook -----------------------------------------------------------------
sage_status sage_debug_qk_tile(const sage_tensor* q_q, const sage_tensor* k_q, int32_t q0, int32_t nq,
                               int32_t k0, int32_t nk, const sage_tensor* out, void* stream) {
    sage_status st = check_basic(q_q, "q_q", 4);
    if (st) return st;
    if ((st = check_basic(k_q, "k_q", 4))) return st;
    const int64_t B = q_q->shape[0], H = q_q->shape[1], Lqp = q_q->shape[2], D = q_q->shape[3];
    const int64_t qs[4] = {B, H, Lqp, D};
    if ((st = check_exact(q_q, "q_q", SAGE_I8, 4, qs))) return st;
    const int64_t Lkp = k_q->shape[2];
    const int64_t ks[4] = {B, H, Lkp, D};
    if ((st = check_exact(k_q, "k_q", SAGE_I8, 4, ks))) return st;
    if (D != 64 && D != 128) return fail(SAGE_ERR_SHAPE, "head dim must be 64 or 128");
    if (Lqp % 128 || Lkp % 128) return fail(SAGE_ERR_SHAPE, "q_q / k_q lengths must be padded to 128");
    if (q0 < 0 || nq < 32 || q0 % 32 || nq % 32 || q0 + nq > Lqp)
        return fail(SAGE_ERR_SHAPE, "query range must be 32-aligned and inside q_q");
    if (k0 < 0 || nk < 128 || k0 % 128 || nk % 128 || k0 + nk > Lkp)
        return fail(SAGE_ERR_SHAPE, "key range must be 128-aligned and inside k_q");
    const int64_t os[4] = {B, H, nq, nk};
    if ((st = check_exact(out, "out", SAGE_I32, 4, os))) return st;
    if ((st = check_device())) return st;
    return launch_status(sage::launch_debug_qk((const int8_t*)q_q->data, (const int8_t*)k_q->data, (int)B,
                                               (int)H, (int)Lqp, (int)Lkp, (int)D, q0, nq, k0, nk,
                                               (int32_t*)out->data, (hipStream_t)stream),
                         "debug qk tile");
}

sage_status sage_debug_qk_tile_mx(const sage_tensor* q_q, const sage_tensor* q_scale,
                                  const sage_tensor* k_q, const sage_tensor* k_scale, int32_t q0,
                                  int32_t nq, int32_t k0, int32_t nk, const sage_tensor* out,
                                  void* stream) {
    sage_status st = check_basic(q_q, "q_q", 4);
    if (st) return st;
    if ((st = check_basic(k_q, "k_q", 4))) return st;
    const int64_t B = q_q->shape[0], H = q_q->shape[1], Lqp = q_q->shape[2], Lkp = k_q->shape[2];
    const int64_t D = 2 * q_q->shape[3];
    if (D != 128) return fail(SAGE_ERR_SHAPE, "MXFP4 score tiles need head dim 128 (q_q [B, H, Lqp, 64])");
    const int64_t qs[4] = {B, H, Lqp, D / 2}, ks[4] = {B, H, Lkp, D / 2};
    const int64_t qe[4] = {B, H, Lqp, D / 32}, ke[4] = {B, H, Lkp, D / 32};
    if ((st = check_exact(q_q, "q_q", SAGE_FP4X2_E2M1, 4, qs))) return st;
    if ((st = check_exact(k_q, "k_q", SAGE_FP4X2_E2M1, 4, ks))) return st;
    if ((st = check_exact(q_scale, "q_scale", SAGE_E8M0, 4, qe))) return st;
    if ((st = check_exact(k_scale, "k_scale", SAGE_E8M0, 4, ke))) return st;
    if (Lqp % 128 || Lkp % 128) return fail(SAGE_ERR_SHAPE, "q_q / k_q lengths must be padded to 128");
    if (q0 < 0 || nq < 32 || q0 % 32 || nq % 32 || q0 + nq > Lqp)
        return fail(SAGE_ERR_SHAPE, "query range must be 32-aligned and inside q_q");
    if (k0 < 0 || nk < 128 || k0 % 128 || nk % 128 || k0 + nk > Lkp)
        return fail(SAGE_ERR_SHAPE, "key range must be 128-aligned and inside k_q");
    const int64_t os[4] = {B, H, nq, nk};
    if ((st = check_exact(out, "out", SAGE_F32, 4, os))) return st;
    if ((st = check_device())) return st;
    return launch_status(sage::launch_debug_qk_mx((const uint8_t*)q_q->data, (const uint8_t*)q_scale->data,
                                                  (const uint8_t*)k_q->data, (const uint8_t*)k_scale->data,
                                                  (int)B, (int)H, (int)Lqp, (int)Lkp, q0, nq, k0, nk,
                                                  (float*)out->data, (hipStream_t)stream),
                         "debug qk tile (MXFP4)");
}

sage_status sage_debug_cvt_e4m3(const sage_tensor* x, const sage_tensor* codes, void* stream) {
    sage_status st = check_basic(x, "x", 1);
    if (st) return st;
    const int64_t n = x->shape[0];
    const int64_t shape[1] = {n};
    if ((st = check_exact(x, "x", SAGE_F32, 1, shape))) return st;
    if ((st = check_exact(codes, "codes", SAGE_U8, 1, shape))) return st;
    if (n == 0) return ok();
    if ((st = check_device())) return st;
    return launch_status(sage::launch_debug_cvt_e4m3((const float*)x->data, (uint8_t*)codes->data, n,
                                                     (hipStream_t)stream),
                         "debug e4m3 conversion");
}

sage_status sage_debug_cvt_e2m1(const sage_tensor* x, int32_t exponent, const sage_tensor* codes,
                                void* stream) {
    sage_status st = check_basic(x, "x", 1);
    if (st) return st;
    const int64_t n = x->shape[0];
    const int64_t shape[1] = {n};
    if ((st = check_exact(x, "x", SAGE_F32, 1, shape))) return st;
    if ((st = check_exact(codes, "codes", SAGE_U8, 1, shape))) return st;
    if (exponent < -127 || exponent > 127)
        return fail(SAGE_ERR_INVALID_ARG, "exponent %d outside the E8M0 range [-127, 127]", (int)exponent);
    if (n == 0) return ok();
    if ((st = check_device())) return st;
    return launch_status(sage::launch_debug_cvt_e2m1((const float*)x->data, (uint8_t*)codes->data, n,
                                                     (int)exponent, (hipStream_t)stream),
                         "debug E2M1 conversion");
}

}  // extern "C"

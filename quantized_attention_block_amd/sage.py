"""Python binding of libsage.so (the gfx950 quantized-attention library).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/sage.h.  PyTorch provides device
memory (outputs and workspaces are torch tensors) and the current stream.
If the shared library has not been built this module raises on first use;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SAGE_LIBRARY selects another build of the same library (the host-only
# sanitizer build of the C ABI, whose launchers always fail)
LIB_PATH = os.environ.get("SAGE_LIBRARY") or os.path.join(_HERE, "libsage.so")

# sage_status
OK, ERR_INVALID_ARG, ERR_DTYPE, ERR_SHAPE, ERR_LAYOUT, ERR_ALIGNMENT, ERR_WORKSPACE, \
    ERR_ARCH, ERR_HIP, ERR_UNSUPPORTED = range(10)
STATUS_NAMES = ["SAGE_OK", "SAGE_ERR_INVALID_ARG", "SAGE_ERR_DTYPE", "SAGE_ERR_SHAPE",
                "SAGE_ERR_LAYOUT", "SAGE_ERR_ALIGNMENT", "SAGE_ERR_WORKSPACE", "SAGE_ERR_ARCH",
                "SAGE_ERR_HIP", "SAGE_ERR_UNSUPPORTED"]
# sage_dtype
F16, BF16, F32, I8, I32, U8, FP8_E4M3FN, FP8_E4M3FNUZ, FP4X2_E2M1, E8M0 = range(1, 11)
QK_INT8, QK_MXFP4 = 0, 1
SCHED_INTERLEAVED, SCHED_PINGPONG = 0, 1   # sage_attn_schedule
DECODE_SCRATCH_BYTES = 32 << 20   # SAGE_DECODE_SCRATCH_BYTES: scratch of sage_paged_decode_noalloc

_TORCH_DTYPES = {
    torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32, torch.int8: I8,
    torch.int32: I32, torch.uint8: U8, torch.float8_e4m3fn: FP8_E4M3FN,
    torch.float8_e4m3fnuz: FP8_E4M3FNUZ,
}
# E2M1 pairs and E8M0 scales as torch dtypes (uint8 tensors carry them too,
# with the dtype passed explicitly to desc)
for _name, _code in (("float4_e2m1fn_x2", FP4X2_E2M1), ("float8_e8m0fnu", E8M0)):
    if hasattr(torch, _name):
        _TORCH_DTYPES[getattr(torch, _name)] = _code


class SageError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 10 else status}: {message}")
        self.status = status


class SageTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5), ("stride", ctypes.c_int64 * 5)]


class QkParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("q_block", ctypes.c_int32),
                ("k_block", ctypes.c_int32), ("smooth_k", ctypes.c_int32)]


class AttnParams(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("qk_mode", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("q_block", ctypes.c_int32), ("k_block", ctypes.c_int32),
                ("hadamard", ctypes.c_void_p), ("schedule", ctypes.c_int32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("window", ctypes.c_int32),
                ("v_transposed", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("q_scale", ctypes.POINTER(SageTensor)), ("num_splits", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_T = ctypes.POINTER(SageTensor)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m quantized_attention_block_amd.build` "
                "(hipcc, gfx950). There is no non-HIP fallback.")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        L.sage_last_error.restype = ctypes.c_char_p
        L.sage_version.restype = ctypes.c_int32
        L.sage_attn_kv_tile.restype = ctypes.c_int32
        L.sage_decode_num_splits.argtypes = [ctypes.c_int32] * 3
        L.sage_decode_num_splits.restype = ctypes.c_int32
        L.sage_quantize_qk_workspace_size.argtypes = [_T, _T, ctypes.POINTER(QkParams),
                                                      ctypes.POINTER(ctypes.c_size_t)]
        L.sage_quantize_qk.argtypes = [_T, _T, ctypes.POINTER(QkParams), _T, _T, _T, _T, _T, _P,
                                       _P, ctypes.c_size_t, _P]
        L.sage_quantize_v_workspace_size.argtypes = [_T, ctypes.POINTER(ctypes.c_size_t)]
        L.sage_quantize_v.argtypes = [_T, _T, _T, _P, ctypes.c_size_t, _P]
        L.sage_attn_fwd.argtypes = [_T, _T, _T, _T, _T, _T, ctypes.POINTER(AttnParams), _T, _P,
                                    ctypes.c_size_t, _P]
        L.sage_paged_decode_workspace_size.argtypes = [_T, _T, _T, ctypes.POINTER(DecodeParams),
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.sage_paged_decode.argtypes = [_T, _T, _T, _T, _T, _T, _T, ctypes.POINTER(DecodeParams),
                                        _T, _P, ctypes.c_size_t, _P]
        L.sage_paged_decode_noalloc.argtypes = [_T, _T, _T, _T, _T, _T, _T,
                                                ctypes.POINTER(DecodeParams), _T, _P]
        L.sage_hadamard_create.argtypes = [ctypes.c_int32, ctypes.c_int32, _P,
                                           ctypes.POINTER(ctypes.c_void_p)]
        L.sage_hadamard_destroy.argtypes = [_P]
        L.sage_debug_qk_tile.argtypes = [_T, _T, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _T, _P]
        L.sage_debug_qk_tile_mx.argtypes = [_T, _T, _T, _T, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _T, _P]
        L.sage_set_quant_wait_us.argtypes = [ctypes.c_int32]
        L.sage_debug_cvt_e4m3.argtypes = [_T, _T, _P]
        L.sage_debug_cvt_e2m1.argtypes = [_T, ctypes.c_int32, _T, _P]
        for name in ("sage_quantize_qk_workspace_size", "sage_quantize_qk",
                     "sage_quantize_v_workspace_size", "sage_quantize_v", "sage_attn_fwd",
                     "sage_paged_decode_workspace_size", "sage_paged_decode",
                     "sage_paged_decode_noalloc",
                     "sage_hadamard_create", "sage_hadamard_destroy", "sage_debug_qk_tile",
                     "sage_debug_qk_tile_mx", "sage_set_quant_wait_us", "sage_debug_cvt_e4m3",
                     "sage_debug_cvt_e2m1"):
            getattr(L, name).restype = st
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise SageError(status, lib().sage_last_error().decode())


def desc(t: Optional[torch.Tensor], dtype: Optional[int] = None) -> Optional[SageTensor]:
    """sage_tensor descriptor of a torch tensor (shape and element strides as
    torch reports them); `dtype` overrides the element type for uint8 tensors
    that carry FP4X2 or E8M0 codes."""
    if t is None:
        return None
    d = SageTensor()
    d.data = t.data_ptr()
    d.dtype = dtype if dtype is not None else _TORCH_DTYPES.get(t.dtype, 0)
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.stride[i] = st
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def pad128(L: int) -> int:
    return (L + 127) // 128 * 128


class Hadamard:
    """Order-128 Sylvester Hadamard rotation kept on one device, built once
    and reused by every MXFP4 quantization (sage_hadamard_create)."""

    def __init__(self, device: int = 0, R: int = 128):
        h = ctypes.c_void_p()
        _check(lib().sage_hadamard_create(R, device, _stream(torch.device("cuda", device)),
                                          ctypes.byref(h)))
        self.handle = h
        self.R = R
        self.device = device

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.sage_hadamard_destroy(self.handle)
            self.handle = None


@dataclass
class QuantizedQK:
    mode: int
    q: torch.Tensor        # INT8 [B,H,Lqp,D] or FP4X2 (uint8) [B,H,Lqp,D/2]
    q_scale: torch.Tensor  # F32 [B,H,Lqp/q_block] or E8M0 (uint8) [B,H,Lqp,D/32]
    k: torch.Tensor
    k_scale: torch.Tensor
    k_mean: Optional[torch.Tensor]
    Lq: int
    Lk: int
    q_block: int
    k_block: int


def sage_quantize_qk(q: torch.Tensor, k: torch.Tensor, *, mode: int = QK_INT8, q_block: int = 128,
                     k_block: int = 64, smooth_k: bool = True,
                     hadamard: Optional[Hadamard] = None, want_mean: bool = True,
                     workspace: Optional[torch.Tensor] = None,
                     into: Optional[QuantizedQK] = None) -> QuantizedQK:
    """q, k: logical [B, L, H, D] fp16/bf16 (any B/L/H strides).  `into`
    reuses the output tensors of an earlier call with the same shapes.  q None:
    K alone; Q is then quantized inside sage_attn_fwd(q=...) (MXFP4: pass the
    same hadamard there)."""
    B, Lk, H, D = k.shape
    Lq = q.shape[1] if q is not None else 0
    dev = k.device
    if into is not None:
        q_out, q_sc, k_out, k_sc, mean = into.q, into.q_scale, into.k, into.k_scale, into.k_mean
        if mode == QK_INT8:
            qd, kd, qsd, ksd = desc(q_out), desc(k_out), desc(q_sc), desc(k_sc)
        else:
            qd, kd = desc(q_out, FP4X2_E2M1), desc(k_out, FP4X2_E2M1)
            qsd, ksd = desc(q_sc, E8M0), desc(k_sc, E8M0)
    elif mode == QK_INT8 and q is None:
        q_out = q_sc = None
        k_out = torch.empty((B, H, pad128(Lk), D), dtype=torch.int8, device=dev)
        k_sc = torch.empty((B, H, pad128(Lk) // k_block), dtype=torch.float32, device=dev)
        qd, kd, qsd, ksd = None, desc(k_out), None, desc(k_sc)
    elif q is None:
        q_out = q_sc = None
        k_out = torch.empty((B, H, pad128(Lk), D // 2), dtype=torch.uint8, device=dev)
        k_sc = torch.empty((B, H, pad128(Lk), D // 32), dtype=torch.uint8, device=dev)
        qd, qsd = None, None
        kd, ksd = desc(k_out, FP4X2_E2M1), desc(k_sc, E8M0)
    elif mode == QK_INT8:
        q_out = torch.empty((B, H, pad128(Lq), D), dtype=torch.int8, device=dev)
        k_out = torch.empty((B, H, pad128(Lk), D), dtype=torch.int8, device=dev)
        q_sc = torch.empty((B, H, pad128(Lq) // q_block), dtype=torch.float32, device=dev)
        k_sc = torch.empty((B, H, pad128(Lk) // k_block), dtype=torch.float32, device=dev)
        qd, kd, qsd, ksd = desc(q_out), desc(k_out), desc(q_sc), desc(k_sc)
    else:
        q_out = torch.empty((B, H, pad128(Lq), D // 2), dtype=torch.uint8, device=dev)
        k_out = torch.empty((B, H, pad128(Lk), D // 2), dtype=torch.uint8, device=dev)
        q_sc = torch.empty((B, H, pad128(Lq), D // 32), dtype=torch.uint8, device=dev)
        k_sc = torch.empty((B, H, pad128(Lk), D // 32), dtype=torch.uint8, device=dev)
        qd, kd = desc(q_out, FP4X2_E2M1), desc(k_out, FP4X2_E2M1)
        qsd, ksd = desc(q_sc, E8M0), desc(k_sc, E8M0)
    if into is None:
        mean = (torch.empty((B, H, D), dtype=torch.float32, device=dev)
                if (smooth_k and want_mean) else None)
    prm = QkParams(mode, q_block, k_block, int(smooth_k))
    qv, kv = desc(q), desc(k)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_quantize_qk_workspace_size(_ref(qv), ctypes.byref(kv),
                                                 ctypes.byref(prm), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = _workspace(nbytes.value, dev)
    _check(lib().sage_quantize_qk(_ref(qv), ctypes.byref(kv), ctypes.byref(prm),
                                  _ref(qd), _ref(qsd), ctypes.byref(kd),
                                  ctypes.byref(ksd), _ref(desc(mean)),
                                  hadamard.handle if hadamard is not None else None,
                                  ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                  _stream(dev)))
    return QuantizedQK(mode, q_out, q_sc, k_out, k_sc, mean, Lq, Lk, q_block, k_block)


def sage_quantize_qk_workspace_size(q: torch.Tensor, k: torch.Tensor, *, mode: int = QK_INT8,
                                    q_block: int = 128, k_block: int = 64,
                                    smooth_k: bool = True) -> int:
    """Bytes of device workspace sage_quantize_qk needs for these inputs."""
    prm = QkParams(mode, q_block, k_block, int(smooth_k))
    nbytes = ctypes.c_size_t()
    _check(lib().sage_quantize_qk_workspace_size(_ref(desc(q)), ctypes.byref(desc(k)),
                                                 ctypes.byref(prm), ctypes.byref(nbytes)))
    return int(nbytes.value)


def sage_set_quant_wait_us(us: int) -> None:
    """Microseconds a block of the single-read quantizers waits for the rest
    of its head before computing the head's statistic itself (process-wide;
    the outputs are the same either way)."""
    _check(lib().sage_set_quant_wait_us(int(us)))


def sage_quantize_v_workspace_size(v: torch.Tensor) -> int:
    """Bytes of device workspace sage_quantize_v needs for this input."""
    nbytes = ctypes.c_size_t()
    _check(lib().sage_quantize_v_workspace_size(ctypes.byref(desc(v)), ctypes.byref(nbytes)))
    return int(nbytes.value)


def sage_quantize_v(v: torch.Tensor, workspace: Optional[torch.Tensor] = None, into=None):
    """v: logical [B, Lk, H, D] fp16/bf16.  Returns (e4m3 [B,H,D,pad128(Lk)],
    fp32 per-channel scales [B,H,D]); `into` reuses such a pair."""
    B, Lk, H, D = v.shape
    dev = v.device
    if into is not None:
        v_out, v_sc = into
    else:
        v_out = torch.empty((B, H, D, pad128(Lk)), dtype=torch.float8_e4m3fn, device=dev)
        v_sc = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    vd = desc(v)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_quantize_v_workspace_size(ctypes.byref(vd), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = _workspace(nbytes.value, dev)
    _check(lib().sage_quantize_v(ctypes.byref(vd), ctypes.byref(desc(v_out)),
                                 ctypes.byref(desc(v_sc)), ctypes.c_void_p(workspace.data_ptr()),
                                 workspace.numel(), _stream(dev)))
    return v_out, v_sc


def sage_attn_fwd(qk: QuantizedQK, v_q: torch.Tensor, v_scale: torch.Tensor, *, causal: bool = False,
                  sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.bfloat16, num_kv_heads: int = 0,
                  q: Optional[torch.Tensor] = None,
                  hadamard: Optional[Hadamard] = None,
                  schedule: int = SCHED_INTERLEAVED) -> torch.Tensor:
    """Quantized attention; `out` is a logical [B, Lq, H, D] fp16/bf16 tensor
    with any B/L/H strides (allocated contiguous when None).  When qk holds K
    alone (sage_quantize_qk(None, k)), `q` is the fp16/bf16 [B, Lq, H, D] Q,
    quantized in the kernel's prologue to the same codes and scales as
    sage_quantize_qk's (MXFP4: rotated by `hadamard`, None for no rotation).
    `schedule`: SCHED_INTERLEAVED or SCHED_PINGPONG (same output bits)."""
    if (qk.q is None) != (q is not None):
        raise ValueError("pass q exactly when qk was quantized without Q")
    if q is not None:
        B, Lq, H, _ = q.shape
    else:
        B, H, _, _ = qk.q.shape
        Lq = qk.Lq
    D = v_q.shape[2]
    dev = qk.k.device
    if out is None:
        out = torch.empty((B, Lq, H, D), dtype=out_dtype, device=dev)
    prm = AttnParams(float(sm_scale), int(causal), qk.mode, B, H, Lq, qk.Lk, D,
                     num_kv_heads, qk.q_block, qk.k_block,
                     hadamard.handle if hadamard is not None else None, int(schedule))
    mx = qk.mode == QK_MXFP4
    kd = desc(qk.k, FP4X2_E2M1) if mx else desc(qk.k)
    ksd = desc(qk.k_scale, E8M0) if mx else desc(qk.k_scale)
    if q is not None:
        qd, qsd = desc(q), None
    elif not mx:
        qd, qsd = desc(qk.q), desc(qk.q_scale)
    else:
        qd, qsd = desc(qk.q, FP4X2_E2M1), desc(qk.q_scale, E8M0)
    _check(lib().sage_attn_fwd(ctypes.byref(qd), _ref(qsd), ctypes.byref(kd),
                               ctypes.byref(ksd), ctypes.byref(desc(v_q)),
                               ctypes.byref(desc(v_scale)), ctypes.byref(prm),
                               ctypes.byref(desc(out)), None, 0, _stream(dev)))
    return out


def sage_attention(q, k, v, *, causal=False, sm_scale=0.0, mode=QK_INT8, k_block=64,
                   hadamard: Optional[Hadamard] = None, out=None):
    """quantize_qk (K) + quantize_v + attn_fwd on strided [B, L, H, D] inputs,
    Q quantized inside the attention kernel (INT8, or MXFP4 rotated by
    `hadamard`)."""
    qk = sage_quantize_qk(None, k, mode=mode, k_block=k_block, hadamard=hadamard, want_mean=False)
    v_q, v_s = sage_quantize_v(v)
    return sage_attn_fwd(qk, v_q, v_s, causal=causal, sm_scale=sm_scale, out=out,
                         out_dtype=q.dtype, q=q, hadamard=hadamard if mode == QK_MXFP4 else None)


def sage_attn_kv_tile() -> int:
    """Keys per KV tile of sage_attn_fwd's online softmax."""
    return int(lib().sage_attn_kv_tile())


def sage_decode_num_splits(window: int, mtp: int, max_ctx: int) -> int:
    return int(lib().sage_decode_num_splits(window, mtp, max_ctx))


def _decode_params(sm_scale, window, v_transposed, max_ctx, q_scale, num_splits=0):
    """DecodeParams plus the descriptor it points to (kept alive by the caller)."""
    qsd = desc(q_scale) if q_scale is not None else None
    prm = DecodeParams(float(sm_scale), int(window), int(v_transposed), int(max_ctx),
                       ctypes.pointer(qsd) if qsd is not None else None, int(num_splits))
    return prm, qsd


def sage_paged_decode(q, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, *, max_ctx: int,
                      window: int = 0, sm_scale: float = 0.0, v_transposed: bool = True,
                      q_scale: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, num_splits: int = 0) -> torch.Tensor:
    """q bf16 / fp16 [B, MTP, Hq, D], or e4m3 with fp32 `q_scale` ([1] or
    [B, MTP, Hq]); caches e4m3 [P, Hkv, page, D] (V transposed: [P, Hkv, D,
    page], or plain like K with v_transposed False) with fp32 scales
    [P, Hkv, page] or [1], or MXFP4 caches (torch.float4_e2m1fn_x2) K
    [P, Hkv, page, D/2], V [P, Hkv, D, page/2] with E8M0 scales
    (torch.float8_e8m0fnu) K [P, Hkv, page, D/32] and V [P, Hkv, D, page/32];
    page_table int32 [B, pages]; ctx_lens int32 [B].  `out` (allocated when
    None) is bf16 or fp16 shaped like q; by default q's dtype, bf16 for an
    e4m3 q."""
    if out is None:
        odt = q.dtype if q.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    prm, _keep = _decode_params(sm_scale, window, v_transposed, max_ctx, q_scale, num_splits)
    qd, ptd, kcd = desc(q), desc(page_table), desc(k_cache)
    if workspace is None:
        nbytes = ctypes.c_size_t()
        _check(lib().sage_paged_decode_workspace_size(ctypes.byref(qd), ctypes.byref(kcd),
                                                      ctypes.byref(ptd), ctypes.byref(prm),
                                                      ctypes.byref(nbytes)))
        workspace = _workspace(nbytes.value, q.device)
    _check(lib().sage_paged_decode(ctypes.byref(qd), ctypes.byref(kcd),
                                   ctypes.byref(desc(v_cache)), ctypes.byref(desc(k_scale)),
                                   ctypes.byref(desc(v_scale)), ctypes.byref(ptd),
                                   ctypes.byref(desc(ctx_lens)), ctypes.byref(prm),
                                   ctypes.byref(desc(out)), ctypes.c_void_p(workspace.data_ptr()),
                                   workspace.numel(), _stream(q.device)))
    return out


def sage_paged_decode_noalloc(q, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, out, *,
                              max_ctx: int, window: int = 0, sm_scale: float = 0.0,
                              v_transposed: bool = True, q_scale: Optional[torch.Tensor] = None,
                              num_splits: int = 0) -> torch.Tensor:
    """sage_paged_decode without a workspace: the library's fixed per-device
    scratch holds the split partials (calls that overlap on one device race).
    `out` is required; nothing is allocated."""
    prm, _keep = _decode_params(sm_scale, window, v_transposed, max_ctx, q_scale, num_splits)
    _check(lib().sage_paged_decode_noalloc(ctypes.byref(desc(q)), ctypes.byref(desc(k_cache)),
                                           ctypes.byref(desc(v_cache)), ctypes.byref(desc(k_scale)),
                                           ctypes.byref(desc(v_scale)), ctypes.byref(desc(page_table)),
                                           ctypes.byref(desc(ctx_lens)), ctypes.byref(prm),
                                           ctypes.byref(desc(out)), _stream(q.device)))
    return out


def sage_paged_decode_workspace_size(q, k_cache, page_table, *, max_ctx: int, window: int = 0) -> int:
    prm = DecodeParams(0.0, int(window), 1, int(max_ctx), None)
    nbytes = ctypes.c_size_t()
    _check(lib().sage_paged_decode_workspace_size(ctypes.byref(desc(q)), ctypes.byref(desc(k_cache)),
                                                  ctypes.byref(desc(page_table)),
                                                  ctypes.byref(prm), ctypes.byref(nbytes)))
    return nbytes.value


def sage_debug_qk_tile(q_q: torch.Tensor, k_q: torch.Tensor, q0: int, nq: int, k0: int,
                       nk: int) -> torch.Tensor:
    B, H = q_q.shape[:2]
    out = torch.empty((B, H, nq, nk), dtype=torch.int32, device=q_q.device)
    _check(lib().sage_debug_qk_tile(ctypes.byref(desc(q_q)), ctypes.byref(desc(k_q)), q0, nq, k0,
                                    nk, ctypes.byref(desc(out)), _stream(q_q.device)))
    return out


def sage_debug_qk_tile_mx(qk: QuantizedQK, q0: int, nq: int, k0: int, nk: int) -> torch.Tensor:
    """fp32 MXFP4 score tile of the attention kernel's QK step (test hook)."""
    B, H = qk.q.shape[:2]
    out = torch.empty((B, H, nq, nk), dtype=torch.float32, device=qk.q.device)
    _check(lib().sage_debug_qk_tile_mx(ctypes.byref(desc(qk.q, FP4X2_E2M1)),
                                       ctypes.byref(desc(qk.q_scale, E8M0)),
                                       ctypes.byref(desc(qk.k, FP4X2_E2M1)),
                                       ctypes.byref(desc(qk.k_scale, E8M0)), q0, nq, k0, nk,
                                       ctypes.byref(desc(out)), _stream(qk.q.device)))
    return out


def sage_debug_cvt_e4m3(x: torch.Tensor) -> torch.Tensor:
    """uint8 e4m3 codes of the fp32 device vector x by the kernels' conversion
    (test hook)."""
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if x.numel():
        _check(lib().sage_debug_cvt_e4m3(ctypes.byref(desc(x)), ctypes.byref(desc(codes)), _stream(x.device)))
    return codes


def sage_debug_cvt_e2m1(x: torch.Tensor, exponent: int) -> torch.Tensor:
    """uint8 E2M1 codes (low nibble) of x * 2^-exponent by the MXFP4
    quantizer's conversion (test hook)."""
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if x.numel():
        _check(lib().sage_debug_cvt_e2m1(ctypes.byref(desc(x)), exponent, ctypes.byref(desc(codes)),
                                         _stream(x.device)))
    return codes


def default_sm_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)

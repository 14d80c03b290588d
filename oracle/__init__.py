"""ctypes wrapper of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module to compute expected values.  Nothing in the
HIP library or its Python binding imports it.

Arrays are numpy, in the oracle's canonical contiguous layouts (see oracle.h).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
BUILT_PATH = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIBRARY selects another build of oracle.cpp (the sanitizer build)
LIB_PATH = os.environ.get("ORACLE_LIBRARY") or BUILT_PATH
SOURCES = [os.path.join(_HERE, "oracle.cpp")]

QK_INT8, QK_MXFP4, QK_FLOAT = 0, 1, 2


def build(force: bool = True) -> str:
    """Compiles liboracle.so with g++ (plain C++17, no fast-math, no FMA
    contraction)."""
    if not force and os.path.exists(BUILT_PATH):
        return BUILT_PATH
    tmp = BUILT_PATH + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", "-Wall", "-o", tmp] + SOURCES
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, BUILT_PATH)
    return BUILT_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


class AttnParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("Lq", ctypes.c_int),
                ("Lk", ctypes.c_int), ("D", ctypes.c_int), ("causal", ctypes.c_int),
                ("sm_scale", ctypes.c_double), ("BN", ctypes.c_int), ("qk_mode", ctypes.c_int),
                ("q_block", ctypes.c_int), ("k_block", ctypes.c_int), ("quant_pv", ctypes.c_int),
                ("nthreads", ctypes.c_int)]


_P = ctypes.c_void_p


class AttnInputs(ctypes.Structure):
    _fields_ = [("q8", _P), ("q_scale", _P), ("k8", _P), ("k_scale", _P),
                ("q4", _P), ("q_e8", _P), ("k4", _P), ("k_e8", _P),
                ("qf", _P), ("kf", _P), ("v8", _P), ("v_scale", _P), ("vf", _P)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("MTP", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("D", ctypes.c_int), ("page_size", ctypes.c_int),
                ("max_pages", ctypes.c_int), ("num_pages", ctypes.c_int), ("window", ctypes.c_int),
                ("tile", ctypes.c_int), ("sm_scale", ctypes.c_double), ("quant", ctypes.c_int),
                ("nthreads", ctypes.c_int), ("q8", ctypes.c_void_p), ("q8_scale", ctypes.c_void_p),
                ("q8_scale_per_tensor", ctypes.c_int)]


def _declare(L):
    u8, f32, i32 = ctypes.c_uint8, ctypes.c_float, ctypes.c_int
    i64 = ctypes.c_int64
    L.orc_e4m3_encode.argtypes = [f32]; L.orc_e4m3_encode.restype = u8
    L.orc_e4m3_decode.argtypes = [u8]; L.orc_e4m3_decode.restype = f32
    L.orc_e2m1_encode.argtypes = [f32]; L.orc_e2m1_encode.restype = u8
    L.orc_e2m1_decode.argtypes = [u8]; L.orc_e2m1_decode.restype = f32
    L.orc_e8m0_decode.argtypes = [u8]; L.orc_e8m0_decode.restype = f32
    L.orc_mx_shared_exponent.argtypes = [f32]; L.orc_mx_shared_exponent.restype = i32
    L.orc_bf16_round.argtypes = [f32]; L.orc_bf16_round.restype = ctypes.c_uint16
    L.orc_fp16_round.argtypes = [f32]; L.orc_fp16_round.restype = ctypes.c_uint16
    L.orc_e4m3_encode_array.argtypes = [_P, i64, _P]; L.orc_e4m3_encode_array.restype = None
    L.orc_e4m3_decode_array.argtypes = [_P, i64, _P]; L.orc_e4m3_decode_array.restype = None
    L.orc_e2m1_code_scaled.argtypes = [f32, i32]; L.orc_e2m1_code_scaled.restype = u8
    L.orc_e2m1_code_scaled_array.argtypes = [_P, i64, i32, _P]
    L.orc_e2m1_code_scaled_array.restype = None
    L.orc_hadamard.argtypes = [i32, _P]; L.orc_hadamard.restype = None
    L.orc_k_mean.argtypes = [_P, i32, i32, i32, i32, _P]; L.orc_k_mean.restype = None
    L.orc_smooth_k.argtypes = [_P, _P, i32, i32, i32, i32, _P]; L.orc_smooth_k.restype = None
    L.orc_quant_int8.argtypes = [_P, i32, i32, i32, i32, i32, _P, _P]
    L.orc_quant_int8.restype = None
    L.orc_quant_v_fp8.argtypes = [_P, i32, i32, i32, i32, _P, _P]
    L.orc_quant_v_fp8.restype = None
    L.orc_rotate.argtypes = [_P, i32, i32, i32, i32, i32, _P]; L.orc_rotate.restype = None
    L.orc_quant_mxfp4.argtypes = [_P, i32, i32, i32, i32, _P, _P]
    L.orc_quant_mxfp4.restype = None
    L.orc_qk_int8_exact.argtypes = [_P, _P, i32]; L.orc_qk_int8_exact.restype = i64
    L.orc_attn_emulated.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(AttnInputs),
                                    _P, i64, _P]
    L.orc_attn_emulated.restype = i32
    L.orc_attn_exact.argtypes = [_P, _P, _P, i32, i32, i32, i32, i32, i32, ctypes.c_double,
                                 _P, i64, i32, _P]
    L.orc_attn_exact.restype = i32
    L.orc_decode_num_splits.argtypes = [i32, i32, i32]; L.orc_decode_num_splits.restype = i32
    L.orc_paged_decode.argtypes = [ctypes.POINTER(DecodeParams), _P, _P, _P, _P, _P, _P, _P, _P]
    L.orc_paged_decode.restype = i32
    L.orc_paged_decode_mx.argtypes = [ctypes.POINTER(DecodeParams), _P, _P, _P, _P, _P, _P, _P, _P]
    L.orc_paged_decode_mx.restype = i32


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---- scalar codecs ---------------------------------------------------------
def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def e2m1_encode(x: float) -> int:
    return int(lib().orc_e2m1_encode(float(x)))


def e2m1_decode(c: int) -> float:
    return float(lib().orc_e2m1_decode(int(c)))


def e8m0_decode(c: int) -> float:
    return float(lib().orc_e8m0_decode(int(c)))


def mx_shared_exponent(amax: float) -> int:
    return int(lib().orc_mx_shared_exponent(float(amax)))


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    f = lib().orc_bf16_round
    flat = np.asarray(x, dtype=np.float32).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def fp16_round_bits(x: np.ndarray) -> np.ndarray:
    f = lib().orc_fp16_round
    flat = np.asarray(x, dtype=np.float32).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_code_scaled(x: float, e: int) -> int:
    """E2M1 code of x * 2^-e (an element of an MX block with shared exponent e)."""
    return int(lib().orc_e2m1_code_scaled(x, e))


def e2m1_code_scaled_array(x: np.ndarray, e: int) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e2m1_code_scaled_array(_ptr(x), x.size, e, _ptr(out))
    return out


def e4m3_decode_array(c: np.ndarray) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().orc_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def hadamard(R: int) -> np.ndarray:
    out = np.empty((R, R), dtype=np.float32)
    lib().orc_hadamard(R, _ptr(out))
    return out


# ---- quantizers (canonical [B,H,L,D] float32 inputs) -----------------------
def k_mean(k: np.ndarray) -> np.ndarray:
    k = _c(k, np.float32)
    B, H, L, D = k.shape
    mu = np.empty((B, H, D), dtype=np.float32)
    lib().orc_k_mean(_ptr(k), B, H, L, D, _ptr(mu))
    return mu


def smooth_k(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    k = _c(k, np.float32)
    mu = _c(mu, np.float32)
    B, H, L, D = k.shape
    out = np.empty_like(k)
    lib().orc_smooth_k(_ptr(k), _ptr(mu), B, H, L, D, _ptr(out))
    return out


def quant_int8(x: np.ndarray, block: int):
    x = _c(x, np.float32)
    B, H, L, D = x.shape
    nb = (L + block - 1) // block
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    lib().orc_quant_int8(_ptr(x), B, H, L, D, block, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_v_fp8(v: np.ndarray):
    v = _c(v, np.float32)
    B, H, L, D = v.shape
    codes = np.empty(v.shape, dtype=np.uint8)
    scales = np.empty((B, H, D), dtype=np.float32)
    lib().orc_quant_v_fp8(_ptr(v), B, H, L, D, _ptr(codes), _ptr(scales))
    return codes, scales


def rotate(x: np.ndarray, R: int = 128) -> np.ndarray:
    x = _c(x, np.float32)
    B, H, L, D = x.shape
    out = np.empty_like(x)
    lib().orc_rotate(_ptr(x), B, H, L, D, R, _ptr(out))
    return out


def quant_mxfp4(x: np.ndarray):
    x = _c(x, np.float32)
    B, H, L, D = x.shape
    codes = np.empty(x.shape, dtype=np.uint8)
    e8 = np.empty((B, H, L, D // 32), dtype=np.uint8)
    lib().orc_quant_mxfp4(_ptr(x), B, H, L, D, _ptr(codes), _ptr(e8))
    return codes, e8


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Packs one-per-byte E2M1 codes two per byte, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def qk_int8_tile(q8: np.ndarray, k8: np.ndarray) -> np.ndarray:
    """Exact integer S = Q8 K8^T for [..., M, D] x [..., N, D] codes (int64)."""
    return np.matmul(q8.astype(np.int64), np.swapaxes(k8.astype(np.int64), -1, -2))


def qk_mxfp4_tile(q4: np.ndarray, q_e8: np.ndarray, k4: np.ndarray, k_e8: np.ndarray,
                  partial_blocks: Optional[int] = None) -> np.ndarray:
    """Exact S = Q K^T of MXFP4 operands (one E2M1 code per byte, [..., M, D]
    and [..., N, D], E8M0 scales [..., M, D/32] and [..., N, D/32]) in float64:
    per 32-channel block the integer sum of (2 e2m1_q)(2 e2m1_k) times
    2^(e_q + e_k - 2), e = E8M0 code - 127.  partial_blocks: sum only the
    first that many blocks.  Exact for every input of this library (block sums
    < 2^13, exponents within binary64's range)."""
    dec2 = np.array([int(round(2 * e2m1_decode(c))) for c in range(16)], np.int64)
    qi, ki = dec2[np.asarray(q4)], dec2[np.asarray(k4)]
    nb = qi.shape[-1] // 32 if partial_blocks is None else partial_blocks
    S = 0.0
    for b in range(nb):
        sl = slice(32 * b, 32 * b + 32)
        isum = np.matmul(qi[..., sl], np.swapaxes(ki[..., sl], -1, -2))
        ex = (np.asarray(q_e8, np.int64)[..., b][..., :, None] - 127) + \
             (np.asarray(k_e8, np.int64)[..., b][..., None, :] - 127) - 2
        S = S + np.ldexp(isum.astype(np.float64), ex)
    return S


# ---- attention -------------------------------------------------------------
def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = _c(np.asarray(rows).reshape(-1, 3), np.int32)
    return r, r.shape[0]


def attn_emulated(*, B, H, Lq, Lk, D, causal, sm_scale, BN, qk_mode, q_block=128,
                  k_block=64, quant_pv=True, rows=None, nthreads=0,
                  q8=None, q_scale=None, k8=None, k_scale=None,
                  q4=None, q_e8=None, k4=None, k_e8=None, qf=None, kf=None,
                  v8=None, v_scale=None, vf=None) -> np.ndarray:
    p = AttnParams(B, H, Lq, Lk, D, int(causal), float(sm_scale), BN, qk_mode, q_block,
                   k_block, int(quant_pv), nthreads)
    keep = []

    def arr(a, dt):
        if a is None:
            return None
        a = _c(a, dt)
        keep.append(a)
        return _ptr(a)

    ins = AttnInputs(arr(q8, np.int8), arr(q_scale, np.float32), arr(k8, np.int8),
                     arr(k_scale, np.float32), arr(q4, np.uint8), arr(q_e8, np.uint8),
                     arr(k4, np.uint8), arr(k_e8, np.uint8), arr(qf, np.float32),
                     arr(kf, np.float32), arr(v8, np.uint8), arr(v_scale, np.float32),
                     arr(vf, np.float32))
    r, n = _rows_arg(rows)
    nout = n if r is not None else B * H * Lq
    out = np.empty((nout, D), dtype=np.float32)
    rc = lib().orc_attn_emulated(ctypes.byref(p), ctypes.byref(ins), _ptr(r), n, _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_attn_emulated failed ({rc})")
    return out if r is not None else out.reshape(B, H, Lq, D)


def attn_exact(q, k, v, causal, sm_scale, rows=None, nthreads=0) -> np.ndarray:
    q, k, v = (_c(a, np.float32) for a in (q, k, v))
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    r, n = _rows_arg(rows)
    nout = n if r is not None else B * H * Lq
    out = np.empty((nout, D), dtype=np.float64)
    lib().orc_attn_exact(_ptr(q), _ptr(k), _ptr(v), B, H, Lq, Lk, D, int(causal),
                         float(sm_scale), _ptr(r), n, nthreads, _ptr(out))
    return out if r is not None else out.reshape(B, H, Lq, D)


def decode_num_splits(window: int, mtp: int, tile: int = 256) -> int:
    return int(lib().orc_decode_num_splits(window, mtp, tile))


def _q8_fields(prm, q8, q8_scale, keep):
    """Fills the pre-quantized query fields: q8 uint8 codes shaped like q,
    q8_scale float32 [B, MTP, Hq] (per row) or [1] (per tensor)."""
    if q8 is None:
        return
    c, s = _c(q8, np.uint8), _c(q8_scale, np.float32)
    keep += [c, s]
    prm.q8, prm.q8_scale = c.ctypes.data, s.ctypes.data
    prm.q8_scale_per_tensor = int(s.size == 1)


def paged_decode(q, k_cache, v_cache, k_scale, v_scale, page_table, ctx_lens, *, window,
                 sm_scale, tile=256, quant=True, nthreads=0, q8=None, q8_scale=None) -> np.ndarray:
    """q: [B, MTP, Hq, D] float32; caches [P, Hkv, page, D] (uint8 codes when
    quant, else float32); scales [P, Hkv, page]; page_table [B, max_pages].
    q8 / q8_scale: the query given in e4m3 (codes shaped like q, fp32 scales
    [B, MTP, Hq] or [1]); q is then only read for its shape."""
    q = _c(q, np.float32)
    B, MTP, Hq, D = q.shape
    P, Hkv, PS, _ = k_cache.shape
    cdt = np.uint8 if quant else np.float32
    kc, vc = _c(k_cache, cdt), _c(v_cache, cdt)
    ks, vs = _c(k_scale, np.float32), _c(v_scale, np.float32)
    pt, cl = _c(page_table, np.int32), _c(ctx_lens, np.int32)
    prm = DecodeParams(B, MTP, Hq, Hkv, D, PS, pt.shape[1], P, window, tile, float(sm_scale),
                       int(quant), nthreads)
    keep = []
    _q8_fields(prm, q8, q8_scale, keep)
    out = np.empty((B, MTP, Hq, D), dtype=np.float32)
    rc = lib().orc_paged_decode(ctypes.byref(prm), _ptr(q), _ptr(kc), _ptr(vc), _ptr(ks),
                                _ptr(vs), _ptr(pt), _ptr(cl), _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_paged_decode failed ({rc})")
    return out


def paged_decode_mx(q, k_codes, k_e8, v_codes, v_e8, page_table, ctx_lens, *, window, sm_scale,
                    tile=256, nthreads=0, q8=None, q8_scale=None) -> np.ndarray:
    """MXFP4 KV cache, one E2M1 code per byte: k_codes [P, Hkv, page, D],
    k_e8 [P, Hkv, page, D/32]; V transposed: v_codes [P, Hkv, D, page],
    v_e8 [P, Hkv, D, page/32]; q [B, MTP, Hq, D] float32."""
    q = _c(q, np.float32)
    B, MTP, Hq, D = q.shape
    P, Hkv, PS, _ = k_codes.shape
    kc, ke, vc, ve = (_c(a, np.uint8) for a in (k_codes, k_e8, v_codes, v_e8))
    pt, cl = _c(page_table, np.int32), _c(ctx_lens, np.int32)
    prm = DecodeParams(B, MTP, Hq, Hkv, D, PS, pt.shape[1], P, window, tile, float(sm_scale), 1,
                       nthreads)
    keep = []
    _q8_fields(prm, q8, q8_scale, keep)
    out = np.empty((B, MTP, Hq, D), dtype=np.float32)
    rc = lib().orc_paged_decode_mx(ctypes.byref(prm), _ptr(q), _ptr(kc), _ptr(ke), _ptr(vc), _ptr(ve),
                                   _ptr(pt), _ptr(cl), _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_paged_decode_mx failed ({rc})")
    return out


# ---- whole prefill pipeline (oracle side) ----------------------------------
def prefill_int8_pipeline(q, k, v, *, causal, sm_scale, BN, q_block=128, k_block=64,
                          mu=None, rows=None, nthreads=0):
    """q/k/v canonical float32 [B,H,L,D].  Returns (out, intermediates).  `mu`
    overrides the K mean (the parity tests pass the HIP path's mean so that
    INT8 K codes are compared given the same mean)."""
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if mu is None:
        mu = k_mean(k)
    ks = smooth_k(k, mu)
    q8, qs = quant_int8(q, q_block)
    k8, kss = quant_int8(ks, k_block)
    v8, vs = quant_v_fp8(v)
    out = attn_emulated(B=B, H=H, Lq=Lq, Lk=Lk, D=D, causal=causal, sm_scale=sm_scale, BN=BN,
                        qk_mode=QK_INT8, q_block=q_block, k_block=k_block, quant_pv=True,
                        rows=rows, nthreads=nthreads, q8=q8, q_scale=qs, k8=k8, k_scale=kss,
                        v8=v8, v_scale=vs)
    return out, dict(mu=mu, q8=q8, q_scale=qs, k8=k8, k_scale=kss, v8=v8, v_scale=vs)


def prefill_mxfp4_pipeline(q, k, v, *, causal, sm_scale, BN, mu=None, rotate_qk=True,
                           rows=None, nthreads=0):
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if mu is None:
        mu = k_mean(k)
    ks = smooth_k(k, mu)
    qr = rotate(q) if rotate_qk else q
    kr = rotate(ks) if rotate_qk else ks
    q4, qe = quant_mxfp4(qr)
    k4, ke = quant_mxfp4(kr)
    v8, vs = quant_v_fp8(v)
    out = attn_emulated(B=B, H=H, Lq=Lq, Lk=Lk, D=D, causal=causal, sm_scale=sm_scale, BN=BN,
                        qk_mode=QK_MXFP4, quant_pv=True, rows=rows, nthreads=nthreads,
                        q4=q4, q_e8=qe, k4=k4, k_e8=ke, v8=v8, v_scale=vs)
    return out, dict(mu=mu, q4=q4, q_e8=qe, k4=k4, k_e8=ke, v8=v8, v_scale=vs,
                     q_rot=qr, k_rot=kr)

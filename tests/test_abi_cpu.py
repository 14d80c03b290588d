"""The C ABI without a GPU: the library loads, exports every function that
include/sage.h declares, and refuses bad arguments before any HIP call (every
case here fails validation, so no device is touched)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def S():
    from quantized_attention_block_amd import sage
    if not os.path.exists(sage.LIB_PATH):
        from quantized_attention_block_amd import build
        build.build()
    sage.lib()
    return sage


def _declared():
    with open(os.path.join(ROOT, "include", "sage.h")) as f:
        txt = f.read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(S):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(S.lib(), n), n
    assert S.lib().sage_version() == 4   # 0.4: adds the conversion test hooks


def test_quant_wait_bound_is_checked(S):
    with pytest.raises(S.SageError):
        S.sage_set_quant_wait_us(-1)
    with pytest.raises(S.SageError):
        S.sage_set_quant_wait_us(1000001)
    S.sage_set_quant_wait_us(2000)   # the default; host-only, no device touched


def test_attn_kv_tile_is_the_one_parity_tests_emulate(S):
    # the oracle's online-softmax block in the attention parity tests, smoke and
    # the CPU baseline is the fixed constant 64; the library must use the same
    assert S.sage_attn_kv_tile() == 64


def test_decode_split_plan_matches_page_and_oracle(S, orc):
    import json
    with open(os.path.join(ROOT, "tests", "golden", "aiter7388_window_tiles.json")) as f:
        g = json.load(f)
    for window, tiles in g["cases"]:
        assert S.sage_decode_num_splits(window, g["mtp"], 32768) == tiles
        assert orc.decode_num_splits(window, g["mtp"], 256) == tiles
    assert S.sage_decode_num_splits(0, 4, 8192) == 32
    assert S.sage_decode_num_splits(4096, 4, 1000) == 4      # capped by the context


FAKE = 1 << 20   # an aligned address that is never dereferenced


def T(dtype, shape, stride=None, data=FAKE):
    d = S_mod().SageTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def S_mod():
    from quantized_attention_block_amd import sage
    return sage


def _qk_call(S, q, k, prm, outs, ws_bytes=1 << 30, hadamard=None):
    r = ctypes.byref
    return S.lib().sage_quantize_qk(r(q), r(k), r(prm), r(outs[0]), r(outs[1]), r(outs[2]),
                                    r(outs[3]), None, hadamard, ctypes.c_void_p(FAKE), ws_bytes, None)


def _int8_outs(S, B, H, Lq, Lk, D, kb=64):
    p = lambda L: (L + 127) // 128 * 128
    return (T(S.I8, (B, H, p(Lq), D)), T(S.F32, (B, H, p(Lq) // 128)),
            T(S.I8, (B, H, p(Lk), D)), T(S.F32, (B, H, p(Lk) // kb)))


def test_quantize_qk_refusals(S):
    B, L, H, D = 1, 256, 2, 128
    q = T(S.BF16, (B, L, H, D))
    k = T(S.BF16, (B, L, H, D))
    prm = S.QkParams(S.QK_INT8, 128, 64, 1)
    outs = _int8_outs(S, B, H, L, L, D)
    # head-dim stride must be 1
    bad = T(S.BF16, (B, L, H, D), stride=(L * H * D * 2, H * D * 2, D * 2, 2))
    assert _qk_call(S, bad, k, prm, outs) == S.ERR_LAYOUT
    # row strides must be multiples of 16 bytes
    bad = T(S.BF16, (B, L, H, D), stride=(L * H * 132, H * 132, 132, 1))
    assert _qk_call(S, bad, k, prm, outs) == S.ERR_ALIGNMENT
    # misaligned base pointer
    assert _qk_call(S, T(S.BF16, (B, L, H, D), data=FAKE + 2), k, prm, outs) == S.ERR_ALIGNMENT
    # unsupported dtype / head dim / block sizes
    assert _qk_call(S, T(S.F32, (B, L, H, D)), k, prm, outs) == S.ERR_DTYPE
    assert _qk_call(S, T(S.BF16, (B, L, H, 96)), T(S.BF16, (B, L, H, 96)), prm, outs) == S.ERR_SHAPE
    assert _qk_call(S, q, k, S.QkParams(S.QK_INT8, 64, 64, 1), outs) == S.ERR_UNSUPPORTED
    assert _qk_call(S, q, k, S.QkParams(7, 128, 64, 1), outs) == S.ERR_INVALID_ARG
    # wrong output shape / dtype / layout
    o = list(outs)
    o[0] = T(S.I8, (B, H, 200, D))
    assert _qk_call(S, q, k, prm, o) == S.ERR_SHAPE
    o = list(outs)
    o[1] = T(S.F16, (B, H, 2))
    assert _qk_call(S, q, k, prm, o) == S.ERR_DTYPE
    o = list(outs)
    o[2] = T(S.I8, (B, H, 256, D), stride=(H * 256 * D, D, H * D, 1))
    assert _qk_call(S, q, k, prm, o) == S.ERR_LAYOUT
    # workspace too small
    assert _qk_call(S, q, k, prm, outs, ws_bytes=16) == S.ERR_WORKSPACE
    msg = S.lib().sage_last_error().decode()
    assert "workspace" in msg
    # MXFP4 needs D = 128 (BLOCK_R = 128)
    q64, k64 = T(S.BF16, (B, L, H, 64)), T(S.BF16, (B, L, H, 64))
    assert _qk_call(S, q64, k64, S.QkParams(S.QK_MXFP4, 128, 64, 1), outs) == S.ERR_SHAPE


def test_hadamard_order_refused(S):
    h = ctypes.c_void_p()
    assert S.lib().sage_hadamard_create(64, 0, None, ctypes.byref(h)) == S.ERR_SHAPE
    assert S.lib().sage_hadamard_create(256, 0, None, ctypes.byref(h)) == S.ERR_SHAPE
    assert not h.value


def test_attn_fwd_refusals(S):
    B, L, H, D = 1, 256, 2, 128
    r = ctypes.byref
    qq, qs, kq, ks = _int8_outs(S, B, H, L, L, D)
    vq = T(S.FP8_E4M3FN, (B, H, D, 256))
    vs = T(S.F32, (B, H, D))
    out = T(S.BF16, (B, L, H, D))

    def call(prm, vq_=vq, out_=out):
        return S.lib().sage_attn_fwd(r(qq), r(qs), r(kq), r(ks), r(vq_), r(vs), r(prm), r(out_),
                                     None, 0, None)

    good = dict(sm_scale=0.0, causal=0, qk_mode=S.QK_INT8, batch=B, heads=H, seqlen_q=L,
                seqlen_k=L, head_dim=D, num_kv_heads=0, q_block=128, k_block=64)
    P = lambda **kw: S.AttnParams(**{**good, **kw})
    assert call(P(), vq_=T(S.FP8_E4M3FNUZ, (B, H, D, 256))) == S.ERR_DTYPE
    assert "fnuz" in S.lib().sage_last_error().decode()
    assert call(P(causal=1, seqlen_k=200)) == S.ERR_UNSUPPORTED
    assert call(P(num_kv_heads=3)) == S.ERR_SHAPE
    assert call(P(head_dim=96)) == S.ERR_SHAPE
    assert call(P(), out_=T(S.BF16, (B, L, H, D), stride=(L * H * D, H * D, D, 2))) == S.ERR_LAYOUT
    assert call(P(), out_=T(S.I32, (B, L, H, D))) == S.ERR_DTYPE
    assert call(P(), out_=T(S.F32, (B, L, H, D), stride=(L * H * D, H * D, 2 * D + 2, 1))) == S.ERR_ALIGNMENT
    assert call(P(seqlen_q=300)) == S.ERR_SHAPE          # q_q padded length no longer matches
    assert call(P(sm_scale=float("nan"))) == S.ERR_INVALID_ARG
    # the ping-pong schedule: INT8 QK, head dim 128 only; unknown schedules refused
    assert call(P(schedule=2)) == S.ERR_INVALID_ARG
    assert call(P(schedule=S.SCHED_PINGPONG, head_dim=64)) == S.ERR_UNSUPPORTED
    assert call(P(schedule=S.SCHED_PINGPONG, qk_mode=S.QK_MXFP4)) == S.ERR_UNSUPPORTED
    assert "ping-pong" in S.lib().sage_last_error().decode()


def test_paged_decode_refusals(S):
    B, MTP, Hq, D, P_, Hkv, page = 2, 4, 16, 128, 8, 1, 128
    r = ctypes.byref
    q = T(S.BF16, (B, MTP, Hq, D))
    kc = T(S.FP8_E4M3FN, (P_, Hkv, page, D))
    vc = T(S.FP8_E4M3FN, (P_, Hkv, D, page))
    ksc = T(S.F32, (P_, Hkv, page))
    vsc = T(S.F32, (P_, Hkv, page))
    pt = T(S.I32, (B, 4))
    cl = T(S.I32, (B,))
    out = T(S.BF16, (B, MTP, Hq, D))

    def call(prm, kc_=kc, vc_=vc, q_=q, ws=1 << 30, pt_=pt):
        return S.lib().sage_paged_decode(r(q_), r(kc_), r(vc_), r(ksc), r(vsc), r(pt_), r(cl),
                                         r(prm), r(out), ctypes.c_void_p(FAKE), ws, None)

    prm = S.DecodeParams(0.0, 256, 1, 512)
    # an FNUZ cache is not gfx950's MFMA format
    assert call(prm, kc_=T(S.FP8_E4M3FNUZ, (P_, Hkv, page, D))) == S.ERR_DTYPE
    assert call(prm, vc_=T(S.FP8_E4M3FNUZ, (P_, Hkv, D, page))) == S.ERR_DTYPE
    assert call(prm, kc_=T(S.BF16, (P_, Hkv, page, D))) == S.ERR_DTYPE
    assert call(prm, q_=T(S.I32, (B, MTP, Hq, D))) == S.ERR_DTYPE
    assert call(prm, q_=T(S.FP8_E4M3FNUZ, (B, MTP, Hq, D))) == S.ERR_DTYPE   # not gfx950's FP8
    # an e4m3 q needs its scales ([1] or [B, MTP, Hq]); a bf16 q takes none
    q8 = T(S.FP8_E4M3FN, (B, MTP, Hq, D))
    assert call(prm, q_=q8) == S.ERR_INVALID_ARG
    qs_bad = T(S.F32, (B, MTP))
    assert call(S.DecodeParams(0.0, 256, 1, 512, ctypes.pointer(qs_bad)), q_=q8) == S.ERR_SHAPE
    qs_i32 = T(S.I32, (1,))
    assert call(S.DecodeParams(0.0, 256, 1, 512, ctypes.pointer(qs_i32)), q_=q8) == S.ERR_DTYPE
    qs_one = T(S.F32, (1,))
    assert call(S.DecodeParams(0.0, 256, 1, 512, ctypes.pointer(qs_one))) == S.ERR_INVALID_ARG
    # e4m3 q rows must start 16-byte aligned: a token stride of 8 bytes is refused
    assert call(S.DecodeParams(0.0, 256, 1, 512, ctypes.pointer(qs_one)),
                q_=T(S.FP8_E4M3FN, (B, MTP, Hq, D), stride=(MTP * Hq * D, 8, D, 1))) == S.ERR_ALIGNMENT
    assert call(prm, ws=64) == S.ERR_WORKSPACE
    assert call(S.DecodeParams(0.0, 256, 1, 4096)) == S.ERR_SHAPE       # table too short
    assert call(S.DecodeParams(0.0, 256, 2, 512)) == S.ERR_INVALID_ARG  # layout flag is 0 or 1
    assert call(S.DecodeParams(0.0, -1, 1, 512)) == S.ERR_INVALID_ARG
    # num_splits: 0 or the plan's count (window 256, MTP 4 within 512 keys: 2); others are not built
    plan = S.lib().sage_decode_num_splits(256, MTP, 512)
    assert plan == 2
    assert call(S.DecodeParams(0.0, 256, 1, 512, None, plan)) == S.ERR_HIP   # valid: reaches the device check
    assert call(S.DecodeParams(0.0, 256, 1, 512, None, plan + 1)) == S.ERR_UNSUPPORTED
    assert call(S.DecodeParams(0.0, 256, 1, 512, None, -1)) == S.ERR_INVALID_ARG
    # plain V [P, Hkv, page, D]: a transposed-shaped cache is refused (page 64 != D)
    kc64, vt64 = T(S.FP8_E4M3FN, (P_, Hkv, 64, D)), T(S.FP8_E4M3FN, (P_, Hkv, D, 64))
    sc64 = T(S.F32, (P_, Hkv, 64))
    plain = S.DecodeParams(0.0, 256, 0, 512)
    st = S.lib().sage_paged_decode(r(q), r(kc64), r(vt64), r(sc64), r(sc64), r(T(S.I32, (B, 8))), r(cl),
                                   r(plain), r(out), ctypes.c_void_p(FAKE), 1 << 30, None)
    assert st == S.ERR_SHAPE
    # fp32 output is refused (bf16 or f16)
    o32 = T(S.F32, (B, MTP, Hq, D))
    assert S.lib().sage_paged_decode(r(q), r(kc), r(vc), r(ksc), r(vsc), r(pt), r(cl), r(prm), r(o32),
                                     ctypes.c_void_p(FAKE), 1 << 30, None) == S.ERR_DTYPE
    # head dims other than 64, 128 and 256
    q96, o96 = T(S.BF16, (B, MTP, Hq, 96)), T(S.BF16, (B, MTP, Hq, 96))
    assert S.lib().sage_paged_decode(r(q96), r(T(S.FP8_E4M3FN, (P_, Hkv, page, 96))),
                                     r(T(S.FP8_E4M3FN, (P_, Hkv, 96, page))), r(ksc), r(vsc), r(pt), r(cl),
                                     r(prm), r(o96), ctypes.c_void_p(FAKE), 1 << 30, None) == S.ERR_UNSUPPORTED
    # pages of 8 or 48 keys: not a multiple of 16 dividing 256
    for pg in (8, 48):
        assert call(prm, kc_=T(S.FP8_E4M3FN, (P_, Hkv, pg, D)), vc_=T(S.FP8_E4M3FN, (P_, Hkv, D, pg)),
                    pt_=T(S.I32, (B, 64))) == S.ERR_UNSUPPORTED
    assert call(prm, kc_=T(S.FP8_E4M3FN, (P_, 3, page, D)), vc_=T(S.FP8_E4M3FN, (P_, 3, D, page))) == S.ERR_SHAPE
    # one scale per tensor is F32 [1] for both K and V
    bad = S.lib().sage_paged_decode(r(q), r(kc), r(vc), r(T(S.F32, (2,))), r(T(S.F32, (1,))), r(pt), r(cl),
                                    r(prm), r(out), ctypes.c_void_p(FAKE), 1 << 30, None)
    assert bad == S.ERR_SHAPE
    mixed = S.lib().sage_paged_decode(r(q), r(kc), r(vc), r(T(S.F32, (1,))), r(vsc), r(pt), r(cl),
                                      r(prm), r(out), ctypes.c_void_p(FAKE), 1 << 30, None)
    assert mixed == S.ERR_SHAPE


def test_paged_decode_mx_refusals(S):
    """The MXFP4 cache (chosen by k_cache's FP4X2 dtype) is validated field by
    field before any HIP call."""
    B, MTP, Hq, D, P_, Hkv, page = 2, 4, 16, 128, 8, 1, 128
    r = ctypes.byref
    q = T(S.BF16, (B, MTP, Hq, D))
    kc = T(S.FP4X2_E2M1, (P_, Hkv, page, D // 2))
    vc = T(S.FP4X2_E2M1, (P_, Hkv, D, page // 2))
    ke = T(S.E8M0, (P_, Hkv, page, D // 32))
    ve = T(S.E8M0, (P_, Hkv, D, page // 32))
    pt = T(S.I32, (B, 4))
    cl = T(S.I32, (B,))
    out = T(S.BF16, (B, MTP, Hq, D))
    prm = S.DecodeParams(0.0, 256, 1, 512)

    def call(kc_=kc, vc_=vc, ke_=ke, ve_=ve, prm_=prm):
        return S.lib().sage_paged_decode(r(q), r(kc_), r(vc_), r(ke_), r(ve_), r(pt), r(cl), r(prm_),
                                         r(out), ctypes.c_void_p(FAKE), 1 << 30, None)

    assert call(kc_=T(S.FP4X2_E2M1, (P_, Hkv, page, D))) == S.ERR_SHAPE          # D / 2 bytes per row
    assert call(vc_=T(S.FP4X2_E2M1, (P_, Hkv, D, page))) == S.ERR_SHAPE          # page / 2 bytes per row
    assert call(vc_=T(S.FP8_E4M3FN, (P_, Hkv, D, page))) == S.ERR_DTYPE          # mixed cache formats
    assert call(ke_=T(S.F32, (P_, Hkv, page, D // 32))) == S.ERR_DTYPE            # E8M0 bytes, not fp32
    assert call(ve_=T(S.E8M0, (P_, Hkv, D, page // 16))) == S.ERR_SHAPE          # one per 32 keys
    assert call(prm_=S.DecodeParams(0.0, 256, 0, 512)) == S.ERR_UNSUPPORTED
    p32 = 32
    assert call(kc_=T(S.FP4X2_E2M1, (P_, Hkv, p32, D // 2)), vc_=T(S.FP4X2_E2M1, (P_, Hkv, D, p32 // 2)),
                ke_=T(S.E8M0, (P_, Hkv, p32, D // 32)), ve_=T(S.E8M0, (P_, Hkv, D, 1)),
                prm_=S.DecodeParams(0.0, 64, 1, 128)) == S.ERR_UNSUPPORTED    # pages of 32 keys
    assert "multiple of 64" in S.lib().sage_last_error().decode()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from quantized_attention_block_amd import sage
    monkeypatch.setattr(sage, "_lib", None)
    monkeypatch.setattr(sage, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sage.lib()


def test_fused_q_refusals(S):
    """K-only quantization (q NULL) and Q quantized inside sage_attn_fwd
    (q_scale NULL): argument checks, no device work."""
    B, L, H, D = 1, 256, 2, 128
    r = ctypes.byref
    k = T(S.BF16, (B, L, H, D))
    _, _, kq, ks = _int8_outs(S, B, H, L, L, D)
    lib = S.lib()

    def qk(prm, q_out=None, q_scale=None):
        return lib.sage_quantize_qk(None, r(k), r(prm), q_out and r(q_out), q_scale and r(q_scale), r(kq), r(ks),
                                    None, None, ctypes.c_void_p(FAKE), 1 << 30, None)

    # MXFP4 K-only takes FP4X2 / E8M0 outputs (INT8 ones are refused)
    assert qk(S.QkParams(S.QK_MXFP4, 128, 64, 1)) == S.ERR_DTYPE
    assert qk(S.QkParams(S.QK_INT8, 128, 64, 1), q_out=T(S.I8, (B, H, L, D))) == S.ERR_INVALID_ARG
    nbytes = ctypes.c_size_t()
    assert lib.sage_quantize_qk_workspace_size(None, r(k), r(S.QkParams(S.QK_INT8, 128, 64, 1)),
                                               r(nbytes)) == S.OK
    vq, vs = T(S.FP8_E4M3FN, (B, H, D, 256)), T(S.F32, (B, H, D))
    out = T(S.BF16, (B, L, H, D))
    good = dict(sm_scale=0.0, causal=1, qk_mode=S.QK_INT8, batch=B, heads=H, seqlen_q=L,
                seqlen_k=L, head_dim=D, num_kv_heads=0, q_block=128, k_block=64)

    def attn(q, **kw):
        return lib.sage_attn_fwd(r(q), None, r(kq), r(ks), r(vq), r(vs), r(S.AttnParams(**{**good, **kw})),
                                 r(out), None, 0, None)

    assert attn(T(S.I8, (B, H, L, D))) == S.ERR_DTYPE                      # needs the fp16/bf16 Q
    assert attn(T(S.BF16, (B, L + 1, H, D))) == S.ERR_SHAPE
    assert attn(T(S.BF16, (B, L, H, D), stride=(L * H * D, 64, D, 1))) == S.ERR_LAYOUT   # rows overlap
    # MXFP4 fused: K codes must be FP4X2 / E8M0 (INT8 ones are refused); a
    # Hadamard only goes with an MXFP4 Q quantized in the kernel
    assert attn(T(S.BF16, (B, L, H, D)), qk_mode=S.QK_MXFP4) == S.ERR_DTYPE
    assert attn(T(S.BF16, (B, L, H, D)), hadamard=FAKE) == S.ERR_INVALID_ARG


def test_paged_decode_noalloc_refuses_above_its_scratch(S):
    """The no-allocation decode refuses, before any HIP call, a decode whose
    split partials need more than the fixed scratch (4096 sequences x 18
    splits x 64 rows x 272 bytes > 32 MiB); a fitting one passes validation
    up to the device check only on a GPU, so it is not called here."""
    r = ctypes.byref
    B, page = 4096, 128
    q = T(S.BF16, (B, 4, 16, 128))
    kc, vc = T(S.FP8_E4M3FN, (8, 1, page, 128)), T(S.FP8_E4M3FN, (8, 1, 128, page))
    ksc, vsc = T(S.F32, (8, 1, page)), T(S.F32, (8, 1, page))
    pt, cl = T(S.I32, (B, 64)), T(S.I32, (B,))
    prm = S.DecodeParams(0.0, 4096, 1, 8192)
    st = S.lib().sage_paged_decode_noalloc(r(q), r(kc), r(vc), r(ksc), r(vsc), r(pt), r(cl), r(prm),
                                           r(T(S.BF16, (B, 4, 16, 128))), None)
    assert st == S.ERR_WORKSPACE
    assert b"scratch" in S.lib().sage_last_error()
    assert S.DECODE_SCRATCH_BYTES == 32 << 20


def test_conversion_hooks_refusals(S):
    """The e4m3 / E2M1 conversion hooks check their descriptors and the
    exponent before any HIP call (CPU tensors: a call that got past
    validation would need a device)."""
    L = S.lib()
    x = torch.zeros(64, dtype=torch.float32)
    c = torch.zeros(64, dtype=torch.uint8)
    d = lambda t, dt=None: ctypes.byref(S.desc(t, dt))
    assert L.sage_debug_cvt_e4m3(d(x.to(torch.float16)), d(c), None) == S.ERR_DTYPE
    assert L.sage_debug_cvt_e4m3(d(x), d(c.to(torch.int32)), None) == S.ERR_DTYPE
    assert L.sage_debug_cvt_e4m3(d(x), d(c[:32]), None) == S.ERR_SHAPE
    assert L.sage_debug_cvt_e4m3(d(x.view(8, 8)), d(c), None) == S.ERR_SHAPE
    assert L.sage_debug_cvt_e4m3(d(torch.zeros(128)[::2]), d(c), None) == S.ERR_LAYOUT
    assert L.sage_debug_cvt_e4m3(None, d(c), None) == S.ERR_INVALID_ARG
    assert L.sage_debug_cvt_e2m1(d(x), 128, d(c), None) == S.ERR_INVALID_ARG
    assert L.sage_debug_cvt_e2m1(d(x), -128, d(c), None) == S.ERR_INVALID_ARG
    assert L.sage_debug_cvt_e2m1(d(x), 0, d(c[:8]), None) == S.ERR_SHAPE
    assert L.sage_debug_cvt_e2m1(d(x.to(torch.float64)), 0, d(c), None) == S.ERR_DTYPE


def test_negative_strides_and_oversized_slices_refused(S):
    """A negative stride would address memory before a view's base, and a
    (b, h) slice of an fp16/bf16 view longer than 2^31 bytes is beyond the
    kernels' 32-bit buffer offsets: both are refused before any HIP call
    (descriptors only; their memory is never touched)."""
    L = S.lib()
    prm = S.QkParams(mode=S.QK_INT8, q_block=128, k_block=64, smooth_k=1)
    nbytes = ctypes.c_size_t()
    k = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    d = S.desc(k)
    assert L.sage_quantize_qk_workspace_size(None, ctypes.byref(d), ctypes.byref(prm),
                                             ctypes.byref(nbytes)) == S.OK
    d.stride[1] = -d.stride[1]
    assert L.sage_quantize_qk_workspace_size(None, ctypes.byref(d), ctypes.byref(prm),
                                             ctypes.byref(nbytes)) == S.ERR_LAYOUT
    # the stacked video-DiT layout (token stride 3 H D = 15360): 69906 tokens
    # fit in one slice's 2^31 bytes, 69907 do not
    for Lk, want in ((69906, S.OK), (69907, S.ERR_UNSUPPORTED)):
        d = S.desc(k)
        d.shape[1] = Lk
        d.shape[2] = 40
        d.stride[0], d.stride[1], d.stride[2] = Lk * 15360, 15360, 128
        assert L.sage_quantize_qk_workspace_size(None, ctypes.byref(d), ctypes.byref(prm),
                                                 ctypes.byref(nbytes)) == want, Lk
        assert L.sage_quantize_v_workspace_size(ctypes.byref(d), ctypes.byref(nbytes)) == want, Lk

"""Paged decode over an MXFP4 KV cache on the GPU: against the oracle's
MXFP4 decode (cosine >= 0.999, max-abs <= 1e-2 beyond the bf16 output's half
ulp), against exact attention on the dequantized cache (cosine >= 0.99),
and against base-2 attention in closed form on exactly representable
inputs."""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from quantized_attention_block_amd import workloads as wl
from tests._util import base2_decode, cosine, require_gpu, say

pytestmark = pytest.mark.gpu

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
E2M1 = np.concatenate([_E2M1, -_E2M1])     # code -> value (sign in bit 3)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _dequant(inp):
    """Float caches of an MXFP4 input: K [P, Hkv, page, D], V [P, Hkv, page, D]."""
    kc, ke = inp.k_codes.numpy(), inp.k_e8.numpy().astype(np.float64)
    vc, ve = inp.v_codes.numpy(), inp.v_e8.numpy().astype(np.float64)
    kf = E2M1[kc] * np.repeat(2.0 ** (ke - 127), 32, axis=-1)
    vf = (E2M1[vc] * np.repeat(2.0 ** (ve - 127), 32, axis=-1)).transpose(0, 1, 3, 2)
    return kf.astype(np.float32), np.ascontiguousarray(vf).astype(np.float32)


def _run(inp, dev, window, max_ctx, sm_scale):
    k4, v4 = inp.packed()
    out = sage.sage_paged_decode(inp.q.to(dev), k4.to(dev).view(torch.float4_e2m1fn_x2),
                                 v4.to(dev).view(torch.float4_e2m1fn_x2),
                                 inp.k_e8.to(dev).view(torch.float8_e8m0fnu),
                                 inp.v_e8.to(dev).view(torch.float8_e8m0fnu),
                                 inp.page_table.to(dev), inp.ctx_lens.to(dev), max_ctx=max_ctx,
                                 window=window, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(orc, inp, window, sm_scale):
    return orc.paged_decode_mx(inp.q.float().numpy(), inp.k_codes.numpy(), inp.k_e8.numpy(),
                               inp.v_codes.numpy(), inp.v_e8.numpy(), inp.page_table.numpy(),
                               inp.ctx_lens.numpy(), window=window, sm_scale=sm_scale)


def _exact(orc, inp, window, sm_scale):
    kf, vf = _dequant(inp)
    ones = np.ones(kf.shape[:3], np.float32)
    return orc.paged_decode(inp.q.float().numpy(), kf, vf, ones, ones, inp.page_table.numpy(),
                            inp.ctx_lens.numpy(), window=window, sm_scale=sm_scale, quant=False)


def _half_ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 8)


def _check(g, o, e):
    assert cosine(g, o) >= 0.999
    assert np.max(np.maximum(np.abs(g - o) - _half_ulp_bf16(o), 0.0)) <= 1e-2
    assert cosine(g, e) >= 0.99


def test_mx_decode_full_workload(dev, orc):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode_mx(w)
    say("MXFP4 paged decode", "batch 16 MTP4 GQA16 page 128 ctx 8192 window 4096")
    g = _run(inp, dev, w.window, w.ctx, w.sm_scale)
    _check(g, _oracle(orc, inp, w.window, w.sm_scale), _exact(orc, inp, w.window, w.sm_scale))


@pytest.mark.parametrize("window,ctx", [(0, 1000), (300, 777), (0, 64), (700, 2049)])
def test_mx_decode_windows_and_contexts(dev, orc, window, ctx):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode_mx(w, batch=3, ctx=ctx)
    say("MXFP4 paged decode", f"window {window} ctx {ctx}")
    g = _run(inp, dev, window, ctx, w.sm_scale)
    _check(g, _oracle(orc, inp, window, w.sm_scale), _exact(orc, inp, window, w.sm_scale))


def test_mx_decode_degenerate_contexts(dev, orc):
    """Contexts 0, 1, 3 (query tokens at negative positions), 4, 5 and 814
    with window 300 (a first split that only query token 0 sees): empty rows
    are 0, the rest match the oracle."""
    w = wl.WORKLOADS["paged_decode"]
    ctxs = [0, 1, 3, 4, 5, 814]
    inp = wl.make_decode_mx(w, batch=len(ctxs), ctx=814)
    inp.ctx_lens[:] = torch.tensor(ctxs, dtype=torch.int32)
    say("MXFP4 paged decode, degenerate contexts", ctxs)
    g = _run(inp, dev, 300, 814, w.sm_scale)
    o = _oracle(orc, inp, 300, w.sm_scale)
    assert np.isfinite(g).all()
    assert not g[0].any() and not g[1, :3].any() and not g[2, :1].any()
    assert not g[(o == 0).all(axis=-1)].any()                             # every empty row
    _check(g, o, _exact(orc, inp, 300, w.sm_scale))


@pytest.mark.parametrize("mtp,hq,hkv,page", [(1, 8, 1, 64), (2, 16, 2, 256), (4, 16, 1, 512)])
def test_mx_decode_shapes(dev, orc, mtp, hq, hkv, page):
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("mx_shape", 40 + page, 2, mtp, hq, hkv, 128, page, 1500, 0)
    inp = wl.make_decode_mx(w)
    say("MXFP4 paged decode", f"mtp {mtp} hq {hq} hkv {hkv} page {page}")
    g = _run(inp, dev, 0, w.ctx, base.sm_scale)
    _check(g, _oracle(orc, inp, 0, base.sm_scale), _exact(orc, inp, 0, base.sm_scale))


@pytest.mark.parametrize("window", [0, 20])
def test_mx_decode_equals_base2_attention(dev, window):
    """Exact inputs: K codes of {0, +-1, +-2} with exponent 127 and a zero
    channel where every Q row has a 448 (q_scale 1); Q in {0, +-2} on two
    channels, alpha = 0.5, so x = q.k / 2 is an integer in [-4, 4]; V codes
    times 2^(e - 127) for e in {126, 127, 128}."""
    rng = np.random.default_rng(95)
    B, MTP, Hq, Hkv, D, PS, max_pages = 2, 4, 4, 1, 128, 64, 2
    P = B * max_pages
    q = np.zeros((B, MTP, Hq, D), np.float32)
    q[..., :2] = rng.choice([0.0, 2.0, -2.0], (B, MTP, Hq, 2))
    q[..., 2] = 448.0
    kc = np.zeros((P, Hkv, PS, D), np.uint8)
    kc[..., :2] = rng.choice(np.array([0, 2, 4, 10, 12], np.uint8), (P, Hkv, PS, 2))   # 0, 1, 2, -1, -2
    kc[..., 3:] = rng.integers(0, 16, (P, Hkv, PS, D - 3))                              # q is 0 there
    ke = np.full((P, Hkv, PS, D // 32), 127, np.uint8)
    vc = rng.integers(0, 16, (P, Hkv, D, PS)).astype(np.uint8)
    ve = rng.integers(126, 129, (P, Hkv, D, PS // 32)).astype(np.uint8)
    table = rng.permutation(P).astype(np.int32).reshape(B, max_pages)
    ctx = np.array([100, 57], np.int32)
    t = torch.from_numpy
    inp = wl.DecodeInputsMX(t(q).to(torch.bfloat16), t(kc), t(ke), t(vc), t(ve), t(table), t(ctx))
    say("MXFP4 paged decode, exact inputs", f"window {window}")
    g = _run(inp, dev, window, max_pages * PS, float(np.log(2.0) / 2))
    kf, vf = _dequant(inp)
    ones = np.ones((P, Hkv, PS), np.float32)
    ref = base2_decode(q, kf, vf, ones, ones, table, ctx, window, Hkv)
    fp16_rows = 2.0 ** -12 * np.abs(vf).max()
    assert np.all(np.abs(g - ref) <= _half_ulp_bf16(ref) + fp16_rows + 1e-4 * np.abs(ref).max())


@pytest.mark.parametrize("window,ctx", [(0, 12000), (8192, 12000)])
def test_mx_decode_more_than_32_splits(dev, orc, window, ctx):
    """47 and 34 splits per sequence: more than one merge batch of 32."""
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("mx_long", 77, 2, 4, 16, 1, 128, 128, ctx, window)
    inp = wl.make_decode_mx(w)
    inp.ctx_lens[1] = ctx - 1000
    assert sage.sage_decode_num_splits(window, 4, ctx) > 32
    say("MXFP4 paged decode > 32 splits", f"window {window} ctx {ctx}")
    g = _run(inp, dev, window, ctx, base.sm_scale)
    _check(g, _oracle(orc, inp, window, base.sm_scale), _exact(orc, inp, window, base.sm_scale))

"""Paged decode over the rest of the aiter page's shape matrix: fp16 and e4m3
queries (e4m3 with one scale per tensor or per (token, head) row, on the FP8
and the MXFP4 cache), the plain V cache layout [P, Hkv, page, D], head dim
256 and fp16 output.  Each is checked against the oracle (cosine >= 0.999,
max-abs <= 1e-2 beyond the output's half ulp) and exact attention (cosine >=
0.99); the plain V layout must also give the transposed layout's output bit
for bit (the same bytes reach the same MFMA operands)."""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from quantized_attention_block_amd import workloads as wl
from tests._util import cosine, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _half_ulp(x, bits):
    a = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - bits)


def _check(g, o, e, out_bits=8):
    assert cosine(g, o) >= 0.999, cosine(g, o)
    err = np.max(np.maximum(np.abs(g - o) - _half_ulp(o, out_bits), 0.0))
    assert err <= 1e-2, err
    assert cosine(g, e) >= 0.99, cosine(g, e)


def _cache(inp, dev, plain_v):
    kc = inp.k_cache.to(dev).view(torch.float8_e4m3fn)
    v = inp.v_cache if plain_v else inp.v_cache.transpose(2, 3).contiguous()
    return kc, v.to(dev).view(torch.float8_e4m3fn)


def _run(inp, dev, window, max_ctx, sm_scale, plain_v=False, q=None, q_scale=None, out=None):
    kc, vc = _cache(inp, dev, plain_v)
    o = sage.sage_paged_decode(inp.q.to(dev) if q is None else q.to(dev), kc, vc, inp.k_scale.to(dev),
                               inp.v_scale.to(dev), inp.page_table.to(dev), inp.ctx_lens.to(dev),
                               max_ctx=max_ctx, window=window, sm_scale=sm_scale, v_transposed=not plain_v,
                               q_scale=None if q_scale is None else q_scale.to(dev), out=out)
    torch.cuda.synchronize()
    return o


def _oracle(orc, inp, window, sm_scale, q=None, q8=None, q8_scale=None):
    qf = (inp.q if q is None else q).float().numpy()
    return orc.paged_decode(qf, inp.k_cache.numpy(), inp.v_cache.numpy(), inp.k_scale.numpy(),
                            inp.v_scale.numpy(), inp.page_table.numpy(), inp.ctx_lens.numpy(),
                            window=window, sm_scale=sm_scale, q8=q8, q8_scale=q8_scale)


def _exact(orc, inp, window, sm_scale, qf=None):
    kf = orc.e4m3_decode_array(inp.k_cache.numpy()) * inp.k_scale.numpy()[..., None]
    vf = orc.e4m3_decode_array(inp.v_cache.numpy()) * inp.v_scale.numpy()[..., None]
    ones = np.ones(inp.k_scale.shape, np.float32)
    q = inp.q.float().numpy() if qf is None else qf
    return orc.paged_decode(q, kf, vf, ones, ones, inp.page_table.numpy(), inp.ctx_lens.numpy(),
                            window=window, sm_scale=sm_scale, quant=False)


@pytest.mark.parametrize("D,page,window,ctx", [(128, 128, 4096, 8192), (128, 16, 300, 1537),
                                               (128, 64, 0, 1000), (64, 32, 700, 2049),
                                               (256, 128, 1000, 3000), (256, 16, 0, 900)])
def test_plain_v_equals_transposed_v(dev, orc, D, page, window, ctx):
    w = wl.DecodeWorkload("fmt", 21, 4, 4, 16, 1, D, page, ctx, window)
    inp = wl.make_decode(w)
    inp.ctx_lens[1] = ctx - 301
    inp.ctx_lens[2] = max(4, ctx // 3)
    say("plain V", f"D {D} page {page} window {window} ctx {ctx}")
    sm = float(D ** -0.5)
    a = _run(inp, dev, window, ctx, sm, plain_v=True)
    b = _run(inp, dev, window, ctx, sm, plain_v=False)
    assert torch.equal(a, b)
    _check(a.float().cpu().numpy(), _oracle(orc, inp, window, sm), _exact(orc, inp, window, sm))


@pytest.mark.parametrize("page,window,ctx,mtp,hq,hkv", [(128, 4096, 8192, 4, 16, 1), (64, 512, 2000, 2, 8, 2),
                                                       (16, 0, 700, 1, 16, 1), (256, 300, 1200, 4, 16, 2)])
def test_head_dim_256(dev, orc, page, window, ctx, mtp, hq, hkv):
    """D = 256 (e4m3 cache): two 128-channel planes per tile, QK summed over
    them, 256-channel partial rows and merge."""
    w = wl.DecodeWorkload("d256", 22, 3, mtp, hq, hkv, 256, page, ctx, window)
    inp = wl.make_decode(w)
    inp.ctx_lens[1] = ctx - 200
    say("D 256", f"page {page} window {window} ctx {ctx} mtp {mtp} hq {hq} hkv {hkv}")
    sm = float(256 ** -0.5)
    g = _run(inp, dev, window, ctx, sm).float().cpu().numpy()
    assert g.shape[-1] == 256
    _check(g, _oracle(orc, inp, window, sm), _exact(orc, inp, window, sm))


def test_fp16_queries_and_output(dev, orc):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=4, ctx=3000)
    q16 = inp.q.float().to(torch.float16)
    say("fp16 queries, fp16 and bf16 output")
    o16 = torch.empty(q16.shape, dtype=torch.float16, device=dev)
    g16 = _run(inp, dev, 1000, 3000, w.sm_scale, q=q16, out=o16).float().cpu().numpy()
    gbf = _run(inp, dev, 1000, 3000, w.sm_scale, q=q16,
               out=torch.empty(q16.shape, dtype=torch.bfloat16, device=dev)).float().cpu().numpy()
    o = _oracle(orc, inp, 1000, w.sm_scale, q=q16)
    e = _exact(orc, inp, 1000, w.sm_scale, qf=q16.float().numpy())
    _check(g16, o, e, out_bits=11)
    _check(gbf, o, e)
    # the two outputs are the same fp32 result rounded two ways
    assert np.abs(g16 - gbf).max() <= np.max(_half_ulp(o, 8)) + np.max(_half_ulp(o, 11))


@pytest.mark.parametrize("per_tensor,plain_v,D", [(False, False, 128), (True, False, 128), (False, True, 256)])
def test_e4m3_queries(dev, orc, per_tensor, plain_v, D):
    """Queries given in e4m3 with their scales: the oracle takes the same
    codes and scales; exact attention takes their values."""
    w = wl.DecodeWorkload("q8", 23, 4, 4, 16, 1, D, 128, 2500, 1024)
    inp = wl.make_decode(w)
    inp.ctx_lens[3] = 1111
    qf = inp.q.float()
    if per_tensor:
        s = (qf.abs().amax() / 448.0).reshape(1)
        codes = (qf / s).to(torch.float8_e4m3fn)
    else:
        s = qf.abs().amax(dim=-1) / 448.0
        codes = (qf / s[..., None]).to(torch.float8_e4m3fn)
    s = s.float().contiguous()
    say("e4m3 queries", f"per tensor {per_tensor} plain V {plain_v} D {D}")
    sm = float(D ** -0.5)
    g = _run(inp, dev, 1024, 2500, sm, plain_v=plain_v, q=codes, q_scale=s).float().cpu().numpy()
    q8 = codes.view(torch.uint8).numpy()
    o = _oracle(orc, inp, 1024, sm, q8=q8, q8_scale=s.numpy())
    qval = (codes.float() * (s if per_tensor else s[..., None])).numpy()
    _check(g, o, _exact(orc, inp, 1024, sm, qf=qval))


def test_e4m3_queries_mxfp4_cache(dev, orc):
    """pa_decode_mxfp4 with e4m3 queries (the aiter page's MXFP4 matrix has bf16
    and e4m3 queries)."""
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode_mx(w, batch=3, ctx=2000)
    k4, v4 = inp.packed()
    qf = inp.q.float()
    s = (qf.abs().amax(dim=-1) / 448.0).float().contiguous()
    codes = (qf / s[..., None]).to(torch.float8_e4m3fn)
    say("MXFP4 cache, e4m3 queries")
    out = sage.sage_paged_decode(codes.to(dev), k4.to(dev).view(torch.float4_e2m1fn_x2),
                                 v4.to(dev).view(torch.float4_e2m1fn_x2),
                                 inp.k_e8.to(dev).view(torch.float8_e8m0fnu),
                                 inp.v_e8.to(dev).view(torch.float8_e8m0fnu), inp.page_table.to(dev),
                                 inp.ctx_lens.to(dev), max_ctx=2000, window=700, sm_scale=w.sm_scale,
                                 q_scale=s.to(dev))
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    o = orc.paged_decode_mx(qf.numpy(), inp.k_codes.numpy(), inp.k_e8.numpy(), inp.v_codes.numpy(),
                            inp.v_e8.numpy(), inp.page_table.numpy(), inp.ctx_lens.numpy(), window=700,
                            sm_scale=w.sm_scale, q8=codes.view(torch.uint8).numpy(), q8_scale=s.numpy())
    assert cosine(g, o) >= 0.999
    assert np.max(np.maximum(np.abs(g - o) - _half_ulp(o, 8), 0.0)) <= 1e-2

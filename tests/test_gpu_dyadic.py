"""The GPU path against closed forms, independently of the oracle: on inputs
where every quantization step is exact (tests._util.dyadic_prefill and
dyadic_decode: integer scores in log2 units, power-of-two or unit scales,
codes equal to the values, a K mean of exactly 0), the INT8 and MXFP4 prefill
pipelines and the FP8 paged decode must reproduce base-2 attention on the
integer scores.  What separates them is only fp32 arithmetic: the row sums
and the PV accumulation over n keys, and the approximate hardware exp2 of
the (integer + log2 448) exponents, bounded together by
softmax_accumulation_bound(n) times the largest |v| (derived there), plus for
the decode the fp16 partial rows (2^-12 of the largest |v_scale V|) and the
bf16 output rounding.  A wrong mask, scale, fold or rescale moves some weight
by a power of two, far outside these bounds."""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from tests._util import (base2_attention, base2_decode, canon, dyadic_decode, dyadic_prefill, require_gpu, say,
                         softmax_accumulation_bound)

pytestmark = pytest.mark.gpu

SM_SCALE = float(np.log(2.0) / 2)   # alpha = fp32(sm_scale log2 e) = 0.5


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _logical(x, dev):
    """Canonical [B, H, L, D] float32 -> logical [B, L, H, D] bf16 (exact here)."""
    t = torch.from_numpy(x).permute(0, 2, 1, 3).contiguous().to(torch.bfloat16)
    assert np.array_equal(t.float().permute(0, 2, 1, 3).numpy(), x)
    return t.to(dev)


@pytest.mark.parametrize("D,causal", [(128, True), (128, False), (64, True)])
def test_int8_pipeline_equals_base2_attention(dev, D, causal):
    L = 200   # two Q blocks (128 + 72 rows), K blocks of 64 with an 8-row tail
    q, k, v = dyadic_prefill(81, L, D, [0.0, 2.0, -2.0, 4.0, -4.0], [0.0, 1.0, -1.0], 254.0, 127.0)
    say("dyadic INT8 prefill", f"D {D} causal {causal} L {L}")
    qk = sage.sage_quantize_qk(_logical(q, dev), _logical(k, dev))
    vq, vs = sage.sage_quantize_v(_logical(v, dev))
    out = sage.sage_attn_fwd(qk, vq, vs, causal=causal, sm_scale=SM_SCALE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(qk.k_mean == 0)
    assert torch.all(qk.q_scale == 2.0) and torch.all(qk.k_scale == 1.0)
    x = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) / 2
    ref = base2_attention(x, v, causal)
    g = canon(out)
    # the kernel sums each row over all L keys (V is exact: codes 112 v, scale 4 / 448)
    assert np.abs(g - ref).max() <= softmax_accumulation_bound(L) * np.abs(v).max()


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_pipeline_equals_base2_attention(dev, causal):
    L, D = 160, 128
    q, k, v = dyadic_prefill(82, L, D, [0.0, 2.0, -2.0], [0.0, 1.0, -1.0, 2.0, -2.0], 4.0, 4.0)
    say("dyadic MXFP4 prefill (no rotation)", f"causal {causal} L {L}")
    qk = sage.sage_quantize_qk(_logical(q, dev), _logical(k, dev), mode=sage.QK_MXFP4, hadamard=None)
    vq, vs = sage.sage_quantize_v(_logical(v, dev))
    out = sage.sage_attn_fwd(qk, vq, vs, causal=causal, sm_scale=SM_SCALE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    x = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) / 2
    ref = base2_attention(x, v, causal)
    g = canon(out)
    # the kernel sums each row over all L keys (V is exact: codes 112 v, scale 4 / 448)
    assert np.abs(g - ref).max() <= softmax_accumulation_bound(L) * np.abs(v).max()


@pytest.mark.parametrize("window,PS,D,plain_v,qkind", [
    (0, 32, 128, False, "bf16"), (20, 32, 128, False, "bf16"), (20, 16, 128, False, "bf16"),
    (20, 32, 64, False, "bf16"),
    (20, 32, 128, True, "bf16"), (0, 16, 64, True, "f16"),           # plain V
    (20, 32, 256, False, "bf16"), (20, 16, 256, True, "bf16"),       # D 256
    (20, 32, 128, False, "e4m3"), (0, 64, 256, True, "e4m3")])       # e4m3 queries
def test_paged_decode_equals_base2_attention(dev, window, PS, D, plain_v, qkind):
    B, MTP, Hq, Hkv = 2, 4, 4, 1
    max_pages = 128 // PS
    ctx = np.array([100, 57], np.int32)
    q, kf, vf, ks, vs, table = dyadic_decode(93, B=B, MTP=MTP, Hq=Hq, Hkv=Hkv, D=D, PS=PS,
                                             max_pages=max_pages)
    say("dyadic paged decode", f"window {window} ctx {ctx.tolist()} page {PS} D {D} plain V {plain_v} q {qkind}")
    to8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn)
    kc, vt = to8(kf), to8(vf if plain_v else vf.transpose(0, 1, 3, 2))
    assert np.array_equal(kc.float().numpy(), kf)
    qt = torch.from_numpy(q)
    # every query value (0, +-2, 448) is exact in each query format; e4m3
    # codes are the values themselves with one scale of 1
    qd = {"bf16": qt.to(torch.bfloat16), "f16": qt.to(torch.float16), "e4m3": qt.to(torch.float8_e4m3fn)}[qkind]
    assert np.array_equal(qd.float().numpy(), q)
    q_scale = torch.ones(1, device=dev) if qkind == "e4m3" else None
    out = sage.sage_paged_decode(qd.to(dev), kc.to(dev), vt.to(dev),
                                 torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev),
                                 torch.from_numpy(table).to(dev), torch.from_numpy(ctx).to(dev),
                                 max_ctx=max_pages * PS, window=window, sm_scale=SM_SCALE,
                                 v_transposed=not plain_v, q_scale=q_scale)
    torch.cuda.synchronize()
    ref = base2_decode(q, kf, vf, ks, vs, table, ctx, window, Hkv)
    g = out.float().cpu().numpy()
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 8)
    vmax = np.abs(vf * vs[..., None]).max()
    fp16_rows = 2.0 ** -12 * vmax
    # each split sums its 256-key tile in fp32; the merge weights are exact
    # powers of two (integer maxima)
    acc = softmax_accumulation_bound(256) * vmax
    assert np.all(np.abs(g - ref) <= half_ulp + fp16_rows + acc)

"""Quantizer parity on the GPU: INT8 Q/K codes and scales, the K mean, e4m3 V
codes and scales, and MXFP4 codes/E8M0 scales, bit-exact against the oracle
(INT8 K is compared given the GPU's mean, which must itself equal the
oracle's)."""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from quantized_attention_block_amd import workloads as wl
from tests._util import canon, require_gpu, say, u8

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict()),                                   # fp16, D=64, 2 Q / 4 K blocks
    ("llm_prefill", dict(Lq=520, Lk=520, B=1, H=3)),    # ragged tail, bf16, D=128
    ("video_dit", dict(Lq=1000, Lk=1000, H=3)),         # stacked strided views, outliers
]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("name,kw", CASES)
@pytest.mark.parametrize("k_block", [64, 128])
def test_int8_qk_bit_exact(dev, orc, name, kw, k_block):
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("int8 quantize", name, kw, k_block)
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_INT8, k_block=k_block)
    torch.cuda.synchronize()
    qc, kc = canon(inp.q), canon(inp.k)
    Lq, Lk = qc.shape[2], kc.shape[2]
    mu_o = orc.k_mean(kc)
    mu_g = qk.k_mean.cpu().numpy()
    assert np.array_equal(mu_g, mu_o)
    q8, qs = orc.quant_int8(qc, 128)
    k8, ks = orc.quant_int8(orc.smooth_k(kc, mu_g), k_block)
    gq, gk = qk.q.cpu().numpy(), qk.k.cpu().numpy()
    assert np.array_equal(gq[:, :, :Lq], q8) and not gq[:, :, Lq:].any()
    assert np.array_equal(gk[:, :, :Lk], k8) and not gk[:, :, Lk:].any()
    gqs, gks = qk.q_scale.cpu().numpy(), qk.k_scale.cpu().numpy()
    assert np.array_equal(gqs, qs)
    assert np.array_equal(gks[..., :ks.shape[-1]], ks) and not gks[..., ks.shape[-1]:].any()


@pytest.mark.parametrize("name,kw", CASES)
def test_v_fp8_bit_exact(dev, orc, name, kw):
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("v quantize", name, kw)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    torch.cuda.synchronize()
    vc = canon(inp.v)
    L = vc.shape[2]
    v8, vs = orc.quant_v_fp8(vc)
    g = u8(v_q).transpose(0, 1, 3, 2)          # [B,H,Lkp,D]
    assert np.array_equal(g[:, :, :L], v8) and not g[:, :, L:].any()
    assert np.array_equal(v_s.cpu().numpy(), vs)


# MXFP4 needs D = 128: the D-128 cases in their own precision, and the ragged
# LLM-prefill case cast to fp16 (the quantizer's fp16 instantiation)
MX_CASES = [(name, kw, None) for name, kw in CASES[1:]] + [("llm_prefill", CASES[1][1], torch.float16)]


def _mx_inputs(dev, name, kw, dtype):
    inp = wl.make_prefill(wl.WORKLOADS[name], device=dev, **kw)
    q, k = inp.q, inp.k
    if dtype is not None:
        q, k = q.to(dtype), k.to(dtype)
    return q, k


@pytest.mark.parametrize("name,kw,dtype", MX_CASES)
def test_mxfp4_without_rotation_bit_exact(dev, orc, name, kw, dtype):
    q, k = _mx_inputs(dev, name, kw, dtype)
    say("mxfp4 quantize (no rotation)", name, kw, q.dtype)
    qk = sage.sage_quantize_qk(q, k, mode=sage.QK_MXFP4)
    torch.cuda.synchronize()
    qc, kc = canon(q), canon(k)
    Lq, Lk = qc.shape[2], kc.shape[2]
    mu_g = qk.k_mean.cpu().numpy()
    assert np.array_equal(mu_g, orc.k_mean(kc))
    q4, qe = orc.quant_mxfp4(qc)
    k4, ke = orc.quant_mxfp4(orc.smooth_k(kc, mu_g))
    gq = orc.unpack_fp4(qk.q.cpu().numpy())
    gk = orc.unpack_fp4(qk.k.cpu().numpy())
    assert np.array_equal(gq[:, :, :Lq], q4) and not gq[:, :, Lq:].any()
    assert np.array_equal(gk[:, :, :Lk], k4) and not gk[:, :, Lk:].any()
    assert np.array_equal(qk.q_scale.cpu().numpy()[:, :, :Lq], qe)
    assert np.array_equal(qk.k_scale.cpu().numpy()[:, :, :Lk], ke)


@pytest.mark.parametrize("name,kw,dtype", MX_CASES)
def test_mxfp4_with_hadamard(dev, orc, name, kw, dtype):
    """The rotation sums 128 products in fp32 on MFMA, so a value that sits on
    an E2M1 rounding boundary can round the other way than the oracle's
    correctly rounded sum: codes agree except on such boundary cases, and the
    dequantized values agree to within one code step."""
    q, k = _mx_inputs(dev, name, kw, dtype)
    had = sage.Hadamard(0)
    say("mxfp4 quantize (hadamard)", name, kw, q.dtype)
    qk = sage.sage_quantize_qk(q, k, mode=sage.QK_MXFP4, hadamard=had)
    torch.cuda.synchronize()
    qc, kc = canon(q), canon(k)
    mu = qk.k_mean.cpu().numpy()
    vals = np.array([orc.e2m1_decode(c) for c in range(16)], np.float32)
    for x, codes, e8 in ((orc.rotate(qc), qk.q, qk.q_scale),
                         (orc.rotate(orc.smooth_k(kc, mu)), qk.k, qk.k_scale)):
        L = x.shape[2]
        o4, oe = orc.quant_mxfp4(x)
        g4 = orc.unpack_fp4(codes.cpu().numpy())[:, :, :L]
        ge = e8.cpu().numpy()[:, :, :L]
        assert (ge == oe).mean() > 0.999
        assert (g4 == o4).mean() > 0.995
        deq = lambda c, e: vals[c] * np.repeat(2.0 ** (e.astype(np.float32) - 127), 32, axis=-1)
        same_e = np.repeat(ge == oe, 32, axis=-1)
        step = np.repeat(2.0 ** (oe.astype(np.float32) - 127), 32, axis=-1) * 2.0
        diff = np.abs(deq(g4, ge) - deq(o4, oe))
        assert (diff[same_e] <= step[same_e] + 1e-30).all()


def _same_qk(a, b):
    for f in ("q", "q_scale", "k", "k_scale", "k_mean"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_single_read_sync_words(dev):
    """The single-read quantizers meet per head through flags in the
    workspace that carry per-call epoch tokens: results must not depend on
    what the workspace held before -- random bytes, the previous call of the
    same shape, or a call of another shape in between."""
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=520, Lk=520, B=1, H=3)
    other = wl.make_prefill(w, device=dev, Lq=1500, Lk=1500, B=1, H=2)
    say("quantizer sync words", "llm_prefill 520 x 3 heads, 1500 x 2 heads between")
    ref_qk = sage.sage_quantize_qk(inp.q, inp.k)
    ref_v = sage.sage_quantize_v(inp.v)
    nq = max(sage.sage_quantize_qk_workspace_size(inp.q, inp.k),
             sage.sage_quantize_qk_workspace_size(other.q, other.k))
    nv = max(sage.sage_quantize_v_workspace_size(inp.v), sage.sage_quantize_v_workspace_size(other.v))
    wq = torch.empty(nq, dtype=torch.uint8, device=dev)
    wv = torch.empty(nv, dtype=torch.uint8, device=dev)
    g = torch.Generator().manual_seed(11)
    for trial in range(5):
        if trial == 0:   # garbage
            wq.copy_(torch.randint(0, 256, (nq,), dtype=torch.uint8, generator=g))
            wv.copy_(torch.randint(0, 256, (nv,), dtype=torch.uint8, generator=g))
        if trial == 3:   # another layout on the same words
            sage.sage_quantize_qk(other.q, other.k, workspace=wq)
            sage.sage_quantize_v(other.v, workspace=wv)
        if trial == 4:   # all zero
            wq.zero_()
            wv.zero_()
        got = sage.sage_quantize_qk(inp.q, inp.k, workspace=wq)
        got_v = sage.sage_quantize_v(inp.v, workspace=wv)
        torch.cuda.synchronize()
        _same_qk(got, ref_qk)
        assert torch.equal(got_v[0].view(torch.uint8), ref_v[0].view(torch.uint8))
        assert torch.equal(got_v[1], ref_v[1])


@pytest.mark.parametrize("name,kw", [
    ("llm_prefill", dict(Lq=2100, Lk=2100, B=1, H=3)),   # 9 chunks, bf16, D 128
    ("tiny", dict(Lq=1000, Lk=1000, B=2, H=2)),          # 4 chunks, fp16, D 64
    ("video_dit", dict(Lq=700, Lk=700, H=2)),            # stacked strided views
])
def test_single_read_wait_bound(dev, name, kw):
    """With a zero wait bound a single-read block that does not find every
    chunk of its head at its first look withdraws its arrival and computes the
    head's statistic from the inputs itself: outputs bit-identical to the
    default, over calls in a row on one workspace, after which the default
    bound works on that workspace again; and in replays of a captured step
    (which share one launch number)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("quantizer wait bound 0", f"{name} {kw}")
    ref_qk = sage.sage_quantize_qk(inp.q, inp.k)
    ref_v = sage.sage_quantize_v(inp.v)
    wq = torch.empty(sage.sage_quantize_qk_workspace_size(inp.q, inp.k), dtype=torch.uint8, device=dev)
    wv = torch.empty(sage.sage_quantize_v_workspace_size(inp.v), dtype=torch.uint8, device=dev)

    def check(qk, v):
        _same_qk(qk, ref_qk)
        assert torch.equal(v[0].view(torch.uint8), ref_v[0].view(torch.uint8))
        assert torch.equal(v[1], ref_v[1])

    try:
        sage.sage_set_quant_wait_us(0)
        for _ in range(3):
            got = sage.sage_quantize_qk(inp.q, inp.k, workspace=wq)
            got_v = sage.sage_quantize_v(inp.v, workspace=wv)
            torch.cuda.synchronize()
            check(got, got_v)
        qk = sage.sage_quantize_qk(inp.q, inp.k, workspace=wq)
        vq, vs = sage.sage_quantize_v(inp.v, workspace=wv)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                sage.sage_quantize_qk(inp.q, inp.k, workspace=wq, into=qk)
                sage.sage_quantize_v(inp.v, workspace=wv, into=(vq, vs))
        torch.cuda.synchronize()
    finally:
        sage.sage_set_quant_wait_us(2000)
    for _ in range(3):
        for t in (qk.q, qk.q_scale, qk.k, qk.k_scale, qk.k_mean, vq.view(torch.uint8), vs):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(qk, (vq, vs))
    got = sage.sage_quantize_qk(inp.q, inp.k, workspace=wq)
    got_v = sage.sage_quantize_v(inp.v, workspace=wv)
    torch.cuda.synchronize()
    check(got, got_v)
    with pytest.raises(sage.SageError):
        sage.sage_set_quant_wait_us(-1)


@pytest.mark.parametrize("name,H", [("tiny", 9), ("llm_prefill", 9)])
def test_two_pass_path_bit_exact(dev, orc, name, H):
    """More chunks than the device holds at once (9 heads x 258 chunks of 256
    tokens, D 64 and D 128): the quantizers take the two-pass kernels (chunk
    statistics, their per-head finish, then the codes), whose results must be
    the oracle's too."""
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, Lq=66000, Lk=66000, B=1, H=H)
    say("two-pass quantizers", f"{name} distribution, {H} heads x 66000 tokens, D {w.D}")
    qk = sage.sage_quantize_qk(inp.q, inp.k)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    torch.cuda.synchronize()
    qc, kc, vc = canon(inp.q), canon(inp.k), canon(inp.v)
    L = kc.shape[2]
    mu_g = qk.k_mean.cpu().numpy()
    assert np.array_equal(mu_g, orc.k_mean(kc))
    q8, qs = orc.quant_int8(qc, 128)
    k8, ks = orc.quant_int8(orc.smooth_k(kc, mu_g), 64)
    assert np.array_equal(qk.q.cpu().numpy()[:, :, :L], q8)
    assert np.array_equal(qk.k.cpu().numpy()[:, :, :L], k8)
    assert np.array_equal(qk.q_scale.cpu().numpy(), qs)
    assert np.array_equal(qk.k_scale.cpu().numpy()[..., :ks.shape[-1]], ks)
    v8, vs = orc.quant_v_fp8(vc)
    assert np.array_equal(u8(v_q).transpose(0, 1, 3, 2)[:, :, :L], v8)
    assert np.array_equal(v_s.cpu().numpy(), vs)


def test_step_replayed_from_a_hip_graph(dev):
    """quantize_qk + quantize_v + attention captured in a HIP graph: every
    replay reproduces the eager step bit for bit, also after the workspaces
    served an eager call of another shape in between (the single-read
    quantizers' epoch words live there and advance on every call)."""
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=1100, Lk=1100, B=1, H=3)
    other = wl.make_prefill(w, device=dev, Lq=700, Lk=700, B=1, H=2)
    say("graph replay of a step", "llm_prefill 1100 x 3 heads")
    nq = max(sage.sage_quantize_qk_workspace_size(inp.q, inp.k),
             sage.sage_quantize_qk_workspace_size(other.q, other.k))
    nv = max(sage.sage_quantize_v_workspace_size(inp.v), sage.sage_quantize_v_workspace_size(other.v))
    wq = torch.empty(nq, dtype=torch.uint8, device=dev)
    wv = torch.empty(nv, dtype=torch.uint8, device=dev)
    qk = sage.sage_quantize_qk(inp.q, inp.k, workspace=wq)
    vq, vs = sage.sage_quantize_v(inp.v, workspace=wv)
    out = sage.sage_attn_fwd(qk, vq, vs, causal=True, sm_scale=w.sm_scale)

    def step():
        sage.sage_quantize_qk(inp.q, inp.k, workspace=wq, into=qk)
        sage.sage_quantize_v(inp.v, workspace=wv, into=(vq, vs))
        sage.sage_attn_fwd(qk, vq, vs, causal=True, sm_scale=w.sm_scale, out=out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (qk.q, qk.q_scale, qk.k, qk.k_scale, qk.k_mean, vq.view(torch.uint8), vs, out)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in (qk.q, qk.q_scale, qk.k, qk.k_scale, qk.k_mean, vq.view(torch.uint8), vs, out):
            t.zero_()
        if r == 2:
            sage.sage_quantize_qk(other.q, other.k, workspace=wq)
            sage.sage_quantize_v(other.v, workspace=wv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (qk.q, qk.q_scale, qk.k, qk.k_scale, qk.k_mean, vq.view(torch.uint8), vs, out)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (r, i)

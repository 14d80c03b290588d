"""Attention parity on the GPU.

* int32 QK score tiles of the attention kernel's own QK step are bit-exact
  against the oracle's integer product;
* outputs match the quantization-emulating oracle (same KV tiles) to
  cosine >= 0.999 and max-abs <= 1e-2 (fp32 outputs; bf16 outputs add half a
  bf16 ulp of the value for their own final rounding), and exact fp64
  attention to cosine >= 0.99 where the quantized method itself reaches it
  (on the outlier-heavy video-DiT inputs the method's own accuracy, measured
  by the oracle alone, is below that: there the GPU must match it);
* at the workloads' full sizes, in the launch configuration the benchmark
  times, sampled rows are checked against the oracle row by row;
* strided layouts, ragged tails, causal masks, GQA and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from quantized_attention_block_amd import workloads as wl
from tests._util import canon, cosine, require_gpu, say

pytestmark = pytest.mark.gpu

BN = 64   # KV tile of the kernel (part of the emulation's numeric definition)
COS_EMUL, MAXABS_EMUL, COS_EXACT = 0.999, 1e-2, 0.99


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _gpu_out(inp, causal, sm_scale, mode=sage.QK_INT8, hadamard=None, k_block=64,
             out_dtype=torch.float32):
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=mode, k_block=k_block, hadamard=hadamard)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    out = sage.sage_attn_fwd(qk, v_q, v_s, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, qk


def _half_ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def _check(out_g, out_o, exact=None, bf16=False, orc_exact=None):
    """out_g: GPU output; out_o: oracle emulation (fp32); exact: fp64 exact
    attention; orc_exact: the oracle emulation's own cosine against exact."""
    c = cosine(out_g, out_o)
    err = np.abs(out_g.astype(np.float64) - out_o)
    if bf16:
        err = np.maximum(err - _half_ulp_bf16(out_o), 0.0)
    m = float(err.max())
    assert c >= COS_EMUL, c
    assert m <= MAXABS_EMUL, m
    if exact is not None:
        ce = cosine(out_g, exact)
        floor = COS_EXACT if orc_exact is None else min(COS_EXACT, orc_exact - 0.002)
        print(f"cosine vs exact: gpu {ce:.5f}, oracle emulation {orc_exact}")
        assert ce >= floor, (ce, orc_exact)


# ---- int32 QK tiles ------------------------------------------------------------
@pytest.mark.parametrize("name,kw,tiles", [
    ("tiny", dict(), None),                                        # every tile
    ("llm_prefill", dict(Lq=520, Lk=520, B=1, H=2), None),         # ragged, every tile
    ("video_dit", dict(Lq=1000, Lk=1000, H=2), None),
])
def test_qk_tiles_bit_exact(dev, orc, name, kw, tiles):
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("qk tiles", name, kw)
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_INT8)
    Lqp, Lkp = qk.q.shape[2], qk.k.shape[2]
    S = sage.sage_debug_qk_tile(qk.q, qk.k, 0, Lqp, 0, Lkp)
    torch.cuda.synchronize()
    ref = orc.qk_int8_tile(qk.q.cpu().numpy(), qk.k.cpu().numpy())
    assert np.abs(ref).max() < 2 ** 31
    assert np.array_equal(S.cpu().numpy().astype(np.int64), ref)


def test_qk_tiles_full_size_sampled(dev, orc):
    """video-DiT at full length: 64 seeded 32x128 tiles plus every tile on the
    ragged edge (keys 32640..32767 hold the last 120 keys and 8 padded rows)."""
    w = wl.WORKLOADS["video_dit"]
    inp = wl.make_prefill(w, device=dev, H=2)
    say("qk tiles full length", w.Lq)
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_INT8)
    q8, k8 = qk.q.cpu().numpy(), qk.k.cpu().numpy()
    Lqp, Lkp = q8.shape[2], k8.shape[2]
    rng = np.random.default_rng(2024)
    picks = [(int(rng.integers(0, Lqp // 32)) * 32, int(rng.integers(0, Lkp // 128)) * 128)
             for _ in range(64)]
    picks += [(Lqp - 32, k0) for k0 in range(0, Lkp, 128 * 31)] + [(q0, Lkp - 128) for q0 in
                                                                    range(0, Lqp, 32 * 97)]
    picks.append((Lqp - 32, Lkp - 128))
    for q0, k0 in picks:
        S = sage.sage_debug_qk_tile(qk.q, qk.k, q0, 32, k0, 128).cpu().numpy()
        ref = orc.qk_int8_tile(q8[:, :, q0:q0 + 32], k8[:, :, k0:k0 + 128])
        assert np.array_equal(S.astype(np.int64), ref), (q0, k0)


def _ulp32(x):
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)


@pytest.mark.parametrize("kw,full", [(dict(Lq=1000, Lk=1000, H=2), True),
                                     (dict(Lq=520, Lk=333, H=1), True),
                                     (dict(), False)])          # full video-DiT length, sampled
def test_mxfp4_qk_tiles_within_one_ulp(dev, orc, kw, full):
    """fp32 MXFP4 score tiles of the attention kernel's QK step against the
    exact block-scaled integer sum (float64): within one fp32 ulp of the
    larger of the exact value and the first instruction's two-block partial
    sum (the MFMA rounds its fp32 accumulator once per instruction), and
    exact wherever the sums are representable."""
    w = wl.WORKLOADS["video_dit_mxfp4"]
    inp = wl.make_prefill(w, device=dev, **kw)
    had = sage.Hadamard(0)
    say("mxfp4 qk tiles", kw)
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_MXFP4, hadamard=had)
    torch.cuda.synchronize()
    q4, qe = orc.unpack_fp4(qk.q.cpu().numpy()), qk.q_scale.cpu().numpy()
    k4, ke = orc.unpack_fp4(qk.k.cpu().numpy()), qk.k_scale.cpu().numpy()
    Lqp, Lkp = q4.shape[2], k4.shape[2]
    if full:
        picks = [(0, Lqp, 0, Lkp)]
    else:
        rng = np.random.default_rng(77)
        picks = [(int(rng.integers(0, Lqp // 32)) * 32, 32, int(rng.integers(0, Lkp // 128)) * 128, 128)
                 for _ in range(16)] + [(Lqp - 32, 32, Lkp - 128, 128)]
    n_exact = n_all = 0
    for q0, nq, k0, nk in picks:
        S = sage.sage_debug_qk_tile_mx(qk, q0, nq, k0, nk).cpu().numpy().astype(np.float64)
        a = (q4[:, :, q0:q0 + nq], qe[:, :, q0:q0 + nq], k4[:, :, k0:k0 + nk], ke[:, :, k0:k0 + nk])
        ex = orc.qk_mxfp4_tile(*a)
        p01 = orc.qk_mxfp4_tile(*a, partial_blocks=2)
        err = np.abs(S - ex)
        assert np.all(err <= _ulp32(np.maximum(np.abs(ex), np.abs(p01)))), (q0, k0, float(err.max()))
        n_exact += int((err == 0).sum())
        n_all += err.size
    print(f"mxfp4 score tiles: {n_exact} of {n_all} exact")


# ---- outputs, reduced sizes (every row) ---------------------------------------------
@pytest.mark.parametrize("name,kw,causal", [
    ("tiny", dict(), False),
    ("tiny", dict(), True),
    ("llm_prefill", dict(Lq=640, Lk=640, B=2, H=2), True),
    ("llm_prefill", dict(Lq=520, Lk=520, B=1, H=2), True),     # ragged causal
    ("llm_prefill", dict(Lq=333, Lk=333, B=1, H=2), False),
    ("video_dit", dict(Lq=1000, Lk=1000, H=2), False),         # strided views, ragged
    ("tiny", dict(Lq=200, Lk=700), False),                     # Lq != Lk, D 64
    ("llm_prefill", dict(Lq=700, Lk=200, B=1, H=2), False),    # Lq != Lk, D 128
])
def test_int8_attention_matches_oracle(dev, orc, name, kw, causal):
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("int8 attention", name, kw, causal)
    out, qk = _gpu_out(inp, causal, w.sm_scale)
    q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
    ref, _ = orc.prefill_int8_pipeline(q, k, v, causal=causal, sm_scale=w.sm_scale, BN=BN,
                                       mu=qk.k_mean.cpu().numpy())
    exact = orc.attn_exact(q, k, v, causal, w.sm_scale)
    _check(canon(out), ref, exact, orc_exact=cosine(ref, exact) if name == "video_dit" else None)


@pytest.mark.parametrize("name,kw,causal", [
    ("llm_prefill", dict(Lq=520, Lk=520, B=1, H=2), True),
    ("video_dit", dict(Lq=700, Lk=1000, H=2), False),
])
def test_int8_attention_k_block_128(dev, orc, name, kw, causal):
    """K quantized per 128 keys: each 64-key tile takes the scale of the
    128-key block it lies in (both schedules for D 128)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, device=dev, **kw)
    say("int8 attention, k_block 128", name, kw, causal)
    out, qk = _gpu_out(inp, causal, w.sm_scale, k_block=128)
    q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
    ref, _ = orc.prefill_int8_pipeline(q, k, v, causal=causal, sm_scale=w.sm_scale, BN=BN, k_block=128,
                                       mu=qk.k_mean.cpu().numpy())
    _check(canon(out), ref, orc.attn_exact(q, k, v, causal, w.sm_scale),
           orc_exact=cosine(ref, orc.attn_exact(q, k, v, causal, w.sm_scale)) if name == "video_dit" else None)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    pp = sage.sage_attn_fwd(qk, v_q, v_s, causal=causal, sm_scale=w.sm_scale, out_dtype=torch.float32,
                            schedule=sage.SCHED_PINGPONG)
    torch.cuda.synchronize()
    assert torch.equal(pp, out)


@pytest.mark.parametrize("causal", [True, False])
def test_int8_attention_fp16_inputs_d128(dev, orc, causal):
    """fp16 Q/K/V at head dim 128 (the D-128 workloads are bf16): the fp16
    paths of the quantizers and of the fused-Q prologue against the oracle."""
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=520, Lk=520, B=1, H=2)
    q, k, v = (x.to(torch.float16) for x in (inp.q, inp.k, inp.v))
    say("int8 attention, fp16 inputs, D 128", causal)
    kq = sage.sage_quantize_qk(None, k)
    v_q, v_s = sage.sage_quantize_v(v)
    out = sage.sage_attn_fwd(kq, v_q, v_s, causal=causal, sm_scale=w.sm_scale, out_dtype=torch.float32, q=q)
    torch.cuda.synchronize()
    qc, kc, vc = canon(q), canon(k), canon(v)
    ref, _ = orc.prefill_int8_pipeline(qc, kc, vc, causal=causal, sm_scale=w.sm_scale, BN=BN,
                                       mu=kq.k_mean.cpu().numpy())
    _check(canon(out), ref, orc.attn_exact(qc, kc, vc, causal, w.sm_scale))


def test_gqa(dev, orc):
    """8 query heads on 2 KV heads: query head h reads KV head h // 4."""
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=384, Lk=384, B=1, H=8)
    kv = wl.make_prefill(w, device=dev, Lq=384, Lk=384, B=1, H=2)
    say("gqa")
    # quantize Q from the 8-head tensor and K from the 2-head tensor separately
    qq = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_INT8)
    kk = sage.sage_quantize_qk(kv.q, kv.k, mode=sage.QK_INT8)
    v_q, v_s = sage.sage_quantize_v(kv.v)
    mixed = sage.QuantizedQK(sage.QK_INT8, qq.q, qq.q_scale, kk.k, kk.k_scale, kk.k_mean, 384, 384,
                             128, 64)
    out = sage.sage_attn_fwd(mixed, v_q, v_s, causal=True, sm_scale=w.sm_scale, num_kv_heads=2,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, k, v = canon(inp.q), canon(kv.k), canon(kv.v)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    mu = np.repeat(kk.k_mean.cpu().numpy(), 4, axis=1)
    ref, _ = orc.prefill_int8_pipeline(q, kr, vr, causal=True, sm_scale=w.sm_scale, BN=BN, mu=mu)
    _check(canon(out), ref, orc.attn_exact(q, kr, vr, True, w.sm_scale))


def _mx_given_gpu_codes(orc, qk, v, w, causal, rows=None, sl=None):
    """The oracle's attention stage fed the GPU's own E2M1 codes and E8M0
    scales (so the last-bit differences of the rotation's fp32 sums, which
    move a few codes, are taken out of the comparison), with V quantized by
    the oracle.  sl: (b, h) to restrict the codes to one head; rows then
    index that head."""
    q4, qe, k4, ke = (t.cpu().numpy() for t in (qk.q, qk.q_scale, qk.k, qk.k_scale))
    if sl is not None:
        b, h = sl
        q4, qe, k4, ke = (x[b:b + 1, h:h + 1] for x in (q4, qe, k4, ke))
    Lq, Lk = qk.Lq, qk.Lk
    q4, k4 = orc.unpack_fp4(q4)[:, :, :Lq], orc.unpack_fp4(k4)[:, :, :Lk]
    qe, ke = qe[:, :, :Lq], ke[:, :, :Lk]
    v8, vs = orc.quant_v_fp8(v)
    B, H, _, D = q4.shape
    return orc.attn_emulated(B=B, H=H, Lq=Lq, Lk=Lk, D=D, causal=causal, sm_scale=w.sm_scale, BN=BN,
                             qk_mode=orc.QK_MXFP4, rows=rows, q4=q4, q_e8=qe, k4=k4, k_e8=ke, v8=v8,
                             v_scale=vs)


def test_mxfp4_attention_matches_oracle(dev, orc):
    w = wl.WORKLOADS["video_dit_mxfp4"]
    inp = wl.make_prefill(w, device=dev, Lq=1000, Lk=1000, H=2)
    had = sage.Hadamard(0)
    say("mxfp4 attention (no rotation, codes bit-exact)")
    out, qk = _gpu_out(inp, False, w.sm_scale, mode=sage.QK_MXFP4)
    q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
    mu = qk.k_mean.cpu().numpy()
    ref, _ = orc.prefill_mxfp4_pipeline(q, k, v, causal=False, sm_scale=w.sm_scale, BN=BN, mu=mu,
                                        rotate_qk=False)
    _check(canon(out), ref)
    say("mxfp4 attention (hadamard)")
    out, qk = _gpu_out(inp, False, w.sm_scale, mode=sage.QK_MXFP4, hadamard=had)
    exact = orc.attn_exact(q, k, v, False, w.sm_scale)
    # element-wise against the oracle's attention stage given the GPU's codes
    given = _mx_given_gpu_codes(orc, qk, v, w, False)
    ref, _ = orc.prefill_mxfp4_pipeline(q, k, v, causal=False, sm_scale=w.sm_scale, BN=BN, mu=mu)
    _check(canon(out), given, exact, orc_exact=cosine(ref, exact))
    # and the whole oracle pipeline (its own rotation and codes): cosine
    assert cosine(canon(out), ref) >= COS_EMUL


# ---- full sizes, sampled rows ---------------------------------------------------------
def _sampled_full(orc, inp, w, causal, heads, rows_per_head, mode=sage.QK_INT8, hadamard=None,
                  seed=0):
    # the benchmark's launch configuration: bf16 output
    out, qk = _gpu_out(inp, causal, w.sm_scale, mode=mode, hadamard=hadamard,
                       out_dtype=torch.bfloat16)
    out = out.float().cpu()
    mu_all = qk.k_mean.cpu().numpy()
    rng = np.random.default_rng(seed)
    got, want, exact = [], [], []
    for (b, h) in heads:
        sl = lambda t: t[b:b + 1, :, h:h + 1].float().cpu().permute(0, 2, 1, 3).contiguous().numpy()
        q, k, v = sl(inp.q), sl(inp.k), sl(inp.v)
        L = q.shape[2]
        rows_i = np.unique(np.concatenate([rng.integers(0, L, rows_per_head), [0, L - 1]]))
        rows = np.stack([np.zeros_like(rows_i), np.zeros_like(rows_i), rows_i], 1)
        mu = mu_all[b:b + 1, h:h + 1]
        if mode == sage.QK_INT8:
            r, _ = orc.prefill_int8_pipeline(q, k, v, causal=causal, sm_scale=w.sm_scale, BN=BN,
                                             mu=mu, rows=rows)
        else:
            r, _ = orc.prefill_mxfp4_pipeline(q, k, v, causal=causal, sm_scale=w.sm_scale, BN=BN,
                                              mu=mu, rows=rows, rotate_qk=hadamard is not None)
        want.append(r)
        exact.append(orc.attn_exact(q, k, v, causal, w.sm_scale, rows=rows))
        got.append(out[b, rows_i, h].numpy())
    return np.concatenate(got), np.concatenate(want), np.concatenate(exact)


def test_llm_prefill_full_size_sampled(dev, orc):
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev)
    say("llm prefill full size")
    g, r, e = _sampled_full(orc, inp, w, True, [(0, 0), (1, 17), (1, 31)], 48)
    _check(g, r, e, bf16=True)


def test_video_dit_full_size_sampled(dev, orc):
    w = wl.WORKLOADS["video_dit"]
    inp = wl.make_prefill(w, device=dev)
    say("video dit full size")
    g, r, e = _sampled_full(orc, inp, w, False, [(0, 0), (0, 39)], 12)
    _check(g, r, e, bf16=True, orc_exact=cosine(r, e))


def test_video_dit_mxfp4_full_size_sampled(dev, orc):
    """Full size: 3 heads x 48 sampled rows element-wise against the oracle's
    attention stage given the GPU's MXFP4 codes, and by cosine against the
    whole oracle pipeline (its own rotation) and exact attention."""
    w = wl.WORKLOADS["video_dit_mxfp4"]
    inp = wl.make_prefill(w, device=dev)
    had = sage.Hadamard(0)
    say("video dit mxfp4 full size")
    heads = [(0, 5), (0, 21), (0, 39)]
    g, r, e = _sampled_full(orc, inp, w, False, heads, 48, mode=sage.QK_MXFP4, hadamard=had, seed=3)
    qk = sage.sage_quantize_qk(inp.q, inp.k, mode=sage.QK_MXFP4, hadamard=had)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    given = []
    for (b, h) in heads:
        v = inp.v[b:b + 1, :, h:h + 1].float().cpu().permute(0, 2, 1, 3).contiguous().numpy()
        L = v.shape[2]
        rows_i = np.unique(np.concatenate([rng.integers(0, L, 48), [0, L - 1]]))
        rows = np.stack([np.zeros_like(rows_i), np.zeros_like(rows_i), rows_i], 1)
        given.append(_mx_given_gpu_codes(orc, qk, v, w, False, rows=rows, sl=(b, h)))
    given = np.concatenate(given)
    _check(g, given, e, bf16=True, orc_exact=cosine(r, e))
    assert cosine(g, r) >= COS_EMUL


# ---- layouts, output strides, determinism ------------------------------------------
def test_layouts_give_identical_results(dev):
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=300, Lk=300, B=2, H=4)
    say("layouts")
    base, _ = _gpu_out(inp, True, w.sm_scale, out_dtype=torch.bfloat16)
    # [B, H, L, D] memory viewed as logical [B, L, H, D]
    bhld = [t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (inp.q, inp.k, inp.v)]
    other = wl.PrefillInputs(*bhld)
    out2, _ = _gpu_out(other, True, w.sm_scale, out_dtype=torch.bfloat16)
    assert torch.equal(base, out2)
    # strided output: a [B, H, L, D] buffer written through a permuted view
    buf = torch.zeros((2, 4, 300, 128), dtype=torch.bfloat16, device=dev)
    qk = sage.sage_quantize_qk(inp.q, inp.k)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    sage.sage_attn_fwd(qk, v_q, v_s, causal=True, sm_scale=w.sm_scale, out=buf.permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    assert torch.equal(buf.permute(0, 2, 1, 3), base)
    # determinism
    out3, _ = _gpu_out(inp, True, w.sm_scale, out_dtype=torch.bfloat16)
    assert torch.equal(base, out3)
    # fp16 output equals the fp32 output rounded to fp16
    o32, _ = _gpu_out(inp, True, w.sm_scale)
    o16, _ = _gpu_out(inp, True, w.sm_scale, out_dtype=torch.float16)
    assert torch.equal(o32.half(), o16)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 127, 128, 129, 192, 255, 256, 257])
def test_boundary_lengths(dev, orc, L):
    """One query or key, and lengths on either side of the 64-key tile and
    the 128-query block: one to five KV tiles, full and ragged."""
    w = wl.WORKLOADS["llm_prefill"]
    inp = wl.make_prefill(w, device=dev, Lq=L, Lk=L, B=1, H=2)
    for causal in (False, True):
        say("boundary length", L, "causal" if causal else "non-causal")
        out, qk = _gpu_out(inp, causal, w.sm_scale)
        q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
        ref, _ = orc.prefill_int8_pipeline(q, k, v, causal=causal, sm_scale=w.sm_scale, BN=BN,
                                           mu=qk.k_mean.cpu().numpy())
        _check(canon(out), ref, orc.attn_exact(q, k, v, causal, w.sm_scale) if L > 1 else None)


@pytest.mark.parametrize("name,Lq,D,causal,dtype", [
    ("llm_prefill", 333, 128, True, torch.bfloat16),     # ragged last Q block
    ("llm_prefill", 4096, 128, True, torch.bfloat16),    # the benchmark's shape
    ("video_dit", 1000, 128, False, torch.bfloat16),     # outlier-heavy Q blocks
    ("llm_prefill", 200, 64, True, torch.float16),
    ("llm_prefill", 520, 128, True, torch.float16),     # fp16 at D 128
    ("video_dit", -700, 128, False, torch.bfloat16),     # Lq 700 against Lk 1500
])
def test_fused_q_quantization_equals_unfused(dev, name, Lq, D, causal, dtype):
    """Q quantized in the attention prologue (sage_quantize_qk(None, k) +
    sage_attn_fwd(q=...)) gives the unfused path's output bit for bit: the
    same INT8 codes and block scales, hence the same kernel arithmetic."""
    w = wl.WORKLOADS[name]
    Lq, Lk = (-Lq, 1500) if Lq < 0 else (Lq, Lq)
    inp = wl.make_prefill(w, Lq=Lq, Lk=Lk, device=dev)
    q, k, v = inp.q, inp.k, inp.v
    if D != q.shape[3] or dtype != q.dtype:
        q, k, v = (x[..., :D].to(dtype) for x in (q, k, v))
    say("fused Q quantization", name, Lq, D, causal, dtype)
    qk = sage.sage_quantize_qk(q, k)
    kq = sage.sage_quantize_qk(None, k)
    v_q, v_s = sage.sage_quantize_v(v)
    ref = sage.sage_attn_fwd(qk, v_q, v_s, causal=causal, sm_scale=w.sm_scale, out_dtype=torch.float32)
    got = sage.sage_attn_fwd(kq, v_q, v_s, causal=causal, sm_scale=w.sm_scale, out_dtype=torch.float32, q=q)
    torch.cuda.synchronize()
    assert kq.q is None and torch.equal(kq.k, qk.k) and torch.equal(kq.k_scale, qk.k_scale)
    assert torch.equal(got, ref)
    bf = sage.sage_attention(q, k, v, causal=causal, sm_scale=w.sm_scale)   # the fused convenience path
    assert torch.equal(bf, ref.to(dtype))


@pytest.mark.parametrize("name,Lq,Lk,H,Hkv,causal,fused,out_dtype", [
    ("llm_prefill", 1100, 1100, 3, 3, True, True, torch.bfloat16),     # 9 Q blocks: the last pair has one
    ("llm_prefill", 4096, 4096, 2, 2, True, True, torch.bfloat16),     # the benchmark's rows, two heads
    ("video_dit", 1000, 1000, 3, 3, False, True, torch.bfloat16),      # ragged tail, strided views
    ("video_dit", 700, 1500, 2, 2, False, False, torch.float32),       # Lq != Lk, Q quantized beforehand
    ("llm_prefill", 520, 520, 4, 2, True, True, torch.float16),        # GQA, 4 query heads on 2 KV heads
    ("video_dit", 32760, 32760, 1, 1, False, True, torch.bfloat16),    # the full video-DiT length, one head
    ("llm_prefill", 1, 1, 2, 2, True, True, torch.bfloat16),           # one row: one tile, second group empty
    ("video_dit", 100, 3000, 2, 2, False, False, torch.float32),       # one Q block against 47 tiles
])
def test_pingpong_schedule_equals_interleaved(dev, name, Lq, Lk, H, Hkv, causal, fused, out_dtype):
    """The wave-pair ping-pong schedule (8-wave workgroups over two Q blocks,
    MFMA and softmax phases of the two wave groups alternating) runs each
    row's arithmetic in the interleaved kernel's order: outputs equal bit for
    bit (the interleaved kernel is the one checked against the oracle)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_prefill(w, Lq=Lq, Lk=Lk, H=H, device=dev)
    q, k, v = inp.q, inp.k, inp.v
    if Hkv != H:
        k, v = k[:, :, :Hkv], v[:, :, :Hkv]
    say("ping-pong schedule", name, Lq, Lk, H, Hkv, causal, "fused Q" if fused else "Q codes", out_dtype)
    qk = sage.sage_quantize_qk(None if fused else q, k, want_mean=False)
    v_q, v_s = sage.sage_quantize_v(v)
    kw = dict(causal=causal, sm_scale=w.sm_scale, out_dtype=out_dtype, num_kv_heads=Hkv,
              q=q if fused else None)
    ref = sage.sage_attn_fwd(qk, v_q, v_s, **kw)
    got = sage.sage_attn_fwd(qk, v_q, v_s, schedule=sage.SCHED_PINGPONG, **kw)
    again = sage.sage_attn_fwd(qk, v_q, v_s, schedule=sage.SCHED_PINGPONG, **kw)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(again, ref)


@pytest.mark.parametrize("Lq,Lk,H,dtype,rotate", [
    (1000, 1000, 2, torch.bfloat16, True),      # strided video-DiT views, ragged last block
    (333, 333, 2, torch.bfloat16, False),       # no rotation
    (700, 1500, 2, torch.bfloat16, True),       # Lq != Lk
    (256, 256, 3, torch.float16, True),         # fp16 inputs: the fp16 Hadamard matrix
    (300, 300, 2, torch.float16, False),        # fp16 inputs, no rotation
    (32760, 32760, 1, torch.bfloat16, True),    # the full video-DiT length, one head
])
def test_fused_mxfp4_q_equals_unfused(dev, Lq, Lk, H, dtype, rotate):
    """Q rotated and quantized to MXFP4 in the attention prologue
    (sage_quantize_qk(None, k) + sage_attn_fwd(q=..., hadamard=...)) gives the
    unfused MXFP4 path's output bit for bit: the prologue runs the MXFP4
    quantizer's rotation and block arithmetic on the same rows."""
    w = wl.WORKLOADS["video_dit_mxfp4"]
    inp = wl.make_prefill(w, Lq=Lq, Lk=Lk, H=H, device=dev)
    q, k, v = inp.q, inp.k, inp.v
    if dtype != q.dtype:
        q, k, v = (x.to(dtype) for x in (q, k, v))
    had = sage.Hadamard(0) if rotate else None
    say("fused MXFP4 Q", Lq, Lk, H, dtype, "rotation" if rotate else "no rotation")
    qk = sage.sage_quantize_qk(q, k, mode=sage.QK_MXFP4, hadamard=had)
    kq = sage.sage_quantize_qk(None, k, mode=sage.QK_MXFP4, hadamard=had)
    v_q, v_s = sage.sage_quantize_v(v)
    ref = sage.sage_attn_fwd(qk, v_q, v_s, sm_scale=w.sm_scale, out_dtype=torch.float32)
    got = sage.sage_attn_fwd(kq, v_q, v_s, sm_scale=w.sm_scale, out_dtype=torch.float32, q=q, hadamard=had)
    torch.cuda.synchronize()
    assert kq.q is None and torch.equal(kq.k, qk.k) and torch.equal(kq.k_scale, qk.k_scale)
    assert torch.equal(got, ref)
    conv = sage.sage_attention(q, k, v, sm_scale=w.sm_scale, mode=sage.QK_MXFP4, hadamard=had)
    assert torch.equal(conv, ref.to(dtype))

"""Pins of the oracle's attention: exact fp64 attention against torch's
scaled_dot_product_attention (float64, CPU) and closed forms; the emulated
(tiled, online-softmax) machinery against exact attention with quantization
switched off; quantized emulation against the bounds its rounding allows."""
import numpy as np
import pytest
import torch

from tests._util import base2_attention, dyadic_prefill


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _sdpa(q, k, v, causal, scale):
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_exact_matches_torch_sdpa(orc, causal):
    q, k, v = _rand((2, 3, 45, 32), 1), _rand((2, 3, 45, 32), 2), _rand((2, 3, 45, 32), 3)
    out = orc.attn_exact(q, k, v, causal, 0.3)
    assert np.allclose(out, _sdpa(q, k, v, causal, 0.3), rtol=1e-12, atol=1e-12)


def test_exact_rows_subset(orc):
    q, k, v = _rand((1, 2, 20, 16), 4), _rand((1, 2, 33, 16), 5), _rand((1, 2, 33, 16), 6)
    full = orc.attn_exact(q, k, v, False, 0.25)
    rows = np.array([[0, 1, 7], [0, 0, 19], [0, 1, 0]])
    sub = orc.attn_exact(q, k, v, False, 0.25, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(sub[r], full[b, h, i])


def test_exact_closed_forms(orc):
    v = _rand((1, 1, 9, 8), 7)
    # one key: the output is that key's value
    out = orc.attn_exact(_rand((1, 1, 4, 8), 8), _rand((1, 1, 1, 8), 9), v[:, :, :1], False, 1.0)
    assert np.allclose(out, np.broadcast_to(v[:, :, :1], out.shape), atol=1e-12)
    # zero queries: uniform weights (mean of V); causal: prefix means
    q0 = np.zeros((1, 1, 9, 8), np.float32)
    k = _rand((1, 1, 9, 8), 10)
    out = orc.attn_exact(q0, k, v, False, 1.0)
    assert np.allclose(out, np.broadcast_to(v.astype(np.float64).mean(2, keepdims=True), out.shape))
    out = orc.attn_exact(q0, k, v, True, 1.0)
    pref = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 10)[None, None, :, None]
    assert np.allclose(out, pref)
    # one dominant key
    k = np.zeros((1, 1, 9, 8), np.float32)
    k[0, 0, 4, 0] = 100.0
    q = np.zeros((1, 1, 1, 8), np.float32)
    q[0, 0, 0, 0] = 1.0
    out = orc.attn_exact(q, k, v, False, 1.0)
    assert np.allclose(out[0, 0, 0], v[0, 0, 4], atol=1e-30 + 1e-12)


def test_smoothing_invariance(orc):
    q = _rand((1, 2, 30, 32), 11)
    k = _rand((1, 2, 50, 32), 12) + _rand((1, 2, 1, 32), 13, 5.0)
    v = _rand((1, 2, 50, 32), 14)
    mu = orc.k_mean(k)
    # K - mu is rounded to fp32 (ulp ~ 5e-7 at |K| ~ 8), so the shift
    # invariance of softmax holds to that rounding, not to fp64 precision.
    a0 = orc.attn_exact(q, k, v, False, 0.2)
    b = orc.attn_exact(q, orc.smooth_k(k, mu), v, False, 0.2)
    assert np.abs(a0 - b).max() < 2e-5
    qq = _rand((1, 2, 50, 32), 15)
    a = orc.attn_exact(qq, k, v, True, 0.2)
    b = orc.attn_exact(qq, orc.smooth_k(k, mu), v, True, 0.2)
    assert np.abs(a - b).max() < 2e-5
    # a per-token (not per-channel) shift is NOT invariant: the check has teeth
    bad = k - k.mean(axis=3, keepdims=True)
    c = orc.attn_exact(q, bad, v, False, 0.2)
    assert np.abs(a0 - c).max() > 1e-3


def _emul_float(orc, q, k, v, causal, scale, BN):
    B, H, Lq, D = q.shape
    return orc.attn_emulated(B=B, H=H, Lq=Lq, Lk=k.shape[2], D=D, causal=causal, sm_scale=scale,
                             BN=BN, qk_mode=orc.QK_FLOAT, quant_pv=False, qf=q, kf=k, vf=v)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BN", [1, 16, 64, 128, 1000])
def test_emulation_without_quantization_is_exact(orc, causal, BN):
    L = 150                                              # ragged against every BN
    q, k, v = _rand((1, 2, L, 32), 21, 2.0), _rand((1, 2, L, 32), 22, 2.0), _rand((1, 2, L, 32), 23)
    out = _emul_float(orc, q, k, v, causal, 0.4, BN)
    ref = orc.attn_exact(q, k, v, causal, 0.4)
    # fp32 state: one rounding per tile of the running rescale, |out| <= ~3
    assert np.abs(out - ref).max() < 1e-5


def test_emulation_row_sum_is_one(orc):
    q, k = _rand((1, 1, 64, 16), 31, 3.0), _rand((1, 1, 200, 16), 32, 3.0)
    ones = np.ones((1, 1, 200, 16), np.float32)
    out = _emul_float(orc, q, k, ones, False, 1.0, 64)
    assert np.abs(out - 1.0).max() < 1e-6


def _tiny_int8(orc, q, k, v, causal, scale, BN, qb=128, kb=64):
    return orc.prefill_int8_pipeline(q, k, v, causal=causal, sm_scale=scale, BN=BN,
                                     q_block=qb, k_block=kb)


def test_int8_pipeline_p_rounding_bound(orc):
    """With V = 1 the output is sum_j P8_j / (448 l); every P8 is within 2^-4
    relative of 448 p (normals) or 2^-10 absolute (subnormals)."""
    L = 300
    q, k = _rand((1, 2, L, 64), 41), _rand((1, 2, L, 64), 42)
    v = np.ones((1, 2, L, 64), np.float32)
    out, it = _tiny_int8(orc, q, k, v, False, 0.125, 128)
    assert np.all(it["v8"] == 0x7E)                      # 448 everywhere
    # |sum P8/(448 l) - 1| <= 2^-4 + Lk * 2^-10 / (448 l); l >= 1 (max term is 1)
    bound = 2.0 ** -4 + L * 2.0 ** -10 / 448.0
    assert np.abs(out - 1.0).max() <= bound


@pytest.mark.parametrize("causal", [False, True])
def test_int8_pipeline_close_to_exact(orc, causal):
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS["tiny"]
    inp = wl.make_prefill(w)
    canon = lambda t: t.float().permute(0, 2, 1, 3).contiguous().numpy()
    q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
    out, _ = _tiny_int8(orc, q, k, v, causal, w.sm_scale, 64)
    ref = orc.attn_exact(q, k, v, causal, w.sm_scale)
    cos = (out.ravel() @ ref.ravel()) / np.linalg.norm(out) / np.linalg.norm(ref)
    assert cos >= 0.999


def test_mxfp4_scores_match_float_path(orc):
    """Inputs that are exactly representable in MXFP4 (E2M1 values times a
    power-of-two block scale): the MXFP4 block arithmetic must reproduce the
    float dot products."""
    rng = np.random.default_rng(51)
    vals = np.array([orc.e2m1_decode(c) for c in range(16)], np.float32)
    B, H, L, D = 1, 2, 96, 64

    def draw(seed):
        r = np.random.default_rng(seed)
        codes = r.integers(0, 16, (B, H, L, D)).astype(np.uint8)
        e = r.integers(124, 130, (B, H, L, D // 32)).astype(np.uint8)
        x = vals[codes] * np.repeat(2.0 ** (e.astype(np.float32) - 127), 32, axis=-1)
        return codes, e, x.astype(np.float32)

    q4, qe, qf = draw(52)
    k4, ke, kf = draw(53)
    v = _rand((B, H, L, D), 54)
    common = dict(B=B, H=H, Lq=L, Lk=L, D=D, causal=False, sm_scale=0.02, BN=32)
    a = orc.attn_emulated(qk_mode=orc.QK_MXFP4, quant_pv=False, q4=q4, q_e8=qe, k4=k4, k_e8=ke,
                          vf=v, **common)
    b = orc.attn_emulated(qk_mode=orc.QK_FLOAT, quant_pv=False, qf=qf, kf=kf, vf=v, **common)
    assert np.abs(a - b).max() < 1e-5


def test_mxfp4_quantizer_roundtrip_on_representable(orc):
    rng = np.random.default_rng(61)
    vals = np.array([orc.e2m1_decode(c) for c in range(8)], np.float32)
    codes = rng.integers(0, 8, (1, 1, 10, 64)).astype(np.uint8)
    codes[..., ::32] = 7                                  # amax = 6 * 2^e in every block
    e = rng.integers(100, 150, (1, 1, 10, 2)).astype(np.uint8)
    x = vals[codes] * np.repeat(2.0 ** (e.astype(np.float32) - 127), 32, axis=-1)
    c4, ce = orc.quant_mxfp4(x.astype(np.float32))
    assert np.array_equal(ce, e) and np.array_equal(c4, codes)


def test_mxfp4_pipeline_against_exact(orc):
    """MXFP4 QK error is the E2M1 grid's (about 11% relative per element at
    one mantissa bit): the emulation must equal exact attention on the
    dequantized (rotated) Q/K up to the e4m3 P/V rounding, and exact attention
    on the original inputs up to that quantization error."""
    q, k, v = _rand((1, 2, 256, 128), 71), _rand((1, 2, 256, 128), 72), _rand((1, 2, 256, 128), 73)
    k = k + _rand((1, 2, 1, 128), 74, 2.0)
    out, it = orc.prefill_mxfp4_pipeline(q, k, v, causal=False, sm_scale=128 ** -0.5, BN=128)
    vals = np.array([orc.e2m1_decode(c) for c in range(16)], np.float32)
    deq = lambda c, e: vals[c] * np.repeat(2.0 ** (e.astype(np.float32) - 127), 32, axis=-1)
    qd, kd = deq(it["q4"], it["q_e8"]), deq(it["k4"], it["k_e8"])
    cos = lambda a, b: (a.ravel() @ b.ravel()) / np.linalg.norm(a) / np.linalg.norm(b)
    on_deq = orc.attn_exact(qd, kd, v, False, 128 ** -0.5)
    assert cos(out, on_deq) >= 0.999
    ref = orc.attn_exact(q, k, v, False, 128 ** -0.5)
    assert cos(out, ref) >= 0.98
    # the rotation is orthogonal: the un-quantized rotated scores are the originals
    sr = it["q_rot"][0, 0].astype(np.float64) @ it["k_rot"][0, 0].astype(np.float64).T
    ks = orc.smooth_k(k, it["mu"])
    s0 = q[0, 0].astype(np.float64) @ ks[0, 0].astype(np.float64).T
    assert np.abs(sr - s0).max() < 1e-3


# ---- quantized emulation on inputs where every rounding is exact -----------
# (tests._util.dyadic_prefill): a dropped or misplaced rescale, scale, mask or
# 448 factor changes some weight by a power of two.

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BN", [32, 64])
def test_int8_pipeline_exact_on_dyadic_inputs(orc, causal, BN):
    """INT8: every Q row has a 254 (q_scale 2, codes Q / 2), K has an
    alternating +-127 channel (k_scale 1 in every 64-row block, also the
    8-row tail), alpha = fp32(ln2 / 2 * log2 e) = 0.5, so x = q.k / 2 with q
    in {0, +-2, +-4} and k in {0, +-1}: integers in [-6, 6].  V in
    {0, +-1, +-2, +-4} with amax 4 (codes 112 v, v_scale 4 / 448)."""
    L, D = 200, 64
    q, k, v = dyadic_prefill(81, L, D, [0.0, 2.0, -2.0, 4.0, -4.0], [0.0, 1.0, -1.0], 254.0, 127.0)
    out, it = _tiny_int8(orc, q, k, v, causal, np.log(2.0) / 2, BN)
    assert np.all(it["mu"] == 0.0)
    assert np.all(it["q_scale"] == 2.0) and np.all(it["k_scale"] == 1.0)
    x = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) / 2
    assert np.array_equal(x, np.round(x)) and np.abs(x).max() <= 6
    ref = base2_attention(x, v, causal)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_pipeline_exact_on_dyadic_inputs(orc, causal):
    """MXFP4 without rotation: every 32-channel block that holds data has amax
    4 (E8M0 exponent 0, E2M1 codes = the values), the others are all zero;
    x = S alpha with alpha = 0.5 and S = q.k with q in {0, +-2}, k in
    {0, +-1, +-2}: integers in [-6, 6]."""
    L, D = 160, 64
    q, k, v = dyadic_prefill(82, L, D, [0.0, 2.0, -2.0], [0.0, 1.0, -1.0, 2.0, -2.0], 4.0, 4.0)
    out, it = orc.prefill_mxfp4_pipeline(q, k, v, causal=causal, sm_scale=np.log(2.0) / 2, BN=32,
                                         rotate_qk=False)
    assert np.all(it["mu"] == 0.0)
    assert np.all(it["q_e8"][..., 0] == 127) and np.all(it["k_e8"][..., 0] == 127)
    x = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) / 2
    assert np.array_equal(x, np.round(x)) and np.abs(x).max() <= 6
    ref = base2_attention(x, v, causal)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()

"""Shared helpers of the parity tests (layout conversions, metrics, and seeded
inputs on which every quantization step is exact)."""
import sys

import numpy as np
import torch


def say(*a):
    """Names the case before a GPU step (flushed, so a fault still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def canon(t: torch.Tensor) -> np.ndarray:
    """Logical [B, L, H, D] tensor -> float32 numpy [B, H, L, D] (exact upcast)."""
    return t.detach().float().permute(0, 2, 1, 3).contiguous().cpu().numpy()


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from quantized_attention_block_amd import sage
    sage.lib()
    return torch.device("cuda", 0)


# ---- inputs on which every quantization step is exact ----------------------
# With integer scores x (in log2 units), 448 * 2^(x - m) is an e4m3 value for
# x - m >= -15, the rescale factors are powers of two, INT8 / MXFP4 / e4m3
# codes of the chosen values are the values themselves (up to a power-of-two
# or fixed scale), and the K mean is exactly 0.  The quantized pipelines must
# then reproduce base-2 attention on the integer scores, written out below in
# float64.

def softmax_accumulation_bound(n):
    """Bound on |out - exact| / max|v| for the GPU softmax-PV on dyadic inputs
    (integer scores, power-of-two or unit scales, e4m3-exact values), where
    every quantization step is exact and only fp32 arithmetic rounds:

    * the row sum l adds n positive fp32 terms on the vector ALU
      (round-to-nearest): relative error at most gamma(n, u) = n u / (1 - n u),
      u = 2^-24, in any summation order;
    * O = sum P8 V8 has exact products (e4m3 x e4m3 fits fp32) accumulated
      by the MFMA, whose internal order and rounding are not documented:
      bounded as if each of the n additions could lose a whole ulp
      (truncation), gamma(n, 2u) sum |P8 V8| <= gamma(n, 2u) 448 l max|V8|
      (P8 >= 0), that is gamma(n, 2u) max|v| after the division by l.  (With
      round-to-nearest here too, the causal MXFP4 case at n = 160 measured
      2.4e-5 of max|v|, above the 2.1e-5 that model allows.);
    * each p = 2^(S c - m + log2 448) comes from the approximate hardware exp2
      of a non-integer argument (log2 448 and the folded offset are rounded to
      fp32): within 2^-19 relatively, enough for P8 = e4m3(448 p) to round to
      its exact value, but it enters l;
    * the epilogue's v_scale product, reciprocal and product: 3 u.
    Together gamma(n, u) + gamma(n, 2u) + 2^-19 + 3 u (relative to max|v|),
    n = the keys one fp32 sum runs over."""
    u = 2.0 ** -24
    gamma = lambda uu: n * uu / (1.0 - n * uu)
    return gamma(u) + gamma(2.0 * u) + 2.0 ** -19 + 3.0 * u


def base2_attention(x, v, causal):
    """sum_j 2^x_ij v_j / sum_j 2^x_ij over visible j (j <= i when causal)."""
    x = x.astype(np.float64)
    if causal:
        Lq, Lk = x.shape[-2:]
        x = np.where(np.tril(np.ones((Lq, Lk), bool)), x, -np.inf)
    w = 2.0 ** (x - x.max(-1, keepdims=True))
    return (w @ v.astype(np.float64)) / w.sum(-1, keepdims=True)


def _paired(rng, vals, shape):
    """Draws from vals for the first half of the tokens (axis 2) and negates
    them for the second half, so every channel sums to exactly 0."""
    B, H, L, D = shape
    half = rng.choice(vals, (B, H, L // 2, D))
    return np.concatenate([half, -half], axis=2)


def dyadic_prefill(seed, L, D, q_vals, k_vals, q_amax_val, k_amax_val, n_score=3):
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    q = np.zeros((B, H, L, D), np.float32)
    k = np.zeros((B, H, L, D), np.float32)
    q[..., :n_score] = rng.choice(q_vals, (B, H, L, n_score))
    k[..., :n_score] = _paired(rng, k_vals, (B, H, L, n_score))
    q[..., n_score] = q_amax_val                       # Q's block amax; K is 0 there
    k[..., n_score + 1] = k_amax_val * (1 - 2 * (np.arange(L) % 2))   # +-, mean 0; Q is 0 there
    v = rng.choice(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], np.float32), (B, H, L, D))
    v[..., 0, :] = 4.0                                  # every channel's amax is 4
    return q, k, v.astype(np.float32)


def dyadic_decode(seed, *, B, MTP, Hq, Hkv, D, PS, max_pages):
    """Decode inputs with exact quantization: every Q row has a 448 (q_scale
    1, codes = Q) in a channel where K is 0; score channels hold q in
    {0, +-2} and k in {0, +-1}; k_scale is 1 or 2 and v_scale 1/2, 1 or 2, so
    with alpha = 0.5 (sm_scale = ln 2 / 2) the scores are integers in [-4, 4]
    and the folded P8 = e4m3(448 p v_scale / vmax) is exact.  Returns float32
    q [B, MTP, Hq, D], cache values kf, vf [P, Hkv, PS, D] (e4m3-exact),
    scales [P, Hkv, PS] and a page table [B, max_pages] (a permutation)."""
    rng = np.random.default_rng(seed)
    P = B * max_pages
    q = np.zeros((B, MTP, Hq, D), np.float32)
    q[..., :2] = rng.choice([0.0, 2.0, -2.0], (B, MTP, Hq, 2))
    q[..., 2] = 448.0
    kf = rng.choice(np.array([0.0, 1.0, -1.0, 0.5, 3.0], np.float32), (P, Hkv, PS, D))
    kf[..., :2] = rng.choice([0.0, 1.0, -1.0], (P, Hkv, PS, 2))
    kf[..., 2] = 0.0
    vf = rng.choice(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -0.5], np.float32), (P, Hkv, PS, D))
    ks = rng.choice(np.array([1.0, 2.0], np.float32), (P, Hkv, PS))
    vs = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), (P, Hkv, PS))
    table = rng.permutation(P).astype(np.int32).reshape(B, max_pages)
    return q, kf, vf, ks, vs, table


def base2_decode(q, kf, vf, ks, vs, table, ctx, window, Hkv):
    """sum_t 2^x_t v_scale_t V_t / sum_t 2^x_t over the window of each query
    (query m of sequence b at position ctx_b - MTP + m), x_t = q.k_t k_scale_t / 2."""
    B, MTP, Hq, D = q.shape
    G = Hq // Hkv
    ref = np.zeros((B, MTP, Hq, D), np.float64)
    for b in range(B):
        pages = table[b]
        kt = kf[pages].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)   # [Hkv, tokens, D]
        vt = vf[pages].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)
        kst = ks[pages].transpose(1, 0, 2).reshape(Hkv, -1)
        vst = vs[pages].transpose(1, 0, 2).reshape(Hkv, -1)
        for m in range(MTP):
            pos = int(ctx[b]) - MTP + m
            lo = max(0, pos - window + 1) if window > 0 else 0
            t = np.arange(lo, pos + 1)
            for hq in range(Hq):
                hk = hq // G
                x = (kt[hk, t].astype(np.float64) @ q[b, m, hq].astype(np.float64)) * kst[hk, t] / 2
                assert np.array_equal(x, np.round(x)) and np.abs(x).max() <= 4
                w = 2.0 ** (x - x.max())
                ref[b, m, hq] = (w * vst[hk, t]) @ vt[hk, t].astype(np.float64) / w.sum()
    return ref

"""Pins of the oracle's paged decode: the page's window-tile counts, reduction
to exact attention of the last MTP rows (float mode), invariance to page
placement and to the split length, and the quantized mode against exact."""
import json
import os

import numpy as np
import pytest

from tests._util import base2_decode, dyadic_decode

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_window_tiles_match_page(orc):
    with open(os.path.join(GOLD, "aiter7388_window_tiles.json")) as f:
        g = json.load(f)
    for window, tiles in g["cases"]:
        assert orc.decode_num_splits(window, g["mtp"], g["tile"]) == tiles
        # and it is the largest number of tile-aligned windows a span of
        # window + mtp - 1 consecutive keys touches, over every alignment
        span = window + g["mtp"] - 1
        brute = max((s + span - 1) // g["tile"] - s // g["tile"] + 1 for s in range(g["tile"]))
        assert brute == tiles


def _contiguous_cache(k, v, page):
    """[B, ctx, Hkv, D] float -> identity-paged caches [P, Hkv, page, D]."""
    B, ctx, Hkv, D = k.shape
    pps = ctx // page
    kc = k.reshape(B, pps, page, Hkv, D).transpose(0, 1, 3, 2, 4).reshape(B * pps, Hkv, page, D)
    vc = v.reshape(B, pps, page, Hkv, D).transpose(0, 1, 3, 2, 4).reshape(B * pps, Hkv, page, D)
    table = np.arange(B * pps, dtype=np.int32).reshape(B, pps)
    return np.ascontiguousarray(kc), np.ascontiguousarray(vc), table


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("window", [0, 40, 100])
@pytest.mark.parametrize("tile", [16, 32, 256])
def test_float_mode_is_exact_attention(orc, window, tile):
    B, ctx, Hq, Hkv, D, MTP, page = 2, 96, 4, 2, 16, 3, 16
    k, v = _rand((B, ctx, Hkv, D), 1), _rand((B, ctx, Hkv, D), 2)
    q = _rand((B, MTP, Hq, D), 3, 2.0)
    kc, vc, table = _contiguous_cache(k, v, page)
    ones = np.ones(kc.shape[:3], np.float32)
    out = orc.paged_decode(q, kc, vc, ones, ones, table, np.full(B, ctx, np.int32),
                           window=window, sm_scale=0.3, tile=tile, quant=False)
    for b in range(B):
        for m in range(MTP):
            pos = ctx - MTP + m
            lo = max(0, pos - window + 1) if window else 0
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                ref = orc.attn_exact(q[b, m, h][None, None, None], k[b, lo:pos + 1, hk][None, None],
                                     v[b, lo:pos + 1, hk][None, None], False, 0.3)
                assert np.abs(out[b, m, h] - ref[0, 0, 0]).max() < 2e-6


def test_float_mode_applies_per_token_scales(orc):
    B, ctx, Hkv, D, page = 1, 64, 1, 8, 16
    k, v = _rand((B, ctx, Hkv, D), 4), _rand((B, ctx, Hkv, D), 5)
    ks = np.abs(_rand((ctx,), 6)) + 0.5
    vs = np.abs(_rand((ctx,), 7)) + 0.5
    q = _rand((B, 1, 2, D), 8)
    kc, vc, table = _contiguous_cache(k, v, page)
    kss = ks.reshape(-1, 1, page)
    vss = vs.reshape(-1, 1, page)
    out = orc.paged_decode(q, kc, vc, kss, vss, table, np.full(B, ctx, np.int32), window=0,
                           sm_scale=0.5, tile=32, quant=False)
    kk = k[0, :, 0] * ks[:, None]
    vv = v[0, :, 0] * vs[:, None]
    for h in range(2):
        ref = orc.attn_exact(q[0, 0, h][None, None, None], kk[None, None], vv[None, None], False, 0.5)
        assert np.abs(out[0, 0, h] - ref[0, 0, 0]).max() < 2e-6


def test_page_permutation_invariance(orc):
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=2, ctx=600)
    q = inp.q.float().numpy()
    kc, vc = inp.k_cache.numpy(), inp.v_cache.numpy()
    ks, vs = inp.k_scale.numpy(), inp.v_scale.numpy()
    table, ctx = inp.page_table.numpy(), inp.ctx_lens.numpy()
    common = dict(window=256, sm_scale=w.sm_scale, tile=256)
    a = orc.paged_decode(q, kc, vc, ks, vs, table, ctx, **common)
    perm = np.random.default_rng(9).permutation(kc.shape[0])
    inv = np.argsort(perm)
    b = orc.paged_decode(q, kc[perm], vc[perm], ks[perm], vs[perm], inv[table].astype(np.int32),
                         ctx, **common)
    assert np.array_equal(a, b)


def test_quant_mode_close_to_exact(orc):
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=2, ctx=1100)
    q = inp.q.float().numpy()
    kc, vc = inp.k_cache.numpy(), inp.v_cache.numpy()
    ks, vs = inp.k_scale.numpy(), inp.v_scale.numpy()
    table, ctx = inp.page_table.numpy(), inp.ctx_lens.numpy()
    out = orc.paged_decode(q, kc, vc, ks, vs, table, ctx, window=512, sm_scale=w.sm_scale)
    kf = orc.e4m3_decode_array(kc) * ks[..., None]
    vf = orc.e4m3_decode_array(vc) * vs[..., None]
    ref = orc.paged_decode(q, kf, vf, np.ones_like(ks), np.ones_like(vs), table, ctx,
                           window=512, sm_scale=w.sm_scale, quant=False)
    cos = (out.ravel() @ ref.ravel()) / np.linalg.norm(out) / np.linalg.norm(ref)
    assert cos >= 0.999
    # the split length changes nothing in float mode
    ref2 = orc.paged_decode(q, kf, vf, np.ones_like(ks), np.ones_like(vs), table, ctx,
                            window=512, sm_scale=w.sm_scale, quant=False, tile=64)
    assert np.abs(ref - ref2).max() < 2e-6


@pytest.mark.parametrize("window,tile", [(0, 32), (20, 32), (0, 256)])
def test_quant_mode_exact_on_dyadic_inputs(orc, window, tile):
    """Quantized decode on inputs where every rounding is exact
    (tests._util.dyadic_decode): the result must be base-2 attention of the
    integer scores over each query's window with the per-token V scale
    applied; a wrong mask, fold, split or merge changes some weight by a
    power of two."""
    MTP, Hq, Hkv = 4, 4, 2
    ctx = np.array([100, 57], np.int32)
    q, kf, vf, ks, vs, table = dyadic_decode(91, B=2, MTP=MTP, Hq=Hq, Hkv=Hkv, D=32, PS=16, max_pages=8)
    kc, vc = orc.e4m3_encode_array(kf), orc.e4m3_encode_array(vf)
    assert np.array_equal(orc.e4m3_decode_array(kc), kf) and np.array_equal(orc.e4m3_decode_array(vc), vf)
    out = orc.paged_decode(q, kc, vc, ks, vs, table, ctx, window=window, sm_scale=np.log(2.0) / 2,
                           tile=tile)
    ref = base2_decode(q, kf, vf, ks, vs, table, ctx, window, Hkv)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


def _mx_cache(seed, P, Hkv, PS, D):
    """Random MXFP4 KV cache (one E2M1 code per byte) with exponents in
    [124, 130], and its dequantized K [P, Hkv, PS, D] and V [P, Hkv, PS, D]."""
    from oracle import e2m1_decode
    rng = np.random.default_rng(seed)
    vals = np.array([e2m1_decode(c) for c in range(16)], np.float64)
    kc = rng.integers(0, 16, (P, Hkv, PS, D)).astype(np.uint8)
    ke = rng.integers(124, 131, (P, Hkv, PS, D // 32)).astype(np.uint8)
    vc = rng.integers(0, 16, (P, Hkv, D, PS)).astype(np.uint8)          # V transposed
    ve = rng.integers(124, 131, (P, Hkv, D, PS // 32)).astype(np.uint8)
    kf = vals[kc] * np.repeat(2.0 ** (ke.astype(np.float64) - 127), 32, axis=-1)
    vf = (vals[vc] * np.repeat(2.0 ** (ve.astype(np.float64) - 127), 32, axis=-1)).transpose(0, 1, 3, 2)
    return kc, ke, vc, ve, kf.astype(np.float32), np.ascontiguousarray(vf).astype(np.float32)


@pytest.mark.parametrize("D,PS,window,tile", [(128, 64, 0, 256), (128, 32, 40, 64), (64, 64, 0, 32)])
def test_mx_decode_equals_fp8_decode_on_shared_values(orc, D, PS, window, tile):
    """E2M1 values times 2^(e - 127) for e in [124, 130] are e4m3 values, so
    an MXFP4 cache has an exact e4m3 twin with unit per-token scales; on it
    the FP8 path computes the same scores, P8 and products (its vmax is 1),
    and the two oracles must agree bit for bit."""
    B, MTP, Hq, Hkv, max_pages = 2, 4, 4, 2, 6
    P = B * max_pages
    rng = np.random.default_rng(7)
    q = rng.standard_normal((B, MTP, Hq, D)).astype(np.float32)
    kc, ke, vc, ve, kf, vf = _mx_cache(8, P, Hkv, PS, D)
    k8, v8 = orc.e4m3_encode_array(kf), orc.e4m3_encode_array(vf)
    assert np.array_equal(orc.e4m3_decode_array(k8), kf) and np.array_equal(orc.e4m3_decode_array(v8), vf)
    table = rng.permutation(P).astype(np.int32).reshape(B, max_pages)
    ctx = np.array([max_pages * PS - 5, 3 * PS + 7], np.int32)
    ones = np.ones((P, Hkv, PS), np.float32)
    common = dict(window=window, sm_scale=D ** -0.5, tile=tile)
    a = orc.paged_decode_mx(q, kc, ke, vc, ve, table, ctx, **common)
    b = orc.paged_decode(q, k8, v8, ones, ones, table, ctx, **common)
    assert np.array_equal(a, b)
    assert np.abs(a).max() > 0


@pytest.mark.parametrize("per_tensor", [True, False])
def test_e4m3_query_exact_on_dyadic_inputs(orc, per_tensor):
    """The query given already in e4m3 (codes + fp32 scale per tensor or per
    (token, head) row) instead of bf16: on the exact inputs of
    test_quant_mode_exact_on_dyadic_inputs, with codes q / s for power-of-two
    scales s (every code exact), the result is base-2 attention again; a
    dropped or misplaced query scale moves every score by a power of two."""
    MTP, Hq, Hkv = 4, 4, 2
    ctx = np.array([100, 57], np.int32)
    q, kf, vf, ks, vs, table = dyadic_decode(91, B=2, MTP=MTP, Hq=Hq, Hkv=Hkv, D=32, PS=16, max_pages=8)
    kc, vc = orc.e4m3_encode_array(kf), orc.e4m3_encode_array(vf)
    rng = np.random.default_rng(3)
    s = np.full((1,), 4.0, np.float32) if per_tensor else \
        rng.choice(np.array([1.0, 2.0, 4.0], np.float32), q.shape[:3])
    qs = (q / (s if per_tensor else s[..., None])).astype(np.float32)
    q8 = orc.e4m3_encode_array(qs)
    assert np.array_equal(orc.e4m3_decode_array(q8), qs)
    junk = np.full_like(q, 123.0)            # only the codes and scales are read
    out = orc.paged_decode(junk, kc, vc, ks, vs, table, ctx, window=20, sm_scale=np.log(2.0) / 2,
                           tile=32, q8=q8, q8_scale=s)
    ref = base2_decode(q, kf, vf, ks, vs, table, ctx, 20, Hkv)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


def test_mx_decode_e4m3_query_equals_fp8_decode(orc):
    """The given-e4m3-query path of the MXFP4 decode agrees bit for bit with
    the FP8 decode's on an MXFP4 cache's exact e4m3 twin (as above)."""
    B, MTP, Hq, Hkv, max_pages, D, PS = 2, 2, 8, 1, 4, 128, 64
    P = B * max_pages
    rng = np.random.default_rng(17)
    kc, ke, vc, ve, kf, vf = _mx_cache(9, P, Hkv, PS, D)
    k8, v8 = orc.e4m3_encode_array(kf), orc.e4m3_encode_array(vf)
    q8 = orc.e4m3_encode_array(rng.standard_normal((B, MTP, Hq, D)).astype(np.float32) * 30)
    qs = rng.uniform(0.01, 0.1, (B, MTP, Hq)).astype(np.float32)
    table = rng.permutation(P).astype(np.int32).reshape(B, max_pages)
    ctx = np.array([max_pages * PS - 9, 2 * PS + 1], np.int32)
    ones = np.ones((P, Hkv, PS), np.float32)
    q = np.zeros((B, MTP, Hq, D), np.float32)
    common = dict(window=0, sm_scale=D ** -0.5, q8=q8, q8_scale=qs)
    a = orc.paged_decode_mx(q, kc, ke, vc, ve, table, ctx, **common)
    b = orc.paged_decode(q, k8, v8, ones, ones, table, ctx, **common)
    assert np.array_equal(a, b) and np.abs(a).max() > 0

"""Pins of the oracle's paged decode: the page's window-tile counts, reduction
to exact attention of the last MTP rows (float mode), invariance to page
placement and to the split length, and the quantized mode against exact."""
import json
import os

import numpy as np
import pytest

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
    """Quantized decode on inputs where every rounding is exact: each Q row has
    a 448 (q_scale 1, codes = Q) in a channel where K is 0, scores use
    channels where q is in {0, +-2} and k in {0, +-1}, k_scale in {1, 2} and
    alpha = fp32(ln2 / 2 * log2 e) = 0.5, so x = q.k k_scale / 2 is an integer
    in [-4, 4]; V codes are e4m3 values and v_scale in {1/2, 1, 2}, so the
    folded P8 = e4m3(448 p v_scale / vmax) is exact.  The result must be
    base-2 attention of those integer scores over each query's window, with
    the per-token V scale applied: a wrong mask, fold, split or merge changes
    some weight by a power of two."""
    rng = np.random.default_rng(91)
    B, MTP, Hq, Hkv, D, PS, max_pages = 2, 4, 4, 2, 32, 16, 8
    P = B * max_pages
    G = Hq // Hkv
    ctx = np.array([100, 57], np.int32)
    q = np.zeros((B, MTP, Hq, D), np.float32)
    q[..., :2] = rng.choice([0.0, 2.0, -2.0], (B, MTP, Hq, 2))
    q[..., 2] = 448.0
    kf = rng.choice(np.array([0.0, 1.0, -1.0, 0.5, 3.0], np.float32), (P, Hkv, PS, D))
    kf[..., :2] = rng.choice([0.0, 1.0, -1.0], (P, Hkv, PS, 2))
    kf[..., 2] = 0.0
    vf = rng.choice(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -0.5], np.float32), (P, Hkv, PS, D))
    ks = rng.choice(np.array([1.0, 2.0], np.float32), (P, Hkv, PS))
    vs = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), (P, Hkv, PS))
    kc, vc = orc.e4m3_encode_array(kf), orc.e4m3_encode_array(vf)
    assert np.array_equal(orc.e4m3_decode_array(kc), kf) and np.array_equal(orc.e4m3_decode_array(vc), vf)
    table = rng.permutation(P).astype(np.int32).reshape(B, max_pages)
    out = orc.paged_decode(q, kc, vc, ks, vs, table, ctx, window=window, sm_scale=np.log(2.0) / 2,
                           tile=tile)
    ref = np.zeros_like(out, dtype=np.float64)
    for b in range(B):
        pages = table[b]
        kt = kf[pages].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)    # [Hkv, tokens, D]
        vt = vf[pages].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)
        kst = ks[pages].transpose(1, 0, 2).reshape(Hkv, -1)
        vst = vs[pages].transpose(1, 0, 2).reshape(Hkv, -1)
        for m in range(MTP):
            pos = ctx[b] - MTP + m
            lo = max(0, pos - window + 1) if window > 0 else 0
            for hq in range(Hq):
                hk = hq // G
                t = np.arange(lo, pos + 1)
                x = (kt[hk, t].astype(np.float64) @ q[b, m, hq].astype(np.float64)) * kst[hk, t] / 2
                assert np.array_equal(x, np.round(x)) and np.abs(x).max() <= 4
                w = 2.0 ** (x - x.max())
                ref[b, m, hq] = (w * vst[hk, t]) @ vt[hk, t].astype(np.float64) / w.sum()
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()

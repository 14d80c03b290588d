"""Paged FP8 decode parity on the GPU: the full batch-16 / MTP4 / GQA16 /
window-4096 workload against the oracle (every row), plus edge cases (no
window, ragged and unequal contexts, MTP1, GQA8 on two KV heads, page 64),
page-placement invariance and determinism."""
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


def _run(inp, dev, window, max_ctx, sm_scale):
    q = inp.q.to(dev)
    kc = inp.k_cache.to(dev).view(torch.float8_e4m3fn)
    vt = inp.v_cache.transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn)
    out = sage.sage_paged_decode(q, kc, vt, inp.k_scale.to(dev), inp.v_scale.to(dev),
                                 inp.page_table.to(dev), inp.ctx_lens.to(dev), max_ctx=max_ctx,
                                 window=window, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(orc, inp, window, sm_scale, quant=True):
    args = (inp.q.float().numpy(), inp.k_cache.numpy(), inp.v_cache.numpy(),
            inp.k_scale.numpy(), inp.v_scale.numpy(), inp.page_table.numpy(),
            inp.ctx_lens.numpy())
    if quant:
        return orc.paged_decode(*args, window=window, sm_scale=sm_scale)
    kf = orc.e4m3_decode_array(args[1]) * args[3][..., None]
    vf = orc.e4m3_decode_array(args[2]) * args[4][..., None]
    return orc.paged_decode(args[0], kf, vf, np.ones_like(args[3]), np.ones_like(args[4]),
                            args[5], args[6], window=window, sm_scale=sm_scale, quant=False)


def _check(g, o, e):
    assert cosine(g, o) >= 0.999
    assert np.abs(g - o).max() <= 1e-2
    assert cosine(g, e) >= 0.99


def test_paged_decode_full_workload(dev, orc):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w)
    say("paged decode full workload")
    g = _run(inp, dev, w.window, w.ctx, w.sm_scale)
    _check(g, _oracle(orc, inp, w.window, w.sm_scale), _oracle(orc, inp, w.window, w.sm_scale, False))
    # determinism
    assert np.array_equal(g, _run(inp, dev, w.window, w.ctx, w.sm_scale))


@pytest.mark.parametrize("window,ctx", [(0, 1000), (4096, 700), (300, 1537), (1, 512)])
def test_paged_decode_windows_and_contexts(dev, orc, window, ctx):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=3, ctx=ctx)
    inp.ctx_lens[1] = max(4, ctx - 257)          # unequal contexts in one batch
    inp.ctx_lens[2] = max(4, ctx // 3)
    say("paged decode", window, ctx)
    g = _run(inp, dev, window, ctx, w.sm_scale)
    _check(g, _oracle(orc, inp, window, w.sm_scale), _oracle(orc, inp, window, w.sm_scale, False))


@pytest.mark.parametrize("mtp,hq,hkv,page", [(1, 16, 1, 128), (4, 16, 2, 128), (2, 8, 1, 64),
                                             (4, 16, 1, 256), (1, 8, 1, 128),    # 8 rows: half a wave
                                             (4, 16, 1, 16), (2, 8, 2, 16)])     # 16-key pages
def test_paged_decode_shapes(dev, orc, mtp, hq, hkv, page):
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("v", 9, 4, mtp, hq, hkv, 128, page, 1200, 512)
    inp = wl.make_decode(w)
    say("paged decode shape", mtp, hq, hkv, page)
    g = _run(inp, dev, w.window, w.ctx, base.sm_scale)
    _check(g, _oracle(orc, inp, w.window, base.sm_scale), _oracle(orc, inp, w.window, base.sm_scale, False))


def test_page_placement_invariance(dev):
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=4, ctx=2000)
    say("page placement")
    a = _run(inp, dev, 1024, 2000, w.sm_scale)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(inp.k_cache.shape[0]))
    inv = torch.argsort(perm)
    moved = wl.DecodeInputs(inp.q, inp.k_cache[perm], inp.v_cache[perm], inp.k_scale[perm],
                            inp.v_scale[perm], inv[inp.page_table.long()].int(), inp.ctx_lens)
    b = _run(moved, dev, 1024, 2000, w.sm_scale)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("page,ctx,window", [(32, 3000, 1024), (32, 4500, 0), (16, 2500, 700)])
def test_paged_decode_long_page_tables(dev, orc, page, ctx, window):
    """More than 64 pages per sequence: the page ids are read after the
    context length instead of whole in lanes (94, 141 and 157 pages here)."""
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("v", 9, 3, 4, 16, 1, 128, page, ctx, window)
    inp = wl.make_decode(w)
    inp.ctx_lens[1] = ctx - 300
    say("paged decode long table", page, ctx, window)
    g = _run(inp, dev, w.window, w.ctx, base.sm_scale)
    _check(g, _oracle(orc, inp, w.window, base.sm_scale), _oracle(orc, inp, w.window, base.sm_scale, False))


def test_paged_decode_per_tensor_scales(dev, orc):
    """One fp32 scale per cache tensor (F32 [1]) instead of per token: the
    same cache values re-encoded with a single scale, against the oracle
    given that scale for every token."""
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=3, ctx=900)
    say("paged decode, per-tensor scales", "batch 3 ctx 900 window 256")
    kf = orc.e4m3_decode_array(inp.k_cache.numpy()) * inp.k_scale.numpy()[..., None]
    vf = orc.e4m3_decode_array(inp.v_cache.numpy()) * inp.v_scale.numpy()[..., None]
    sk, sv = np.float32(np.abs(kf).max() / 448.0), np.float32(np.abs(vf).max() / 448.0)
    k8 = torch.from_numpy(orc.e4m3_encode_array((kf / sk).astype(np.float32)))
    v8 = torch.from_numpy(orc.e4m3_encode_array((vf / sv).astype(np.float32)))
    q = inp.q.to(dev)
    out = sage.sage_paged_decode(q, k8.to(dev).view(torch.float8_e4m3fn),
                                 v8.transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn),
                                 torch.tensor([sk], device=dev), torch.tensor([sv], device=dev),
                                 inp.page_table.to(dev), inp.ctx_lens.to(dev), max_ctx=900, window=256,
                                 sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    full = lambda x: np.full(inp.k_scale.shape, x, np.float32)
    o = orc.paged_decode(inp.q.float().numpy(), k8.numpy(), v8.numpy(), full(sk), full(sv),
                         inp.page_table.numpy(), inp.ctx_lens.numpy(), window=256, sm_scale=w.sm_scale)
    e = orc.paged_decode(inp.q.float().numpy(), kf, vf, full(1.0), full(1.0), inp.page_table.numpy(),
                         inp.ctx_lens.numpy(), window=256, sm_scale=w.sm_scale, quant=False)
    _check(g, o, e)


@pytest.mark.parametrize("mtp,hq,hkv,page,window", [(4, 16, 1, 128, 512), (1, 8, 1, 16, 0), (2, 16, 2, 64, 300)])
def test_paged_decode_head_dim_64(dev, orc, mtp, hq, hkv, page, window):
    """D = 64 (e4m3 cache): the tiles hold 128-byte K rows and 128 V^T rows
    whose channels past 64 the copies fill with zeros."""
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("v", 9, 3, mtp, hq, hkv, 64, page, 1300, window)
    inp = wl.make_decode(w)
    inp.ctx_lens[1] = 700
    say("paged decode D 64", mtp, hq, hkv, page, window)
    sm = float(1.0 / np.sqrt(64))
    g = _run(inp, dev, w.window, w.ctx, sm)
    assert g.shape[-1] == 64
    _check(g, _oracle(orc, inp, w.window, sm), _oracle(orc, inp, w.window, sm, False))


@pytest.mark.parametrize("window,ctx,mtp", [(0, 12000, 4), (8192, 12000, 4), (0, 8500, 1)])
def test_paged_decode_more_than_32_splits(dev, orc, window, ctx, mtp):
    """More splits than one merge batch (32): no window over 12000 tokens (47
    splits), the aiter page's window 8192 with MTP 4 (34 splits), and 8500
    tokens without a window (34 splits, one past the batch); the merge then
    carries a running maximum across batches of splits."""
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("v", 9, 2, mtp, 16, 1, 128, 128, ctx, window)
    inp = wl.make_decode(w)
    inp.ctx_lens[1] = ctx - 1000
    assert sage.sage_decode_num_splits(window, mtp, ctx) > 32
    say("paged decode > 32 splits", window, ctx, mtp)
    g = _run(inp, dev, window, ctx, base.sm_scale)
    _check(g, _oracle(orc, inp, window, base.sm_scale), _oracle(orc, inp, window, base.sm_scale, False))


# Contexts 0 (no query position), 1 and 3 (below MTP 4: the first query
# tokens sit at negative positions and see no key), 4 and 5; 814 with window
# 300 starts the window at key 511, so its first split holds one key that only
# query token 0 sees and the other three rows are empty in that split.
DEGENERATE_CTX = [0, 1, 3, 4, 5, 814]


def test_paged_decode_degenerate_contexts(dev, orc):
    """Rows with no visible key anywhere are 0; rows with none in one split
    take nothing from it; the rest match the oracle."""
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=len(DEGENERATE_CTX), ctx=814)
    inp.ctx_lens[:] = torch.tensor(DEGENERATE_CTX, dtype=torch.int32)
    say("paged decode, degenerate contexts", DEGENERATE_CTX)
    g = _run(inp, dev, 300, 814, w.sm_scale)
    o = _oracle(orc, inp, 300, w.sm_scale)
    assert np.isfinite(g).all()
    assert not g[0].any() and not g[1, :3].any() and not g[2, :1].any()   # positions < 0
    assert not g[(o == 0).all(axis=-1)].any()                             # every empty row
    _check(g, o, _oracle(orc, inp, 300, w.sm_scale, False))


def test_paged_decode_context_above_max_ctx(dev, orc):
    """A context length above params.max_ctx (the page table still covering
    it) is treated as max_ctx: the output is finite and equals the oracle's at
    the clamped length."""
    base = wl.WORKLOADS["paged_decode"]
    w = wl.DecodeWorkload("v", 9, 3, 4, 16, 1, 128, 128, 2048, 0)
    inp = wl.make_decode(w)
    max_ctx = 1000
    inp.ctx_lens[:] = torch.tensor([1000, 1900, 600], dtype=torch.int32)
    say("paged decode, ctx above max_ctx", inp.ctx_lens.tolist(), max_ctx)
    g = _run(inp, dev, 0, max_ctx, base.sm_scale)
    assert np.isfinite(g).all()
    clamped = wl.DecodeInputs(inp.q, inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale, inp.page_table,
                              torch.clamp(inp.ctx_lens, max=max_ctx))
    _check(g, _oracle(orc, clamped, 0, base.sm_scale), _oracle(orc, clamped, 0, base.sm_scale, False))


def test_paged_decode_explicit_num_splits(dev):
    """num_splits given as the plan's count runs the same plan (bit-identical
    output); any other count is refused before anything is enqueued."""
    w = wl.WORKLOADS["paged_decode"]
    inp = wl.make_decode(w, batch=2, ctx=3000)
    say("paged decode explicit num_splits")
    args = (inp.q.to(dev), inp.k_cache.to(dev).view(torch.float8_e4m3fn),
            inp.v_cache.transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn),
            inp.k_scale.to(dev), inp.v_scale.to(dev), inp.page_table.to(dev), inp.ctx_lens.to(dev))
    kw = dict(max_ctx=3000, window=w.window, sm_scale=w.sm_scale)
    plan = sage.sage_decode_num_splits(w.window, w.mtp, 3000)
    a = sage.sage_paged_decode(*args, **kw)
    b = sage.sage_paged_decode(*args, num_splits=plan, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(sage.SageError) as err:
        sage.sage_paged_decode(*args, num_splits=plan + 1, **kw)
    assert err.value.status == sage.ERR_UNSUPPORTED

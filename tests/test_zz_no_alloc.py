"""sage_paged_decode_noalloc: the decode with its split partials in the
library's fixed per-device scratch instead of a workspace.  Its output must
equal sage_paged_decode's (the same kernels) on two calls in a row, the second
with a smaller problem, and a decode whose partials exceed the scratch is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from quantized_attention_block_amd import workloads as wl
from tests._util import cosine, require_gpu, say

pytestmark = pytest.mark.gpu


def _dev_inputs(inp, dev):
    return dict(q=inp.q.to(dev), k=inp.k_cache.to(dev).view(torch.float8_e4m3fn),
                v=inp.v_cache.transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn),
                ks=inp.k_scale.to(dev), vs=inp.v_scale.to(dev), pt=inp.page_table.to(dev),
                ctx=inp.ctx_lens.to(dev))


def _both(d, max_ctx, window, sm_scale):
    ref = sage.sage_paged_decode(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"],
                                 max_ctx=max_ctx, window=window, sm_scale=sm_scale)
    out = torch.full_like(d["q"], float("nan"))
    sage.sage_paged_decode_noalloc(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], out,
                                   max_ctx=max_ctx, window=window, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_decode_equals_workspace_decode(orc):
    dev = require_gpu()
    w = wl.WORKLOADS["paged_decode"]
    # 1: the full decode workload (16 sequences, 18 splits each)
    big = wl.make_decode(w)
    say("no-alloc decode: full workload")
    out, ref = _both(_dev_inputs(big, dev), w.ctx, w.window, w.sm_scale)
    assert torch.equal(out, ref)
    o = orc.paged_decode(big.q.float().numpy(), big.k_cache.numpy(), big.v_cache.numpy(),
                         big.k_scale.numpy(), big.v_scale.numpy(), big.page_table.numpy(),
                         big.ctx_lens.numpy(), window=w.window, sm_scale=w.sm_scale)
    g = out.float().cpu().numpy()
    assert cosine(g, o) >= 0.999 and np.abs(g - o).max() <= 1e-2
    # 2: right after, a smaller problem (3 sequences, unequal shorter
    # contexts, no window): the scratch still holds the first call's partials
    small = wl.make_decode(w, batch=3, ctx=1500)
    small.ctx_lens[1] = 700
    small.ctx_lens[2] = 5
    say("no-alloc decode: smaller problem after the full one")
    out2, ref2 = _both(_dev_inputs(small, dev), 1500, 0, w.sm_scale)
    assert torch.equal(out2, ref2)
    o2 = orc.paged_decode(small.q.float().numpy(), small.k_cache.numpy(), small.v_cache.numpy(),
                          small.k_scale.numpy(), small.v_scale.numpy(), small.page_table.numpy(),
                          small.ctx_lens.numpy(), window=0, sm_scale=w.sm_scale)
    g2 = out2.float().cpu().numpy()
    assert cosine(g2, o2) >= 0.999 and np.abs(g2 - o2).max() <= 1e-2


def test_noalloc_decode_refuses_more_than_the_scratch():
    dev = require_gpu()
    w = wl.WORKLOADS["paged_decode"]
    d = _dev_inputs(wl.make_decode(w, batch=2, ctx=512), dev)
    # 4096 sequences x 18 splits x 64 rows x 272 bytes > 32 MiB: refused from
    # the descriptors alone (the tensors below are never read)
    q = torch.empty((4096, 4, 16, 128), dtype=torch.bfloat16, device=dev)
    pt = torch.zeros((4096, 64), dtype=torch.int32, device=dev)
    ctx = torch.full((4096,), 8192, dtype=torch.int32, device=dev)
    assert sage.sage_paged_decode_workspace_size(q, d["k"], pt, max_ctx=8192, window=4096) > \
        sage.DECODE_SCRATCH_BYTES
    with pytest.raises(sage.SageError) as e:
        sage.sage_paged_decode_noalloc(q, d["k"], d["v"], d["ks"], d["vs"], pt, ctx, torch.empty_like(q),
                                       max_ctx=8192, window=4096, sm_scale=w.sm_scale)
    assert e.value.status == sage.ERR_WORKSPACE


def test_decode_replayed_from_a_hip_graph():
    """Both decode entry points captured into a HIP graph (the no-allocation
    one is meant for callers under capture): every replay, with eager work
    and synchronizations between replays, equals the eager decode bit for
    bit."""
    dev = require_gpu()
    w = wl.WORKLOADS["paged_decode"]
    d = _dev_inputs(wl.make_decode(w), dev)
    kw = dict(max_ctx=w.ctx, window=w.window, sm_scale=w.sm_scale)
    say("decode graph: eager reference")
    ref = sage.sage_paged_decode(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], **kw)
    torch.cuda.synchronize()
    ws = torch.empty(sage.sage_paged_decode_workspace_size(d["q"], d["k"], d["pt"], max_ctx=w.ctx,
                                                           window=w.window) + 256,
                     dtype=torch.uint8, device=dev)
    out_ws, out_na = torch.empty_like(ref), torch.empty_like(ref)
    # one eager call of each form before capture (library set-up, such as the
    # scratch address lookup, happens outside the graph)
    sage.sage_paged_decode(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], out=out_ws,
                           workspace=ws, **kw)
    sage.sage_paged_decode_noalloc(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], out_na, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("decode graph: capture")
    with torch.cuda.graph(graph):
        sage.sage_paged_decode(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], out=out_ws,
                               workspace=ws, **kw)
        sage.sage_paged_decode_noalloc(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["pt"], d["ctx"], out_na,
                                       **kw)
    for i in range(3):
        out_ws.fill_(float("nan"))
        out_na.fill_(float("nan"))
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        say(f"decode graph: replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_ws, ref), i
        assert torch.equal(out_na, ref), i

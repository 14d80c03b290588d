"""Benchmark of the quantized-attention hot path on one MI355X.

One step = quantize Q/K (K channel mean + INT8 blocks) + quantize V (e4m3,
per-channel scale, transposed) + fused quantized attention, on the
LLM-prefill workload (B=2, H=32, Lq=Lk=4096, D=128, bf16, causal), inputs
resident in HBM, launched eagerly; the same step replayed from a HIP graph
(each replay first checked bit-equal to an eager step) is reported beside it.
Prints one JSON line:

  value        = 4 B H Lq Lk D / t_step  (the metric's own formula, TOPS)
  roofline     = the attention kernel alone: algorithmic ops (unmasked causal
                 pairs, 4 D per pair) / its average launch time, measured with
                 HIP events on the stream it runs on, against the INT8/FP8 MFMA
                 peak (5.0 POPS dense)
  cpu_baseline = the CPU oracle (quantize + step-by-step emulation) on a
                 bounded sample of query rows of the same workload
  extra        = the paged FP8 decode workload (HBM GB/s) and, with --all,
                 the video-DiT INT8 and MXFP4 workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_MFMA_TOPS = 5000.0      # INT8 and FP8 dense MFMA, MI355X
PEAK_MXFP4_MIX_TOPS = 4.0 / (2.0 / 10100.0 + 2.0 / 5000.0)   # half FP4 QK, half FP8 PV
PEAK_HBM_GBS = 8000.0


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_attention_block_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, src_names):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("src_hash") != _src_hash(*src_names):
        return None
    return t.get("bytes_per_launch")


def _events_time(fn, reps, stream):
    """Average duration of one call of fn (one kernel launch), each call
    bracketed by its own pair of HIP events on `stream` (gaps between
    launches are not counted)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    ev[-1][1].synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps * 1e-3   # seconds per call


def prefill_bench(wname, steps, warmup, dev, mode=None, fused_q=True):
    """fused_q (INT8): Q is quantized in the attention kernel's prologue
    (sage_quantize_qk(None, k) + sage_attn_fwd(q=...)), which gives the
    unfused step's output bit for bit; the unfused step is timed beside it."""
    from quantized_attention_block_amd import sage
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS[wname]
    mode = (sage.QK_MXFP4 if w.qk_mode == "mxfp4" else sage.QK_INT8) if mode is None else mode
    fused_q = fused_q and mode == sage.QK_INT8
    inp = wl.make_prefill(w, device=dev)
    had = sage.Hadamard(dev.index or 0) if mode == sage.QK_MXFP4 else None
    stream = torch.cuda.current_stream(dev)
    # preallocated outputs and workspaces: the timed step only launches kernels
    qk_in = None if fused_q else inp.q
    qk = sage.sage_quantize_qk(qk_in, inp.k, mode=mode, hadamard=had, want_mean=False)
    v_q, v_s = sage.sage_quantize_v(inp.v)
    out = torch.empty((w.B, w.Lq, w.H, w.D), dtype=torch.bfloat16, device=dev)
    ws_qk = torch.empty(max(16, sage.sage_quantize_qk_workspace_size(inp.q, inp.k, mode=mode)),
                        dtype=torch.uint8, device=dev)
    ws_v = torch.empty(sage.sage_quantize_v_workspace_size(inp.v), dtype=torch.uint8, device=dev)

    def quant():
        sage.sage_quantize_qk(qk_in, inp.k, mode=mode, hadamard=had, workspace=ws_qk, into=qk)
        sage.sage_quantize_v(inp.v, workspace=ws_v, into=(v_q, v_s))

    def attn():
        sage.sage_attn_fwd(qk, v_q, v_s, causal=w.causal, sm_scale=w.sm_scale, out=out,
                           q=inp.q if fused_q else None)

    def step():
        quant()
        attn()

    # untimed pre-warm (~0.2 s of steps) so clocks have settled before the
    # W warm-up steps and the K timed ones
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    # The same step captured once in a HIP graph and replayed (context): each
    # replay is first checked bit for bit against an eager step, with eager
    # work in between.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError(f"{wname}: graph replay differs from the eager step")
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    t_step_graph = (time.perf_counter() - t0) / steps
    t_step_unfused = None
    if fused_q:   # the unfused step (Q's INT8 copy written and read), same inputs
        qk_u = sage.sage_quantize_qk(inp.q, inp.k, want_mean=False)
        out_u = torch.empty_like(out)

        def step_u():
            sage.sage_quantize_qk(inp.q, inp.k, workspace=ws_qk, into=qk_u)
            sage.sage_quantize_v(inp.v, workspace=ws_v, into=(v_q, v_s))
            sage.sage_attn_fwd(qk_u, v_q, v_s, causal=w.causal, sm_scale=w.sm_scale, out=out_u)
        for _ in range(warmup + 1):
            step_u()
        torch.cuda.synchronize()
        if not torch.equal(out_u, out):
            raise RuntimeError(f"{wname}: fused Q quantization differs from the unfused step")
        t0 = time.perf_counter()
        for _ in range(steps):
            step_u()
        torch.cuda.synchronize()
        t_step_unfused = (time.perf_counter() - t0) / steps
    # attention kernel alone, HIP events on its stream
    attn()
    t_attn = min(_events_time(attn, max(steps, 10), stream) for _ in range(3))
    L = w.Lq
    pairs = w.B * w.H * (L * (L + 1) // 2 if w.causal else w.Lq * w.Lk)
    ops_alg = 4.0 * pairs * w.D
    literal = 4.0 * w.B * w.H * w.Lq * w.Lk * w.D
    peak = PEAK_MXFP4_MIX_TOPS if mode == sage.QK_MXFP4 else PEAK_MFMA_TOPS
    achieved = ops_alg / t_attn / 1e12
    src = ["attn_fwd.hip", "sage_device.hpp"]
    return dict(w=w, t_step=t_step, t_step_graph=t_step_graph, t_attn=t_attn, fused_q=fused_q,
                t_step_unfused=t_step_unfused,
                value=literal / t_step / 1e12,
                attn_literal_tops=literal / t_attn / 1e12,
                roofline={"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                          "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                          "traffic": _traffic(f"attn_fwd_{wname}", src)})


def decode_bench(steps, warmup, dev, pools=32, mx=False):
    """mx: the same decode over an MXFP4 cache (E2M1 + E8M0, the next step the
    aiter page names), timed the same way."""
    from quantized_attention_block_amd import sage
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS["paged_decode"]
    # rotate among independent KV pools (> 256 MB in total) so the timed reads
    # come from HBM, not the MALL
    sets = []
    for i in range(pools):
        if mx:
            inp = wl.make_decode_mx(w, pool_seed=i)
            k4, v4 = inp.packed()
            sets.append(dict(
                q=inp.q.to(dev), k=k4.to(dev).view(torch.float4_e2m1fn_x2),
                v=v4.to(dev).view(torch.float4_e2m1fn_x2), ks=inp.k_e8.to(dev).view(torch.float8_e8m0fnu),
                vs=inp.v_e8.to(dev).view(torch.float8_e8m0fnu), pt=inp.page_table.to(dev),
                ctx=inp.ctx_lens.to(dev)))
            continue
        inp = wl.make_decode(w, pool_seed=i)
        sets.append(dict(
            q=inp.q.to(dev), k=inp.k_cache.to(dev).view(torch.float8_e4m3fn),
            v=inp.v_cache.transpose(2, 3).contiguous().to(dev).view(torch.float8_e4m3fn),
            ks=inp.k_scale.to(dev), vs=inp.v_scale.to(dev), pt=inp.page_table.to(dev),
            ctx=inp.ctx_lens.to(dev)))
    s0 = sets[0]
    ws = torch.empty(sage.sage_paged_decode_workspace_size(s0["q"], s0["k"], s0["pt"], max_ctx=w.ctx,
                                                           window=w.window) + 256,
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(s0["q"])
    idx = [0]

    def call():
        s = sets[idx[0] % pools]
        idx[0] += 1
        sage.sage_paged_decode(s["q"], s["k"], s["v"], s["ks"], s["vs"], s["pt"], s["ctx"],
                               max_ctx=w.ctx, window=w.window, sm_scale=w.sm_scale, out=out,
                               workspace=ws)

    for _ in range(warmup * 10):
        call()
    torch.cuda.synchronize()
    # one decode (decode + merge kernels) per pool, captured once and replayed:
    # the device time per call without Python launch overhead
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(pools):
            call()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t = min(_events_time(graph.replay, max(10, steps), stream) for _ in range(5)) / pools
    t_eager = _events_time(call, 200, stream)
    keys = min(w.ctx, w.window + w.mtp - 1)
    # bytes per key and KV head: K and V codes plus their scales (e4m3: D + D
    # bytes and two fp32; MXFP4: D/2 + D/2 bytes and D/32 + D/32 E8M0 bytes)
    per_key = (w.D + w.D // 16) if mx else (2 * w.D + 8)
    alg_bytes = w.batch * w.hkv * keys * per_key + 2 * (w.batch * w.mtp * w.hq * w.D * 2)
    gbs = alg_bytes / t / 1e9
    fmt = "MXFP4 (E2M1 + E8M0)" if mx else "FP8"
    return {"metric": f"paged {fmt} decode HBM GB/s (decode + merge)", "value": round(gbs, 1),
            "unit": "GB/s", "us_per_call": round(t * 1e6, 3),
            "us_per_call_eager_launch": round(t_eager * 1e6, 2), "algorithmic_bytes": alg_bytes,
            "workload": "batch16 MTP4 GQA16 D128 page128 ctx8192 window4096 " +
                        ("mxfp4 E8M0 per 32 (K: channels, V: keys)" if mx else "fp8-e4m3 per-token"),
            "kv_pools_rotated": pools,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic("paged_decode_mxfp4" if mx else "paged_decode",
                                             ["decode.hip", "sage_device.hpp"])}}


def cpu_baseline(wname, target_s=15.0):
    """The oracle as it stands, on a bounded sample: quantize one (b, h) head
    of the workload and emulate a seeded sample of its query rows."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from quantized_attention_block_amd import workloads as wl
    w = wl.WORKLOADS[wname]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    inp = wl.make_prefill(w, B=1, H=1)
    canon = lambda t: t.float().permute(0, 2, 1, 3).contiguous().numpy()
    q, k, v = canon(inp.q), canon(inp.k), canon(inp.v)
    rng = np.random.default_rng(11)

    def run(nrows):
        ri = np.sort(rng.integers(0, w.Lq, nrows))
        rows = np.stack([np.zeros_like(ri), np.zeros_like(ri), ri], 1)
        t0 = time.perf_counter()
        oracle.prefill_int8_pipeline(q, k, v, causal=w.causal, sm_scale=w.sm_scale, BN=64,
                                     rows=rows, nthreads=cores)
        return time.perf_counter() - t0

    # the per-run cost is one head's quantization plus a per-row emulation
    # cost: two probes give both, then the sample is sized to ~target_s
    t1, t2 = run(64), run(512)
    per_row = max((t2 - t1) / 448.0, 1e-7)
    nrows = int(max(512, min(2_000_000, (target_s - t1) / per_row)))
    t = run(nrows)
    literal = 4.0 * nrows * w.Lk * w.D      # same formula per query row as the GPU value
    return {"value": round(literal / t / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "seconds": round(t, 2),
            "sample": f"{nrows} seeded query rows of one (b,h) head of {w.name} "
                      f"(Lk={w.Lk}, D={w.D}, causal={w.causal}): K mean + INT8/e4m3 quantization "
                      f"of that head + step-by-step emulation of those rows, C++ threads={cores}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llm_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time the video-DiT workloads")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU split is described, not built)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    r = prefill_bench(args.workload, args.steps, args.warmup, dev)
    w = r["w"]
    extra = {"attn_kernel_us": round(r["t_attn"] * 1e6, 1),
             "attn_kernel_tops_literal": round(r["attn_literal_tops"], 1),
             "quantize_us": round((r["t_step"] - r["t_attn"]) * 1e6, 1),
             "ms_per_step_hip_graph": round(r["t_step_graph"] * 1e3, 4)}
    if r["t_step_unfused"] is not None:
        extra["ms_per_step_unfused_q"] = round(r["t_step_unfused"] * 1e3, 4)
        extra["tops_unfused_q"] = round(r["value"] * r["t_step"] / r["t_step_unfused"], 2)
    if not args.no_decode:
        extra["paged_decode"] = decode_bench(args.steps, args.warmup, dev)
        extra["paged_decode_mxfp4"] = decode_bench(args.steps, args.warmup, dev, mx=True)
    if args.all:
        for wn in ("video_dit", "video_dit_mxfp4"):
            rr = prefill_bench(wn, max(3, args.steps // 4), 2, dev)
            extra[wn] = {"value": round(rr["value"], 1), "unit": "TOPS",
                         "ms_per_step": round(rr["t_step"] * 1e3, 3),
                         "attn_kernel_ms": round(rr["t_attn"] * 1e3, 3), "roofline": rr["roofline"]}
    line = {
        "metric": "quantized attn fwd TOPS (4BHLqLkD/t) + % gfx950 MFMA peak; decode HBM GB/s",
        "value": round(r["value"], 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["t_step"] * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8 QK / fp8-e4m3 PV, fp32 softmax, bf16 in/out", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len_q": w.Lq,
                   "seq_len_k": w.Lk, "head_dim": w.D, "causal": w.causal,
                   "q_block": w.q_block, "k_block": w.k_block,
                   "step": ("quantize_qk (K) + quantize_v + attn_fwd (Q quantized in its prologue)"
                            if r["fused_q"] else "quantize_qk + quantize_v + attn_fwd")},
        "roofline": r["roofline"],
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Summaries of rocprofv3 runs for the profiles/ folder.

stats   <run_results.db> <out.txt> <command...>
    Per-kernel call count, average and total duration from a
    `rocprofv3 --kernel-trace --stats` run (table top_kernels).
traffic <out.json> <copy_bytes> <copy_rd_dir>,<copy_wr_dir> <label>=<rd_dir>,<wr_dir> ...
    HBM bytes per launch of the library's kernels from the L2-to-memory
    request counters, read directly: bytes read = 32 TCC_EA0_RDREQ_32B +
    64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B, bytes written =
    64 TCC_EA0_WRREQ_64B + 32 (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B) (the
    first pass per label collects the four read counters, the second the
    two write counters; rocprofv3 --pmc -f csv).  Entries of an existing
    <out.json> whose label is not given again are kept, so one workload can
    be re-collected alone after its kernel changed.  No scale factor is
    applied: the copy run (copy_bytes read and written by one plain device
    copy, see `copy`) is reported beside them as a check of the formulas.
    Entries are keyed "<kernel>@<label>" and carry the hash of the kernel's
    source files, so a reader can tell when they no longer describe the code.
copy <bytes>
    Three device-to-device copies of <bytes> (the check run of `traffic`).
counters <kernel fragment> <MFMA instructions per wave-step> <out.txt> <label=pass_dir[,pass_dir...]>...
    SQ / GRBM counters of one kernel (rocprofv3 --pmc passes over the same
    command, one directory per pass) per workload label, as per-wave-step
    instruction counts and pipe utilisations.  MI355X: 8 XCDs, 1024 SIMDs.
"""
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_attention_block_amd", "csrc")

# library kernel (base name) -> the source files it is built from
KERNEL_SOURCES = {
    "k_attn_fwd": ["attn_fwd.hip", "sage_device.hpp"],
    "k_paged_decode": ["decode.hip", "sage_device.hpp"],
    "k_decode_merge": ["decode.hip", "sage_device.hpp"],
    "k_quant_qk_fused": ["quantize.hip", "sage_device.hpp"],
    "k_quant_v_fused": ["quantize.hip", "sage_device.hpp"],
    "k_quant_mxfp4": ["quantize.hip", "sage_device.hpp"],
    "k_quant_int8": ["quantize.hip", "sage_device.hpp"],
    "k_mean_partial": ["quantize.hip", "sage_device.hpp"],
    "k_v_amax": ["quantize.hip", "sage_device.hpp"],
    "k_v_quant": ["quantize.hip", "sage_device.hpp"],
}
# how the runs behind a traffic summary are taken (from /tmp, TMPDIR=/tmp)
COLLECTION = {
    "read_pass": "rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum "
                 "TCC_EA0_RDREQ_128B_sum -d <dir> -o run --output-format csv -- python bench.py --only <label> "
                 "--steps 2 --warmup 1",
    "write_pass": "rocprofv3 --pmc TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum -d <dir> -o run --output-format csv "
                  "-- python bench.py --only <label> --steps 2 --warmup 1",
    "copy_passes": "the same two passes over: python quantized_attention_block_amd/rocprof_summary.py copy 268435456",
    "summary": "python quantized_attention_block_amd/rocprof_summary.py traffic profiles/traffic.json 268435456 "
               "<copy_rd>,<copy_wr> <label>=<rd>,<wr> ...",
}
READ_COUNTERS = {"TCC_EA0_RDREQ_32B_sum": 32, "TCC_EA0_RDREQ_64B_sum": 64, "TCC_EA0_RDREQ_128B_sum": 128}


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats(db, out, command):
    """One line per (kernel, launch grid): launches of one kernel on different
    workloads differ in grid size, so their durations are kept apart."""
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, grid_x, grid_y, grid_z, workgroup_x * workgroup_y * workgroup_z, "
        "count(*), avg(duration), min(duration), sum(duration), max(vgpr_count), "
        "max(accum_vgpr_count), max(sgpr_count), max(lds_size), max(scratch_size) "
        "from kernels group by name, grid_x, grid_y, grid_z order by sum(duration) desc").fetchall()
    total = sum(r[8] for r in rows) or 1
    with open(out, "w") as f:
        f.write("# rocprofv3 --kernel-trace --stats summary, one line per kernel and launch grid\n")
        f.write(f"# command: {' '.join(command)}\n")
        f.write("# durations in microseconds; grid in work-items (x*y*z), block = work-items per workgroup;\n")
        f.write("# vgpr/agpr/sgpr per lane or wave as allocated, lds and scratch in bytes per workgroup / lane\n")
        f.write(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'total_us':>11} {'pct':>6} {'grid':>9} {'block':>5} "
                f"{'vgpr':>4} {'agpr':>4} {'sgpr':>4} {'lds':>6} {'scr':>4}  kernel\n")
        for (name, gx, gy, gz, wg, n, avg, mn, tot, vg, ag, sg, lds, scr) in rows:
            f.write(f"{n:>6} {avg / 1e3:>10.2f} {mn / 1e3:>10.2f} {tot / 1e3:>11.1f} {100.0 * tot / total:>6.2f} "
                    f"{gx * gy * gz:>9} {wg:>5} {vg:>4} {ag:>4} {sg:>4} {lds:>6} {scr:>4}  {name[:120]}\n")


def _pmc_rows(d):
    """(kernel name, counter) -> per-dispatch values of every counter CSV under d."""
    vals = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def _bytes(rd, wr, name):
    """Average bytes read and written per dispatch of kernel `name` (None if absent)."""
    reads = [rd.get((name, c)) for c in READ_COUNTERS]
    wq, w64 = wr.get((name, "TCC_EA0_WRREQ_sum")), wr.get((name, "TCC_EA0_WRREQ_64B_sum"))
    if any(v is None for v in reads) or wq is None or w64 is None:
        return None
    avg = lambda v: sum(v) / len(v)
    rbytes = sum(avg(v) * size for v, size in zip(reads, READ_COUNTERS.values()))
    wbytes = 64.0 * avg(w64) + 32.0 * (avg(wq) - avg(w64))
    total_req = rd.get((name, "TCC_EA0_RDREQ_sum"))
    sized_req = sum(avg(v) for v in reads)
    return {"read_bytes": round(rbytes), "write_bytes": round(wbytes),
            "bytes_per_launch": round(rbytes + wbytes), "dispatches": [len(reads[0]), len(wq)],
            # requests of a size none of the three counters sees (0 when they partition the total)
            "unsized_read_requests": round(avg(total_req) - sized_req) if total_req else None}


def traffic(out, copy_bytes, copy_dirs, groups):
    crd, cwr = (_pmc_rows(d) for d in copy_dirs.split(","))
    names = {k[0] for k in crd}
    copy = max((_bytes(crd, cwr, n) for n in names), key=lambda b: b["read_bytes"] if b else -1)
    res = {"method": "direct TCC_EA0 request counters, no scale factor (see rocprof_summary.py)",
           "collection": COLLECTION,
           "copy_check": {"bytes_copied": copy_bytes, "read_bytes": copy["read_bytes"],
                          "write_bytes": copy["write_bytes"],
                          "read_ratio": round(copy["read_bytes"] / copy_bytes, 4),
                          "write_ratio": round(copy["write_bytes"] / copy_bytes, 4)},
           "kernels": {}}
    labels = {g.split("=", 1)[0] for g in groups}
    if os.path.exists(out):
        with open(out) as f:
            prev = json.load(f).get("kernels", {})
        res["kernels"].update({k: v for k, v in prev.items() if k.split("@", 1)[1] not in labels})
    for g in groups:
        label, dirs = g.split("=", 1)
        rd, wr = (_pmc_rows(d) for d in dirs.split(","))
        for name in sorted({k[0] for k in rd}):
            base = next((b for b in KERNEL_SOURCES if b + "<" in name or b + "(" in name), None)
            if base is None:
                continue
            b = _bytes(rd, wr, name)
            if b is None:
                continue
            key = f"{base}@{label}"
            if key in res["kernels"]:   # several instances of one kernel: keep the busiest
                if res["kernels"][key]["bytes_per_launch"] >= b["bytes_per_launch"]:
                    continue
            res["kernels"][key] = {"kernel": name[:160], **b, "src_hash": src_hash(KERNEL_SOURCES[base])}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


def copy(nbytes):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {nbytes} bytes 3 times", flush=True)


# the passes behind a `counters` summary (one rocprofv3 run each, from /tmp)
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
    "SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU_TRANS_F32 "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_ANY SQ_LDS_IDX_ACTIVE",
    "SQ_INSTS_SALU SQ_INSTS_SMEM SQ_INST_CYCLES_VMEM SQ_WAIT_ANY SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA "
    "SQ_INSTS_BRANCH SQ_ACTIVE_INST_FLAT",
]


def counters(frag, mfma_per_step, out, groups):
    n_xcd, n_simd = 8, 1024
    lines = ["# rocprofv3 --pmc counter summary of kernels matching '%s' (average per dispatch)" % frag,
             "# per wave-step = per wave and per KV tile (SQ_INSTS_MFMA / %d)" % mfma_per_step,
             "# SQ_*_CYCLES and SQ_WAVE_CYCLES count quad-cycles; GRBM_GUI_ACTIVE is summed over XCDs",
             "# passes (from /tmp, TMPDIR=/tmp; <label> = the workload):"]
    lines += ["#   rocprofv3 --pmc %s -d <dir>/p%d -o run --output-format csv -- python bench.py --only <label> "
              "--steps 2 --warmup 1" % (c, i + 1) for i, c in enumerate(COUNTER_PASSES)]
    lines.append("# then: python quantized_attention_block_amd/rocprof_summary.py counters '%s' %d <out> "
                 "<label>=<dir>/p1,<dir>/p2,<dir>/p3 ..." % (frag, mfma_per_step))
    for g in groups:
        label, dirs = g.split("=", 1)
        m = {}
        for d in dirs.split(","):
            for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
                for r in csv.DictReader(open(fn)):
                    if frag in r["Kernel_Name"]:
                        m.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        m = {k: sum(v) / len(v) for k, v in m.items()}
        steps = m["SQ_INSTS_MFMA"] / mfma_per_step
        gui = m["GRBM_GUI_ACTIVE"] / n_xcd
        lines.append("")
        lines.append("[%s] wave-steps per dispatch %.0f, GPU cycles %.0f" % (label, steps, gui))
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
                  "SQ_INSTS_LDS", "SQ_INSTS_SMEM", "SQ_INSTS_BRANCH"):
            if c in m:
                lines.append("  %-26s %8.1f per wave-step" % (c, m[c] / steps))
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * gui)
        lines.append("  MFMA busy                  %8.3f of SIMD cycles" % busy)
        lines.append("  MFMA co-executing VALU     %8.3f of MFMA-busy cycles"
                     % (m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"]))
        lines.append("  SIMD cycles per wave-step  %8.0f" % (n_simd * gui / steps))
        lines.append("  resident waves per SIMD    %8.2f" % (4 * m["SQ_WAVE_CYCLES"] / (n_simd * gui)))
        lines.append("  waiting for an instruction %8.3f of wave cycles (SQ_WAIT_INST_ANY)"
                     % (m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]))
        lines.append("  LDS bank conflicts         %8.0f cycles per dispatch" % m.get("SQ_LDS_BANK_CONFLICT", 0.0))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif sys.argv[1] == "counters":
        counters(sys.argv[2], int(sys.argv[3]), sys.argv[4], sys.argv[5:])
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], int(sys.argv[3]), sys.argv[4], sys.argv[5:])
    elif sys.argv[1] == "copy":
        copy(int(sys.argv[2]))
    else:
        raise SystemExit(__doc__)

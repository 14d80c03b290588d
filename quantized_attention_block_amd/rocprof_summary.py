"""Summaries of rocprofv3 runs for the profiles/ folder.

stats   <run_results.db> <out.txt> <command...>
    Per-kernel call count, average and total duration from a
    `rocprofv3 --kernel-trace --stats` run (table top_kernels).
traffic <fetch_dir> <write_dir> <cal_fetch_dir> <cal_write_dir> <copy_bytes> <out.json>
    Per-launch FETCH_SIZE / WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc
    -f csv) of the library's kernels, scaled by the copy calibration
    (known bytes / counter reading of a plain copy of copy_bytes), keyed by
    kernel and workload, with the hash of the kernel's source files so a
    reader can tell when the numbers no longer describe the code.
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

# kernel-name fragment -> (traffic key, source files it is built from)
KERNELS = {
    "k_attn_fwd<128, false, true>": ("attn_fwd_llm_prefill", ["attn_fwd.hip", "sage_device.hpp"]),
    "k_paged_decode<128, false>": ("paged_decode", ["decode.hip", "sage_device.hpp"]),
    "k_paged_decode<128, true>": ("paged_decode_mxfp4", ["decode.hip", "sage_device.hpp"]),
    "k_decode_merge": ("decode_merge", ["decode.hip", "sage_device.hpp"]),
    "k_quant_qk_fused<128, true>": ("quant_qk_llm_prefill", ["quantize.hip", "sage_device.hpp"]),
    "k_quant_v_fused<128, true>": ("quant_v_llm_prefill", ["quantize.hip", "sage_device.hpp"]),
}


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


def _pmc(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    vals = {}
    for fn in files:
        for r in csv.DictReader(open(fn)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _avg_for(vals, frag):
    got = [v for k, vs in vals.items() if frag in k for v in vs]
    return (sum(got) / len(got), len(got)) if got else (None, 0)


def traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, copy_bytes, out):
    cf, cw = _pmc(cal_fetch_dir, "FETCH_SIZE"), _pmc(cal_write_dir, "WRITE_SIZE")
    # the copy kernel is the only (or the largest) dispatch of the calibration run
    cal_fetch = max(sum(v) / len(v) for v in cf.values()) * 1024.0
    cal_write = max(sum(v) / len(v) for v in cw.values()) * 1024.0
    f_scale, w_scale = copy_bytes / cal_fetch, copy_bytes / cal_write
    fv, wv = _pmc(fetch_dir, "FETCH_SIZE"), _pmc(write_dir, "WRITE_SIZE")
    res = {"_calibration": {"copy_bytes": copy_bytes, "fetch_counter_bytes": cal_fetch,
                            "write_counter_bytes": cal_write, "fetch_scale": f_scale,
                            "write_scale": w_scale}}
    for frag, (key, srcs) in KERNELS.items():
        fa, nf = _avg_for(fv, frag)
        wa, nw = _avg_for(wv, frag)
        if fa is None or wa is None:
            continue
        fb, wb = fa * 1024.0 * f_scale, wa * 1024.0 * w_scale
        res[key] = {"kernel": frag, "dispatches": [nf, nw], "fetch_bytes": round(fb),
                    "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
                    "src_hash": src_hash(srcs)}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


def counters(frag, mfma_per_step, out, groups):
    n_xcd, n_simd = 8, 1024
    lines = ["# rocprofv3 --pmc counter summary of kernels matching '%s' (average per dispatch)" % frag,
             "# per wave-step = per wave and per KV tile (SQ_INSTS_MFMA / %d)" % mfma_per_step,
             "# SQ_*_CYCLES and SQ_WAVE_CYCLES count quad-cycles; GRBM_GUI_ACTIVE is summed over XCDs"]
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
        traffic(*sys.argv[2:6], int(sys.argv[6]), sys.argv[7])
    else:
        raise SystemExit(__doc__)

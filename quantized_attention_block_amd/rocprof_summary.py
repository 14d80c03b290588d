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
    "k_attn_fwd<128, false>": ("attn_fwd_llm_prefill", ["attn_fwd.hip", "sage_device.hpp"]),
    "k_paged_decode<128>": ("paged_decode", ["decode.hip", "sage_device.hpp"]),
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
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels order by total_duration desc").fetchall()
    with open(out, "w") as f:
        f.write("# rocprofv3 --kernel-trace --stats summary\n")
        f.write(f"# command: {' '.join(command)}\n")
        f.write("# durations in microseconds\n")
        f.write(f"{'calls':>7} {'avg_us':>10} {'total_us':>12} {'pct':>6}  kernel\n")
        for name, calls, total, avg, pct in rows:
            f.write(f"{calls:>7} {avg:>10.2f} {total:>12.1f} {pct:>6.2f}  {name[:150]}\n")


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


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4:])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:6], int(sys.argv[6]), sys.argv[7])
    else:
        raise SystemExit(__doc__)

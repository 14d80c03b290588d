"""Plain device-to-device copy of a known size, run under rocprofv3 --pmc to
calibrate the FETCH_SIZE / WRITE_SIZE counters: the counters of this copy are
compared with the bytes it must move, and that ratio scales the counters of
the library's kernels into HBM bytes.

    python -m quantized_attention_block_amd.hbm_calibration [--mib 256] [--reps 4]
"""
import argparse
import json

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=256)
    ap.add_argument("--reps", type=int, default=4)
    args = ap.parse_args()
    n = args.mib << 20
    dev = torch.device("cuda", 0)
    # two source buffers, so consecutive copies do not read what the previous
    # one left in the caches (each 256 MiB buffer alone fills the MALL)
    src = [torch.full((n,), i + 1, dtype=torch.uint8, device=dev) for i in range(2)]
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for i in range(args.reps):
        dst.copy_(src[i % 2])
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": args.reps}))


if __name__ == "__main__":
    main()

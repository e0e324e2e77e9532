"""A plain device-to-device copy of a known size, repeated: the reference the
HBM traffic counters (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) are scaled by.
Each copy reads and writes exactly --mib MiB.

    python -m nvfp4_block_scaled_route_amd.copy_calibration [--mib 256] [--reps 5]
"""
from __future__ import annotations

import argparse

import torch


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=256)
    ap.add_argument("--reps", type=int, default=5)
    args = ap.parse_args()
    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}", flush=True)


if __name__ == "__main__":
    main()

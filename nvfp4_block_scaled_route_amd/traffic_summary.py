"""HBM traffic of the expert step from rocprofv3 PMC runs.

Reads four counter collections (rocprofv3 --pmc ... --output-format csv), each
counter in a run of its own:

    <dir>/FETCH_SIZE, <dir>/WRITE_SIZE              python bench.py --workload W ...
    <copy dir>/copy_FETCH_SIZE, <copy dir>/copy_WRITE_SIZE
                                                    copy_calibration.py --mib M --reps R

scales the expert kernels' per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) by what
the same counters read for a device copy of known size (times the launches of
one layer step: the expert-TP slices each launch the step), and writes
profiles/experts_<W>_traffic.json (with the SHA-256 of the kernel sources, so
that bench.py reports the figure only while they are unchanged) and prints a
markdown table.

    python -m nvfp4_block_scaled_route_amd.traffic_summary --dir <rocprofv3 output dir> \\
        --workload prefill_t4096 --copy-mib 256 [--copy-dir <dir>] [--launches-per-step 8]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["nvfp4_block_scaled_route_amd/csrc/experts.hip",
           "nvfp4_block_scaled_route_amd/csrc/experts_tiled.hip",
           "nvfp4_block_scaled_route_amd/csrc/experts.hpp",
           "nvfp4_block_scaled_route_amd/csrc/finalize.hpp",
           "nvfp4_block_scaled_route_amd/csrc/common.hpp"]
# the kernels moe_experts_fwd launches (the other expert variants the bench
# times beside it, W4A16 and BF16, are not part of the step)
EXPERT_KERNELS = ("gemm1_kernel", "gemm2_kernel", "gemm1_wg_kernel", "gemm2_wg_kernel", "experts_fused_kernel",
                  "tiled_fused_kernel")


def is_expert_kernel(name: str) -> bool:
    """Whether a demangled kernel name is one of EXPERT_KERNELS (whole name)."""
    return any(f"moe::{k}<" in name or f"moe::{k}(" in name for k in EXPERT_KERNELS)


def per_dispatch(run_dir: str, counter: str) -> dict:
    """kernel name -> mean counter value per dispatch (summed over instances)."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(lambda: defaultdict(float))
    for path in files:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def summarize(run_dir: str, copy_dir: str, copy_mib: float, workload: str, launches_per_step: int = 1):
    """The traffic record of one workload and its table rows: each expert
    kernel's mean FETCH_SIZE and WRITE_SIZE per dispatch, divided by what the
    counters read per KiB of the calibration copy, summed over the kernels of
    one launch and multiplied by the launches of a step."""
    fetch = per_dispatch(os.path.join(run_dir, "FETCH_SIZE"), "FETCH_SIZE")
    write = per_dispatch(os.path.join(run_dir, "WRITE_SIZE"), "WRITE_SIZE")
    cfetch = per_dispatch(os.path.join(copy_dir, "copy_FETCH_SIZE"), "FETCH_SIZE")
    cwrite = per_dispatch(os.path.join(copy_dir, "copy_WRITE_SIZE"), "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    # the copy kernel is the one whose counters are largest
    fetch_factor = max(cfetch.values()) / copy_kib
    write_factor = max(cwrite.values()) / copy_kib

    kernels = sorted(k for k in fetch if is_expert_kernel(k))
    rows, total = [], 0.0
    rec = {"workload": workload, "kernels": kernels, "fetch_factor": fetch_factor,
           "write_factor": write_factor, "launches_per_step": launches_per_step}
    for k in kernels:
        rb = fetch[k] / fetch_factor * 1024.0
        wb = write.get(k, 0.0) / write_factor * 1024.0
        rows.append((k, fetch[k], write.get(k, 0.0), rb / 1e6, wb / 1e6))
        total += rb + wb
    rec["per_kernel"] = [{"kernel": k, "fetch_kib": f, "write_kib": w, "read_mb": r, "write_mb": x}
                         for k, f, w, r, x in rows]
    rec["traffic_bytes_per_launch"] = total
    rec["traffic_bytes"] = total * launches_per_step
    h = hashlib.sha256()
    for src in SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    rec["sources"] = SOURCES
    rec["sources_sha256"] = h.hexdigest()
    return rec, rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dir", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--copy-mib", type=float, required=True)
    ap.add_argument("--copy-dir", default=None,
                    help="where copy_FETCH_SIZE and copy_WRITE_SIZE are (default: --dir)")
    ap.add_argument("--launches-per-step", type=int, default=1,
                    help="expert-step launches per layer step (the expert-TP slices)")
    args = ap.parse_args()

    rec, rows = summarize(args.dir, args.copy_dir or args.dir, args.copy_mib, args.workload,
                          args.launches_per_step)
    out = os.path.join(ROOT, "profiles", f"experts_{args.workload}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"calibration: copy of {args.copy_mib:g} MiB reads FETCH_SIZE x{rec['fetch_factor']:.4f}, "
          f"WRITE_SIZE x{rec['write_factor']:.4f} per KiB moved")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |")
    print("|---|---|---|---|---|")
    for k, f, w, r, x in rows:
        print(f"| `{k}` | {f:.1f} | {w:.1f} | {r:.2f} | {x:.3f} |")
    total = rec["traffic_bytes_per_launch"]
    print(f"traffic per launch: {total / 1e6:.2f} MB; per step ({args.launches_per_step} launches): "
          f"{rec['traffic_bytes'] / 1e6:.2f} MB -> {out}")


if __name__ == "__main__":
    main()

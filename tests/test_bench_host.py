"""Host-side accounting of bench.py, on the CPU: the algorithmic bytes and
flops it divides by (checked against the per-expert weight bytes 27/16 I H and
the 6 R H I matrix flops of the routed rows), the dispatch rule that picks the
MFMA roofline, the committed HBM-traffic record and its source hash, and the
refusal of more than one GPU."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np

import bench
from nvfp4_block_scaled_route_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_weight_bytes_per_expert():
    """w13 codes + scales (2I x H/2, 2I x H/16) and w2 codes + scales (H x I/2,
    H x I/16): 27/16 I H bytes an expert; decode_b8's 42 touched experts are the
    111 476 736 weight bytes its bench line reports."""
    for name in ("decode_b8", "decode_b64_zipf", "expert_tp8_b32", "prefill_t4096"):
        wl = W.WORKLOADS[name]
        counts = np.zeros(wl.E, np.int64)
        counts[0] = 1
        ab = bench.algorithmic_bytes(wl, counts)
        assert ab["weights"] * 16 == 27 * wl.I * wl.H, name
    wl = W.WORKLOADS["decode_b8"]
    counts = np.zeros(wl.E, np.int64)
    counts[:42] = 1
    counts[:22] += 1                                     # 64 routes over 42 experts
    ab = bench.algorithmic_bytes(wl, counts)
    assert ab["touched"] == 42 and ab["weights"] == 111_476_736
    routes = int(counts.sum())
    assert routes == 64
    other = wl.T * (wl.H // 2 + wl.H // 16) + 2 * routes * (wl.I // 2 + wl.I // 16) + routes * wl.H * 2
    assert ab["other"] == other and ab["total"] == ab["weights"] + other


def test_bytes_with_the_finalize_and_slices():
    """With the finalize in the step, every slice's rows are read once more and
    the output written; with tp slices the input is read and rows written once
    a slice, the weights and the intermediate once in total."""
    wl = W.WORKLOADS["expert_tp8_b32"]
    counts = np.zeros(wl.E, np.int64)
    counts[:96] = 2
    counts[96:112] = 4
    routes = int(counts.sum())
    assert routes == wl.T * wl.K
    a = bench.algorithmic_bytes(wl, counts)
    f = bench.algorithmic_bytes(wl, counts, finalize=True)
    assert a["weights"] == f["weights"] == 112 * 27 * wl.I * wl.H // 16
    assert f["total"] - a["total"] == wl.tp * routes * wl.H * 2 + wl.T * wl.H * 2
    assert a["other"] == (wl.tp * wl.T * 9 * wl.H // 16 + 2 * routes * 9 * wl.I // 16
                          + wl.tp * routes * wl.H * 2)


def test_matrix_flops_of_the_routed_rows():
    """GEMM1 (2I x H) and GEMM2 (H x I) per route, 2 flops a multiply-add:
    6 R H I; prefill_t4096's 32768 routes give 1.237 TFLOP."""
    wl = W.WORKLOADS["prefill_t4096"]
    counts = np.full(wl.E, wl.T * wl.K // wl.E, np.int64)
    f = bench.algorithmic_flops(wl, counts)
    assert f == 6.0 * wl.T * wl.K * wl.H * wl.I
    assert abs(f - 1.23695e12) < 1e8


def test_roofline_choice_follows_the_dispatch_rule():
    """The register-tiled MFMA kernels (and the f16 MFMA roofline) only where
    an expert has on average a quarter of a 128-row block or more."""
    assert bench.mfma_bound(W.WORKLOADS["prefill_t4096"])
    for name in ("decode_b8", "decode_b64_zipf", "expert_tp8_b32", "tiny"):
        assert not bench.mfma_bound(W.WORKLOADS[name]), name


def test_traffic_record_matches_its_sources(tmp_path, monkeypatch):
    """A record is used while the kernel sources hash the same as when its
    counters were taken, and dropped (None) once one of them changes; every
    committed record either matches its sources or is dropped."""
    import hashlib
    for fn in os.listdir(os.path.join(ROOT, "profiles")):
        if fn.startswith("experts_") and fn.endswith("_traffic.json"):
            with open(os.path.join(ROOT, "profiles", fn)) as f:
                rec = json.load(f)
            got = bench.measured_traffic(rec["workload"])
            assert got is None or got == float(rec["traffic_bytes"]), fn
    src = "pkg/kernel.hip"
    os.makedirs(tmp_path / "pkg")
    with open(tmp_path / src, "w") as f:
        f.write("// kernel\n")
    rec = {"workload": "w", "traffic_bytes": 123.0, "sources": [src],
           "sources_sha256": hashlib.sha256(b"// kernel\n").hexdigest()}
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / "experts_w_traffic.json", "w") as f:
        json.dump(rec, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w") == 123.0
    with open(tmp_path / src, "a") as f:
        f.write("// changed\n")
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, counter, rows):
    """rocprofv3's counter_collection.csv columns the summary reads: one row a
    counter instance, (kernel, dispatch id, value)."""
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for k, d, v in rows:
            f.write(f'{d},"{k}",{counter},{v}\n')


def test_traffic_summary_scales_by_the_copy_and_the_launches(tmp_path):
    """FETCH_SIZE and WRITE_SIZE of a dispatch are summed over its instances
    and averaged over dispatches, divided by what the same counter reads per KiB
    of a copy of known size, summed over the step's expert kernels (a kernel the
    step does not launch left out) and multiplied by the launches of a step."""
    from nvfp4_block_scaled_route_amd import traffic_summary as ts
    step = "void moe::experts_fused_kernel<8, 4, 2, false>(moe::ExpArgs, unsigned int, moe::FinFuse)"
    tiled = "moe::tiled_fused_kernel(moe::ExpArgs, int, int, int, int)"
    other = "void moe::w16_gemm1_kernel<4>(moe::W16Args)"
    for name in (step, tiled):
        assert ts.is_expert_kernel(name)
    assert not ts.is_expert_kernel(other) and not ts.is_expert_kernel("moe::finalize_kernel<2>(moe::Fin)")
    run = tmp_path / "run"
    # two dispatches of the step kernel, two counter instances each: 600 and 400 KiB fetched
    _counter_csv(run / "FETCH_SIZE", "FETCH_SIZE",
                 [(step, 1, 250.0), (step, 1, 350.0), (step, 2, 100.0), (step, 2, 300.0), (other, 3, 9e9)])
    _counter_csv(run / "WRITE_SIZE", "WRITE_SIZE", [(step, 1, 20.0), (step, 2, 30.0), (other, 3, 9e9)])
    # a 1 MiB copy whose FETCH_SIZE reads half the KiB moved and WRITE_SIZE all of them
    _counter_csv(run / "copy_FETCH_SIZE", "FETCH_SIZE", [("copy", 1, 512.0), ("fill", 2, 8.0)])
    _counter_csv(run / "copy_WRITE_SIZE", "WRITE_SIZE", [("copy", 1, 1024.0)])
    rec, rows = ts.summarize(str(run), str(run), 1.0, "w", launches_per_step=8)
    assert rec["kernels"] == [step] and len(rows) == 1
    assert rec["fetch_factor"] == 0.5 and rec["write_factor"] == 1.0
    per_launch = (500.0 / 0.5 + 25.0) * 1024.0
    assert rec["traffic_bytes_per_launch"] == per_launch
    assert rec["traffic_bytes"] == 8 * per_launch
    assert rec["sources"] == ts.SOURCES and len(rec["sources_sha256"]) == 64
    # the committed records were written the same way: per step = launches x per launch
    for fn in os.listdir(os.path.join(ROOT, "profiles")):
        if fn.startswith("experts_") and fn.endswith("_traffic.json"):
            with open(os.path.join(ROOT, "profiles", fn)) as f:
                r = json.load(f)
            assert abs(r["traffic_bytes"] - r["launches_per_step"] * r["traffic_bytes_per_launch"]) \
                <= 1e-9 * r["traffic_bytes"], fn

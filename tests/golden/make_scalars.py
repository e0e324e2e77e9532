"""Writes tests/golden/scalars.json: the intermediate global scale a2_gscale of
every workload. Calls only the oracle and the seeded input generator.

The runner page ("MuseSparkModelOptNvFp4FusedMoE.process_weights_after_loading")
folds the intermediate's global scale into g1_scale_c (a13 * w3_gs / a2). Its
value comes from calibration, which the pages do not show. The reading here is
the plain one: pick the scale that maps the largest intermediate magnitude of
the workload (|silu(g) * u| with the scale taken as 1, over the routes of the
first 256 tokens) onto the largest NVFP4 magnitude, 6 * 448 = 2688, rounded to
fp32. Run: python tests/golden/make_scalars.py [name ...]
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from nvfp4_block_scaled_route_amd import workloads as W  # noqa: E402
from oracle.layer import intermediate_amax  # noqa: E402

CALIBRATION_TOKENS = 256
NVFP4_MAX = 6.0 * 448.0


def calibrate(name: str) -> dict:
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, a2_gscale=1.0)
    amax = intermediate_amax(inp, CALIBRATION_TOKENS)
    a2 = np.float32(NVFP4_MAX / amax)
    return {"fp32_hex": np.array([a2], dtype=">f4").tobytes().hex(), "value": float(a2),
            "amax_unit_scale": amax, "tokens": min(CALIBRATION_TOKENS, wl.T)}


def main(names):
    path = os.path.join(HERE, "scalars.json")
    table = {"a2_gscale": {}}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    for name in names or W.ORDER:
        table["a2_gscale"][name] = calibrate(name)
        print(name, table["a2_gscale"][name], flush=True)
    table["about"] = ("intermediate global scale per workload: 2688 / max |silu(g) u| over the "
                      "routes of the first 256 tokens, unit scale; written by make_scalars.py")
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])

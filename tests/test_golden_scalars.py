"""The stored intermediate global scales are what the calibration script computes
from the oracle (checked on the small workloads, where it takes seconds)."""
import numpy as np
import pytest

from nvfp4_block_scaled_route_amd import workloads as W
from tests.golden.make_scalars import calibrate


@pytest.mark.parametrize("name", ["tiny", "decode_b8"])
def test_stored_scale_matches_calibration(name):
    fresh = calibrate(name)
    assert fresh["fp32_hex"] == np.array([W.stored_a2_gscale(name)], dtype=">f4").tobytes().hex()


def test_calibrated_intermediate_fits_nvfp4():
    from oracle import layer as L
    from oracle.formats import decode_e4m3
    r = L.layer(W.make_inputs(W.WORKLOADS["tiny"]))
    sf = decode_e4m3(r["h_sf"])
    assert sf.max() <= 448 and np.mean(sf == 448) < 0.05 and np.all(sf > 0)

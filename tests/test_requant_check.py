"""The intermediate check of the GPU parity tests, exercised on the CPU with the
oracle standing in for a kernel: an intermediate requantized from h moved
within its error bound passes (its codes differ only at rounding boundaries);
a code or scale moved one step away from a boundary fails, and so does a code
two steps off."""
import numpy as np
import pytest

from nvfp4_block_scaled_route_amd import workloads as W
from oracle import formats as F
from oracle.layer import layer
from oracle.quant import quantize_nvfp4

from .gpu_common import abs_gemm1, check_requant, h_error_bound


@pytest.fixture(scope="module")
def case():
    wl = W.Workload("reqcheck", T=16, H=512, I=256, E=4, K=2, tile_m=16, seed=9)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    from oracle.layer import intermediate_amax
    inp = W.make_inputs(wl, a2_gscale=float(np.float32(2688.0 / intermediate_amax(probe))))
    ref = layer(inp)
    p = ref["rows_idx"]
    tokens = ref["meta"]["perm2tok"][p]
    experts = ref["meta"]["tile_expert"][p // wl.tile_m]
    abs_acc1 = abs_gemm1(ref["a_codes"], ref["a_sf"], tokens, experts, inp.w13_codes, inp.w13_sf)
    eb = h_error_bound(ref["acc1"], abs_acc1, experts, inp.g1_alphas, inp.g1_scale_c, ref["h"], wl.H)
    return ref, eb


def _run(ref, eb, codes, sf, max_frac=1e-3):
    check_requant(codes, sf, ref["h"], ref["h_codes"], ref["h_sf"], lambda sel: eb[sel], "cpu", max_frac)


def test_identical_intermediate_passes(case):
    ref, eb = case
    _run(ref, eb, ref["h_codes"].copy(), ref["h_sf"].copy())


def test_perturbed_within_bound_passes(case):
    """h moved by up to half its bound towards the nearest boundary flips
    codes right at boundaries only; those flips pass."""
    ref, eb = case
    h = ref["h"].astype(np.float64)
    rng = np.random.default_rng(0)
    moved = (h + rng.uniform(-0.5, 0.5, h.shape) * eb).astype(np.float32)
    codes, sf = quantize_nvfp4(moved, 1.0)
    _run(ref, eb, codes, sf, max_frac=1.0)


def _far_from_boundary(ref, eb):
    """A (row, element) whose oracle code is 2 (1.0) or 3 (1.5) and whose h sits
    in the middle of its rounding interval."""
    n = F.unpack_nibbles(ref["h_codes"])
    d = F.decode_e4m3(ref["h_sf"]).astype(np.float64)
    h = ref["h"].astype(np.float64)
    for r, i in zip(*np.nonzero((n & 7) == 3)):
        x = abs(h[r, i]) / d[r, i // 16]
        if abs(x - 1.5) < 0.05 and eb[r, i] < 0.01 * d[r, i // 16]:
            return r, i
    raise AssertionError("no interior code in the case")


def test_off_grid_code_fails(case):
    ref, eb = case
    r, i = _far_from_boundary(ref, eb)
    n = F.unpack_nibbles(ref["h_codes"]).copy()
    n[r, i] = (n[r, i] & 8) | 4                     # 1.5 -> 2.0, one step, but h is mid-interval
    with pytest.raises(AssertionError):
        _run(ref, eb, F.pack_nibbles(n), ref["h_sf"].copy())
    n[r, i] = (n[r, i] & 8) | 5                     # two steps
    with pytest.raises(AssertionError):
        _run(ref, eb, F.pack_nibbles(n), ref["h_sf"].copy())


def test_off_boundary_scale_fails(case):
    ref, eb = case
    r, i = _far_from_boundary(ref, eb)
    sf = ref["h_sf"].copy()
    sf[r, i // 16] += 1
    with pytest.raises(AssertionError):
        _run(ref, eb, ref["h_codes"].copy(), sf)

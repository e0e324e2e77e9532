"""NVFP4 quantization of activations (and of the intermediate after the gated
activation). Test infrastructure (see ``oracle/__init__``).

What the pages fix: the expert input is quantized with one fp32 global scale
into e2m1 codes packed two per byte, [T, H/2], and e4m3 scales per 16 values,
[T, H/16], in the plain row-major ("not swizzled") layout (the model page,
"_prepared_nvfp4_forward": ``scaled_fp4_quant(x, global_scale,
is_sf_swizzled_layout=False)``; the runner page,
"MuseSparkModelOptNvFp4FusedMoE.process_weights_after_loading":
``a1_gscale = 1 / a13``). The global scale multiplies the values into the range
the scales were calibrated for; the GEMM undoes it with the per-expert alphas,
which carry ``a13`` (the same process_weights_after_loading).

What the pages leave open, and the reading taken (the usual NVFP4 recipe):
per block of 16 values along the row,

    amax = max |x_i|                       (exact)
    s    = fl32(fl32(amax * gscale) / 6)   (6 = largest e2m1 magnitude)
    sf   = e4m3(s)                         (nearest even, saturating)
    d    = decode(sf)
    code_i = 0 for every i                 if d == 0
    code_i = e2m1(fl32(x_i * fl32(gscale / d)))   otherwise

Every step is one correctly rounded fp32 operation in this order: the codes
are integers decided by floats, so the decision is taken in the kernels'
precision with the kernels' operation order.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_e4m3, encode_e2m1, encode_e4m3, pack_nibbles

SF_VEC = 16


def quantize_nvfp4(x: np.ndarray, gscale: float) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [rows, n] (n % 16 == 0) -> (codes uint8 [rows, n/2],
    scales uint8 e4m3 [rows, n/16])."""
    x = np.asarray(x, dtype=np.float32)
    rows, n = x.shape
    assert n % SF_VEC == 0, "the row length must be a multiple of 16"
    g = np.float32(gscale)
    blocks = x.reshape(rows, n // SF_VEC, SF_VEC)
    amax = np.max(np.abs(blocks), axis=-1)                                  # exact
    s = ((amax * g).astype(np.float32) / np.float32(6.0)).astype(np.float32)
    sf = encode_e4m3(s)
    d = decode_e4m3(sf).astype(np.float32)                                  # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d == 0, np.float32(0.0), (g / d).astype(np.float32)).astype(np.float32)
    scaled = (blocks * r[..., None]).astype(np.float32)
    codes = encode_e2m1(scaled)
    codes = np.where((d == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return pack_nibbles(codes.reshape(rows, n)), sf.astype(np.uint8)


def dequantize_nvfp4(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """(codes [rows, n/2], scales [rows, n/16]) -> float64 [rows, n]: each element
    is e2m1(code) * e4m3(scale) of its block, in the globally scaled domain.
    Every such value is a multiple of 2^-10 with at most 6 significant bits."""
    from .formats import decode_e2m1, unpack_nibbles
    vals = decode_e2m1(unpack_nibbles(codes))
    rows, n = vals.shape
    s = decode_e4m3(sf)
    return (vals.reshape(rows, n // SF_VEC, SF_VEC) * s[..., None]).reshape(rows, n)

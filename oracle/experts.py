"""The routed experts: grouped GEMM1, gated activation with requantization,
grouped GEMM2. Test infrastructure (see ``oracle/__init__``).

What the pages fix (the runner page, "MuseSparkTrtLlmNvFp4Experts.apply_routed"
and "MuseSparkModelOptNvFp4FusedMoE.process_weights_after_loading"; the
flashinfer_ops page, "nvfp4_arguments"):
  * GEMM1 runs the NVFP4 input against w13 [E, 2I, H/2] with its e4m3 scales;
    rows [0, I) are the gate projection (w1), rows [I, 2I) the up projection
    (w3) -- the two weight global scales w13_weight_scale_2[:, 0] and [:, 1];
  * the activation is SwiGLU with no clamp, alpha or beta ("W4A4 SwiGLU");
  * output1_scale_gate_scalar = g1_alphas scales the gate side,
    output1_scale_scalar = g1_scale_c the up side, and g1_scale_c already holds
    the intermediate's global scale 1/a2, so the intermediate is requantized
    to NVFP4 with a unit global scale; output2_scale_scalar = g2_alphas scales
    GEMM2, whose rows are bf16 and are not finalized by the op.

Readings: g = acc_gate * g1_alphas[e] is the SiLU input ("keep the SiLU gate
input exact", the runner page, "_process_hopper_marlin_weights"),
u = acc_up * g1_scale_c[e]; h = silu(g) * u with silu(g) = g / (1 + e^-g),
all in fp64, then rounded to fp32 for the requantization decision (the
kernels' precision). GEMM2 rows are bf16(acc2 * g2_alphas[e]), rounded once,
to nearest even, from the fp64 value.

Exactness of the GEMMs: every dequantized operand is e2m1 * e4m3, a multiple
of 2^-10, so every product is a multiple of 2^-20. When sum_k |a_k| |w_k| stays
below 2^33 every partial sum is such a multiple below 2^53 * 2^-20 and is an
fp64 number, so the fp64 matrix product is exact in any summation order. The
bound is checked on every call (``_exact_matmul``).
"""
from __future__ import annotations

import numpy as np

from .formats import f64_to_bf16
from .quant import dequantize_nvfp4, quantize_nvfp4

EXACT_LIMIT = 2.0 ** 33


def _exact_matmul(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    """a [M, K] @ w[N, K].T for dequantized NVFP4 operands, exact (see above)."""
    if a.shape[0] == 0:
        return np.zeros((0, w.shape[0]))
    bound = float(np.abs(a).sum(axis=1).max()) * float(np.abs(w).max(initial=0.0))
    if not bound < EXACT_LIMIT:
        raise ArithmeticError(f"GEMM operand magnitudes {bound:.3g} exceed the exact range")
    return a @ w.T


def silu64(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gemm1(a_codes, a_sf, tokens, experts, w13_codes, w13_sf) -> np.ndarray:
    """Route r = (tokens[r], experts[r]) -> acc1 [R, 2I] float64 (exact)."""
    tokens = np.asarray(tokens)
    experts = np.asarray(experts)
    n2 = w13_codes.shape[1]
    acc = np.zeros((len(tokens), n2), dtype=np.float64)
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        a = dequantize_nvfp4(a_codes[tokens[sel]], a_sf[tokens[sel]])
        w = dequantize_nvfp4(w13_codes[e], w13_sf[e])
        acc[sel] = _exact_matmul(a, w)
    return acc


def swiglu_requant(acc1, experts, g1_alphas, g1_scale_c):
    """acc1 [R, 2I] -> (h fp32 [R, I], codes [R, I/2], scales [R, I/16])."""
    I = acc1.shape[1] // 2
    experts = np.asarray(experts)
    g = acc1[:, :I] * np.asarray(g1_alphas, dtype=np.float64)[experts][:, None]
    u = acc1[:, I:] * np.asarray(g1_scale_c, dtype=np.float64)[experts][:, None]
    h = (silu64(g) * u).astype(np.float32)
    codes, sf = quantize_nvfp4(h, 1.0)
    return h, codes, sf


def gemm2(h_codes, h_sf, experts, w2_codes, w2_sf) -> np.ndarray:
    """Route r's intermediate -> acc2 [R, H] float64 (exact)."""
    experts = np.asarray(experts)
    acc = np.zeros((len(experts), w2_codes.shape[1]), dtype=np.float64)
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        a = dequantize_nvfp4(h_codes[sel], h_sf[sel])
        w = dequantize_nvfp4(w2_codes[e], w2_sf[e])
        acc[sel] = _exact_matmul(a, w)
    return acc


def gemm2_rows_bf16(acc2, experts, g2_alphas) -> np.ndarray:
    scaled = acc2 * np.asarray(g2_alphas, dtype=np.float64)[np.asarray(experts)][:, None]
    return f64_to_bf16(scaled)


def experts_forward(a_codes, a_sf, tokens, experts, w13_codes, w13_sf, w2_codes, w2_sf,
                    g1_alphas, g1_scale_c, g2_alphas) -> dict:
    """All routed-expert steps for the routes (tokens[r], experts[r])."""
    acc1 = gemm1(a_codes, a_sf, tokens, experts, w13_codes, w13_sf)
    h, h_codes, h_sf = swiglu_requant(acc1, experts, g1_alphas, g1_scale_c)
    acc2 = gemm2(h_codes, h_sf, experts, w2_codes, w2_sf)
    rows = gemm2_rows_bf16(acc2, experts, g2_alphas)
    return dict(acc1=acc1, h=h, h_codes=h_codes, h_sf=h_sf, acc2=acc2, rows=rows)

"""The W4A16 expert variant: bf16 activations against the same NVFP4 weights.
Test infrastructure (see ``oracle/__init__``).

What the pages fix (the runner page, "MuseSparkModelOptNvFp4FusedMoE": the
route-major Marlin W4A16 GEMMs on Hopper, SwiGLU required;
"_process_hopper_marlin_weights"):
  * the activations are not quantized; the GEMMs take them in the activation
    dtype against the NVFP4 weights (codes times e4m3 block scales times a
    per-expert fp32 global scale);
  * GEMM1 applies one global scale to both halves of w13: the gate's,
    w13_weight_scale_2[:, 0], "keeping the SiLU gate input exact";
  * the up side is then off by up/gate, and GEMM2 compensates it: its global
    scale becomes w2_weight_scale_2 * (w13_weight_scale_2[:, 1] /
    w13_weight_scale_2[:, 0]) -- exact because SwiGLU is linear in the up side.

Readings (not on the pages): the gated activation's output h is held in the
activation dtype, bf16, between the GEMMs (rounded once from fp64 here); the
GEMM2 rows are bf16 as in the W4A4 path; the folded scalars are formed in fp32
as the passage writes them, s13 = gate, s2 = fp32(w2 * fp32(up / gate)). The
products of bf16 activations with NVFP4 weights and the sums are taken in fp64.
"""
from __future__ import annotations

import numpy as np

from .experts import silu64
from .formats import bf16_to_f64, f64_to_bf16
from .quant import dequantize_nvfp4


def fold_scalars(gate_gs, up_gs, w2_gs) -> tuple[np.ndarray, np.ndarray]:
    """Per-expert weight global scales -> (s13 for both halves of GEMM1, s2 for
    GEMM2), fp32."""
    gate = np.asarray(gate_gs, dtype=np.float32)
    up = np.asarray(up_gs, dtype=np.float32)
    w2 = np.asarray(w2_gs, dtype=np.float32)
    return gate.copy(), (w2 * (up / gate).astype(np.float32)).astype(np.float32)


def experts_w4a16(x_bf16, tokens, experts, w13_codes, w13_sf, w2_codes, w2_sf, s13, s2,
                  round_h: bool = True) -> dict:
    """Routes r = (tokens[r], experts[r]) -> dict(acc1 [R, 2I], h [R, I] (bf16
    bits if round_h, else fp64), acc2 [R, H], rows bf16 bits [R, H])."""
    tokens = np.asarray(tokens)
    experts = np.asarray(experts)
    I = w13_codes.shape[1] // 2
    H = w2_codes.shape[1]
    R = len(tokens)
    acc1 = np.zeros((R, 2 * I))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        acc1[sel] = bf16_to_f64(x_bf16[tokens[sel]]) @ dequantize_nvfp4(w13_codes[e], w13_sf[e]).T
    s13e = np.asarray(s13, dtype=np.float64)[experts][:, None]
    g = acc1[:, :I] * s13e
    u = acc1[:, I:] * s13e
    h64 = silu64(g) * u
    h = f64_to_bf16(h64) if round_h else h64
    hv = bf16_to_f64(h) if round_h else h64
    acc2 = np.zeros((R, H))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        acc2[sel] = hv[sel] @ dequantize_nvfp4(w2_codes[e], w2_sf[e]).T
    scaled = acc2 * np.asarray(s2, dtype=np.float64)[experts][:, None]
    return dict(acc1=acc1, h=h, acc2=acc2, rows=f64_to_bf16(scaled), rows64=scaled)

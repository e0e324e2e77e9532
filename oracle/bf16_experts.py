"""The BF16 expert layers: the routed experts of the layers an NVFP4 checkpoint
leaves unquantized. Test infrastructure (see ``oracle/__init__``).

What the pages fix (the flashinfer_ops page, "routed_experts_bf16" and
"bf16_arguments"; the runner page, "MuseSparkUnquantizedFusedMoE"): the op
takes the normed bf16 rows and the fp32 router logits, routes in-op with the
same routing method, bias and scaling factor as the NVFP4 layers, runs GEMM1
against bf16 w13 (gate and up), the gated activation, GEMM2 against bf16 w2,
and returns unfinalized rows (do_finalize=False) for the same post-expert
finalize.

Readings (not on the pages): the weights are read in their logical layout
(w13 [E, 2I, H] with the gate rows first, w2 [E, H, I]), the activation is
SwiGLU without scalars, the intermediate is held in bf16 between the GEMMs and
the rows are bf16 (each rounded once, to nearest even). Products and sums are
taken in fp64.
"""
from __future__ import annotations

import numpy as np

from .experts import silu64
from .formats import bf16_to_f64, f64_to_bf16


def experts_bf16(x_bf16, tokens, experts, w13_bf16, w2_bf16) -> dict:
    """Routes r = (tokens[r], experts[r]) -> dict(acc1 [R, 2I], h bf16 bits
    [R, I], acc2 [R, H], rows bf16 bits [R, H])."""
    tokens = np.asarray(tokens)
    experts = np.asarray(experts)
    I = w13_bf16.shape[1] // 2
    H = w2_bf16.shape[1]
    R = len(tokens)
    acc1 = np.zeros((R, 2 * I))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        acc1[sel] = bf16_to_f64(x_bf16[tokens[sel]]) @ bf16_to_f64(w13_bf16[e]).T
    h = f64_to_bf16(silu64(acc1[:, :I]) * acc1[:, I:])
    acc2 = np.zeros((R, H))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        acc2[sel] = bf16_to_f64(h[sel]) @ bf16_to_f64(w2_bf16[e]).T
    return dict(acc1=acc1, h=h, acc2=acc2, rows=f64_to_bf16(acc2))

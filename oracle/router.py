"""Router logits and the full routing chain (logits, then top-k routing). Test
infrastructure (see ``oracle/__init__``).

What the pages fix (the model page, "MuseSpark1xMoE"): the router is a linear
layer without bias from the router input (hidden size D) to the E local
experts, with fp32 parameters and an fp32 output ("GateLinear", out_dtype and
params_dtype float32); the router input is fp32 on the decode path
("wants_fp32_router_input"); the model's router output multiplier is folded
into the router weight as it loads ("_load_router_weight"), so the op is a plain
product. "_route_topk_and_pool" runs the full routing chain: the logits, then
"_compute_routing" on them (the routing of ``oracle/routing.py``).

What the pages leave open, and the reading taken: the accumulation precision of
the fp32 product. Each logit here is the fp32 rounding of the dot product
computed exactly: the products of two fp32 values are exact in fp64, and
``math.fsum`` returns their correctly rounded sum; that fp64 value is rounded to
fp32. Any fp32 accumulation is an approximation of this value. The width D of
the router input is not given by the workloads; they take D = H.
"""
from __future__ import annotations

import math

import numpy as np

from .routing import route


def router_logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x fp32 [T, D], w fp32 [E, D] (the router weight, multiplier folded in)
    -> logits fp32 [T, E]."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    T, D = x.shape
    E, D2 = w.shape
    assert D == D2
    out = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        prods = x[t][None, :] * w                # exact in fp64
        for e in range(E):
            out[t, e] = np.float32(math.fsum(prods[e].tolist()))
    return out


def route_from_hidden(x, w, expert_bias, K, route_scale=1.0, is_padding=None):
    """The full routing chain: router logits, then top-k routing ->
    (ids int32 [T, K], weights fp32 [T, K], logits fp32 [T, E])."""
    logits = router_logits(x, w)
    ids, weights = route(logits, expert_bias, K, route_scale, is_padding)
    return ids, weights, logits

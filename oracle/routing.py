"""MuseSpark1x top-k routing. Test infrastructure (see ``oracle/__init__``).

The pages fix the method (the runner page, "validate_deployment": the routing
must classify as sigmoid scores, plus an expert bias, sum-renormalized, no
expert groups, route scale 1.0; the model page, "MuseSpark1xMoE": scores by
sigmoid, ``router_score_division_eps=1e-15``, ``renormalize=True``,
``e_score_correction_bias``; the model page, "_prepared_nvfp4_forward":
padding tokens route nowhere, their ids are -1).

Readings where the pages are silent:
  * the expert bias takes part in the selection only; the weights are the
    unbiased sigmoid scores of the chosen experts, renormalized (the plain
    meaning of a score "correction" bias). ``bias_in_weights=True`` selects the
    other reading for tests;
  * ties between equal keys go to the lower expert index; the K chosen experts
    are listed by key, descending;
  * w_k = fl32(s_k / fl32(sum_k s_k + 1e-15)) * route_scale, the sum taken in
    fp32 over k = 0 .. K-1 in that order;
  * sigmoid is defined by one written algorithm so that two independent
    implementations agree to the bit (``sigmoid32``).
Padding tokens: ids -1, weights 0.
"""
from __future__ import annotations

import numpy as np

F = np.float32

# sigmoid32: s(l) = 1 / (1 + exp(-l)), with exp by Cody and Waite's additive
# range reduction x = n ln2 + r, |r| <= ln2 / 2, and the degree-7 Taylor
# polynomial of e^r in Horner form. No fused multiply-add anywhere: every
# operation below is one correctly rounded fp32 operation, in this order.
LOG2E = F(1.4426950408889634)
LN2_HI = F(0.693359375)              # 355/512: n * LN2_HI is exact for |n| < 2^15
LN2_LO = F(0.6931471805599453 - 0.693359375)
TAYLOR = [F(1.0 / 5040.0), F(1.0 / 720.0), F(1.0 / 120.0), F(1.0 / 24.0),
          F(1.0 / 6.0), F(0.5), F(1.0), F(1.0)]
EXP_HI = F(80.0)                     # exp(x) for x > 80: the sigmoid is taken as 0 (true value < 2e-35)
EXP_LO = F(-20.0)                    # exp(x) for x < -20 is below half an ulp of 1: sigmoid 1


def exp32(x: np.ndarray) -> np.ndarray:
    """exp for x in [-20, 80] (float32 in, float32 out), by the algorithm above."""
    x = np.asarray(x, dtype=F)
    n = np.rint((x * LOG2E).astype(F)).astype(F)          # round half to even
    r = (x - (n * LN2_HI).astype(F)).astype(F)
    r = (r - (n * LN2_LO).astype(F)).astype(F)
    p = TAYLOR[0]
    for c in TAYLOR[1:]:
        p = ((p * r).astype(F) + c).astype(F)
    return np.ldexp(p, n.astype(np.int32)).astype(F)       # exact scaling by 2^n


def sigmoid32(logit: np.ndarray) -> np.ndarray:
    l = np.asarray(logit, dtype=F)
    x = (-l).astype(F)
    xc = np.clip(x, EXP_LO, EXP_HI)
    e = exp32(xc)
    s = (F(1.0) / (F(1.0) + e).astype(F)).astype(F)
    s = np.where(x > EXP_HI, F(0.0), s)
    s = np.where(x < EXP_LO, F(1.0), s)
    return s.astype(F)


def route(logits: np.ndarray, expert_bias: np.ndarray | None, top_k: int,
          route_scale: float = 1.0, is_padding: np.ndarray | None = None,
          eps: float = 1e-15, bias_in_weights: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """logits fp32 [T, E] -> (ids int32 [T, K], weights fp32 [T, K])."""
    logits = np.asarray(logits, dtype=F)
    T, E = logits.shape
    assert 1 <= top_k <= E
    s = sigmoid32(logits)
    bias = np.zeros(E, dtype=F) if expert_bias is None else np.asarray(expert_bias, dtype=F)
    key = (s + bias[None, :]).astype(F)
    # Stable sort of -key: equal keys keep ascending expert order.
    order = np.argsort(-key, axis=1, kind="stable")[:, :top_k]
    ids = order.astype(np.int32)
    chosen = np.take_along_axis(key if bias_in_weights else s, order, axis=1).astype(F)
    total = np.zeros(T, dtype=F)
    for k in range(top_k):
        total = (total + chosen[:, k]).astype(F)
    denom = (total + F(eps)).astype(F)
    w = (chosen / denom[:, None]).astype(F)
    w = (w * F(route_scale)).astype(F)
    if is_padding is not None:
        pad = np.asarray(is_padding).astype(bool)
        ids[pad] = -1
        w[pad] = F(0.0)
    return ids, w

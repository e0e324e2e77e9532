"""One MoE layer's routed-expert path, composed from the oracle's steps, and the
rel-L2 probe. Test infrastructure (see ``oracle/__init__``).

The order of the steps is the runner page's ("MuseMoERunner",
"MuseSparkTrtLlmNvFp4Experts.apply_routed", "MusePostExpertFinalize") and the
model page's ("_prepared_nvfp4_forward"): quantize the expert input, route,
run the routed experts up to the GEMM2 rows, finalize.
"""
from __future__ import annotations

import numpy as np

from . import experts as ex
from .finalize import finalize, finalize_routes
from .formats import bf16_to_f64
from .permute import permute
from .quant import quantize_nvfp4
from .routing import route


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    """sqrt(sum (a - b)^2 / sum b^2) in fp64, b the reference (the expert_tp page,
    "probe_rel_l2": norms in fp64 so that large bf16 rows cannot overflow them)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.sum(b * b))
    num = float(np.sum((a - b) ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(np.sqrt(num / den))


def quantize_input(inp):
    x = bf16_to_f64(inp.x_bf16).astype(np.float32)
    return quantize_nvfp4(x, float(inp.a1_gscale[0]))


def route_inputs(inp, route_scale: float = 1.0, is_padding=None):
    return route(inp.logits, inp.expert_bias, inp.wl.K, route_scale, is_padding)


def layer(inp, tile_m: int | None = None, is_padding=None) -> dict:
    """The whole layer on every token (sizes the oracle finishes in seconds)."""
    wl = inp.wl
    m = wl.tile_m if tile_m is None else tile_m
    a_codes, a_sf = quantize_input(inp)
    ids, weights = route_inputs(inp, is_padding=is_padding)
    meta = permute(ids, 0, wl.E, m)
    p = np.nonzero(meta["perm2tok"] >= 0)[0]
    tokens = meta["perm2tok"][p]
    experts = meta["tile_expert"][p // m]
    fw = ex.experts_forward(a_codes, a_sf, tokens, experts, inp.w13_codes, inp.w13_sf,
                            inp.w2_codes, inp.w2_sf, inp.g1_alphas, inp.g1_scale_c,
                            inp.g2_alphas)
    rows = np.zeros((meta["rows_max"], wl.H), dtype=np.uint16)
    rows[p] = fw["rows"]
    out = finalize(rows, meta["exp2perm"], weights, inp.norm_weight_bf16, wl.gain_center,
                   wl.eps, wl.weight_before_norm)
    return dict(a_codes=a_codes, a_sf=a_sf, ids=ids, weights=weights, meta=meta,
                rows_idx=p, rows=rows, out=out, **{k: v for k, v in fw.items() if k != "rows"})


def layer_sampled(inp, token_idx, a_codes=None, a_sf=None, ids=None, weights=None) -> dict:
    """The layer's output for a sample of tokens only: their routes' GEMM rows
    (in route order) and their finalized outputs. The permutation does not
    change any token's output, so it is not needed here."""
    wl = inp.wl
    token_idx = np.asarray(token_idx, dtype=np.int64)
    if a_codes is None:
        a_codes, a_sf = quantize_input(inp)
    if ids is None:
        ids, weights = route_inputs(inp)
    sub_ids = ids[token_idx]
    served = sub_ids >= 0
    tt, kk = np.nonzero(served)
    tokens = token_idx[tt]
    experts = sub_ids[tt, kk]
    fw = ex.experts_forward(a_codes, a_sf, tokens, experts, inp.w13_codes, inp.w13_sf,
                            inp.w2_codes, inp.w2_sf, inp.g1_alphas, inp.g1_scale_c,
                            inp.g2_alphas)
    rr = np.zeros((len(token_idx), wl.K, wl.H), dtype=np.uint16)
    rr[tt, kk] = fw["rows"]
    out = finalize_routes(rr, served, weights[token_idx], inp.norm_weight_bf16,
                          wl.gain_center, wl.eps, bool(wl.weight_before_norm))
    return dict(route_rows=rr, served=served, out=out, ids=sub_ids, **fw)


def intermediate_amax(inp, n_tokens: int | None = None) -> float:
    """Largest |silu(g) * u| over the routes of the first n_tokens tokens, with the
    intermediate global scale taken as 1 (g1_scale_c without it): what the
    workloads' intermediate global scale is calibrated from."""
    wl = inp.wl
    T = wl.T if n_tokens is None else min(n_tokens, wl.T)
    a_codes, a_sf = quantize_input(inp)
    ids, _ = route_inputs(inp)
    tt, kk = np.nonzero(ids[:T] >= 0)
    experts = ids[tt, kk]
    acc1 = ex.gemm1(a_codes, a_sf, tt, experts, inp.w13_codes, inp.w13_sf)
    h, _, _ = ex.swiglu_requant(acc1, experts, inp.g1_alphas, inp.g1_scale_c)
    return float(np.max(np.abs(h.astype(np.float64))))

"""Post-expert finalize: per-route RMSNorm, top-k weighted fp32 reduce.
Test infrastructure (see ``oracle/__init__``).

The pages define it as torch ops (the runner page, "MusePostExpertFinalize",
"_finalize_native" -- "the kernels' reference" -- and "_finalize_chunk"):
gather each route's GEMM2 row by its permuted index (-1 reads as a zero row),
when the rows are tensor-parallel partial sums add them before the norm (in
fp32, then one bf16 rounding: the expert_tp page, "probe_rel_l2"), apply the
post-expert RMSNorm with an fp32 output, multiply by the route's weight, sum
over the K routes in fp32 and write the bf16 output. The norm weight is used in
the activation dtype and the gain centre is added in fp32 ("_effective_weight").
The post-expert norm is "MuseSpark1xRMSNormWithInputScale" with a zero-centred
gain around "one" (the model page, "MuseSpark1xMoE"); norms of that kind apply
their weight before normalizing (the model page, "_uses_flashinfer_dual_norm").

Readings: RMSNorm over the H values of a row, y = z / sqrt(mean(z^2) + eps),
with z = gamma * r when the weight applies before the norm and
y = gamma * (r / sqrt(mean(r^2) + eps)) otherwise; gamma = fl32(w + centre).
The norm is computed in fp64 and its output rounded to fp32 (the pages' fp32
norm output); weight products and the k-sum (k ascending) are fp32, as the
pages fix; the output is bf16, nearest even.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, f32_to_bf16, f64_to_bf16


def sum_partials(partials: list[np.ndarray]) -> np.ndarray:
    """bf16 partial rows (uint16) -> bf16(fp32 sum over partials in order)."""
    acc = bf16_to_f64(partials[0]).astype(np.float32)
    for p in partials[1:]:
        acc = (acc + bf16_to_f64(p).astype(np.float32)).astype(np.float32)
    return f32_to_bf16(acc)


def gamma_f32(norm_weight_bf16, gain_center: float, H: int) -> np.ndarray:
    if norm_weight_bf16 is None:
        w = np.ones(H, dtype=np.float32)
    else:
        w = bf16_to_f64(norm_weight_bf16).astype(np.float32)
    return (w + np.float32(gain_center)).astype(np.float32)


def rmsnorm_f32out(r: np.ndarray, gamma: np.ndarray, eps: float, weight_before_norm: bool) -> np.ndarray:
    """r float64 [..., H] -> float32 [..., H]."""
    g = gamma.astype(np.float64)
    eps64 = float(np.float32(eps))
    if weight_before_norm:
        z = g * r
        y = z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps64)
    else:
        y = g * (r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps64))
    return y.astype(np.float32)


def finalize_routes(route_rows_bf16: np.ndarray, served: np.ndarray, weights: np.ndarray,
                    norm_weight_bf16, gain_center: float, eps: float,
                    weight_before_norm: bool) -> np.ndarray:
    """route_rows [T, K, H] bf16 bits, served [T, K] bool, weights fp32 [T, K] -> out bf16 [T, H]."""
    T, K, H = route_rows_bf16.shape
    r = bf16_to_f64(route_rows_bf16)
    r = np.where(np.asarray(served)[..., None], r, 0.0)
    y = rmsnorm_f32out(r, gamma_f32(norm_weight_bf16, gain_center, H), eps, weight_before_norm)
    w = np.asarray(weights, dtype=np.float32)
    acc = np.zeros((T, H), dtype=np.float32)
    for k in range(K):
        acc = (acc + (y[:, k, :] * w[:, k][:, None]).astype(np.float32)).astype(np.float32)
    return f32_to_bf16(acc)


def route_rows(rows_bf16: np.ndarray, exp2perm: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The GEMM2 row of every route in route order (-1 reads as row 0, masked),
    as the expert_tp page's "route_rows" defines it."""
    idx = np.asarray(exp2perm, dtype=np.int64)
    served = idx >= 0
    g = rows_bf16[np.maximum(idx, 0)]
    g = np.where(served[..., None], g, np.uint16(0)).astype(np.uint16)
    return g, served


def finalize(rows_bf16, exp2perm, weights, norm_weight_bf16, gain_center, eps,
             weight_before_norm, partials: list | None = None) -> np.ndarray:
    """Permuted rows [Rp, H] (or a list of tensor-parallel partial rows, summed
    first) -> out bf16 [T, H]."""
    if partials is not None:
        rows_bf16 = sum_partials(partials)
    rr, served = route_rows(rows_bf16, exp2perm)
    return finalize_routes(rr, served, weights, norm_weight_bf16, gain_center, eps,
                           bool(weight_before_norm))

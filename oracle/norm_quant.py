"""Pre-expert RMSNorm fused into the NVFP4 input quantizer. Test infrastructure
(see ``oracle/__init__``).

What the pages fix (the model page, "MuseSpark1xMoE"): the pooled hidden state
passes the pre-expert norm, an RMSNorm with a weight, a zero-centred gain
("post_norm_gain_center_type" "one") and eps ``rms_norm_eps``, before it is
quantized for the experts. When the norm has a weight applied *after*
normalizing and no variance override ("norm_fuses_into_nvfp4_quant"), the
decode path runs the norm inside the quantizer: one op takes the pooled rows,
the norm weight, its eps, the fused gain centre and the input global scale and
returns the NVFP4 codes and block scales ("_prepared_nvfp4_forward",
``norm_quant_trtllm_nvfp4(pooled, num_tokens, norm.weight, eps, gain_center,
global_scale)``).

What the pages leave open, and the readings taken:
  * the norm is y_j = (x_j * r) * gamma_j with r = 1/sqrt(mean_j x_j^2 + eps)
    (eps inside the root) and gamma_j = fl32(w_j + gain_center), the weight
    stored in the activation dtype (the same gain convention as the
    post-expert finalize, the runner page, "_effective_weight");
  * a fused norm has no reason to round its output to the activation dtype:
    y stays fp32 and goes straight into the quantizer (``quantize_nvfp4``);
  * precision, step by step (each fl32 one correctly rounded fp32 operation):
        s  = sum_j x_j^2          exact value, rounded once to fp64
        ms = fl32(fl64(s / H))
        r  = fl32(1 / fl32(sqrt(fl32(ms + eps))))
        y_j = fl32(fl32(x_j * r) * gamma_j)
    The squares of bf16 values are exact in fp64; the sum is taken with
    ``math.fsum`` (the correctly rounded sum). A kernel that sums in fp64 in
    another order agrees on ms unless the exact sum lies within a few fp64 ulps
    of an fp32 rounding boundary.
  * a missing norm weight means w = 1.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_to_f64
from .quant import quantize_nvfp4


def norm_scale(x_bf16: np.ndarray, eps: float) -> np.ndarray:
    """bf16 bits [T, H] -> the fp32 reciprocal RMS r of every row, [T]."""
    x = bf16_to_f64(np.asarray(x_bf16, dtype=np.uint16))
    T, H = x.shape
    r = np.empty(T, dtype=np.float32)
    e = np.float32(eps)
    for t in range(T):
        s = math.fsum((x[t] * x[t]).tolist())          # squares exact in fp64
        ms = np.float32(s / H)
        d = np.float32(ms + e)
        q = np.float32(np.sqrt(d))
        r[t] = np.float32(np.float32(1.0) / q)
    return r


def gamma(norm_weight_bf16, gain_center: float, H: int) -> np.ndarray:
    """fl32(w + gain_center), w = 1 where no weight is given."""
    if norm_weight_bf16 is None:
        w = np.ones(H, dtype=np.float32)
    else:
        w = bf16_to_f64(np.asarray(norm_weight_bf16, dtype=np.uint16)).astype(np.float32)
    return (w + np.float32(gain_center)).astype(np.float32)


def normalize(x_bf16: np.ndarray, norm_weight_bf16, gain_center: float, eps: float) -> np.ndarray:
    """bf16 bits [T, H] -> the fp32 normalized rows y [T, H]."""
    x = bf16_to_f64(np.asarray(x_bf16, dtype=np.uint16)).astype(np.float32)   # exact
    r = norm_scale(x_bf16, eps)
    g = gamma(norm_weight_bf16, gain_center, x.shape[1])
    return ((x * r[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)


def norm_quant(x_bf16: np.ndarray, norm_weight_bf16, gain_center: float, eps: float,
               gscale: float) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [T, H] -> (codes uint8 [T, H/2], e4m3 scales uint8 [T, H/16])."""
    return quantize_nvfp4(normalize(x_bf16, norm_weight_bf16, gain_center, eps), gscale)

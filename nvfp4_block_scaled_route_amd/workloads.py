"""Seeded synthetic workloads for one NVFP4 routed-MoE layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds only random draws and plain data handling (dtype casts,
byte packing of already-random nibbles). None of the method's arithmetic lives
here: no quantizer, no routing, no GEMM, no norm. Random numbers the method
would consume are drawn here and passed in as inputs.

The five workloads are the routed-expert shapes of the MuseSpark1x MoE layer:
a tiny correctness case, decode at the build batch b = 8 (the batch the
specialized-decode runtime warms up and probes at, "FlashInferOps" on the
flashinfer_ops page), decode at b = 64 with Zipf-skewed routing, a prefill
chunk, and one expert-tensor-parallel slice set (the expert_tp page).

Every tensor draws from its own child stream of ``SeedSequence(seed)`` so the
order of generation does not matter.

Readings of the workload descriptions:
  * block scales "drawn from U[0.5, 2]": the scale byte is drawn uniformly from
    the e4m3 codes whose values lie in [0.5, 2] (0x30 .. 0x40 inclusive);
  * weight global scales are 1.0, so the per-expert kernel scalars are the
    drawn alphas: g1_alphas ~ U[0.5, 1.5]; g1_scale_c = U[0.5, 1.5] times the
    intermediate global scale a2_gscale; g2_alphas = U[0.5, 1.5] divided by it.
    a2_gscale is a stored per-workload constant (tests/golden/scalars.json),
    written by a script that calls only the oracle: it maps the largest
    intermediate magnitude of the workload onto the NVFP4 range 6 * 448;
  * activations bf16 N(0, 1) (fp32 draws rounded to bf16 to nearest even);
    the prefill chunk multiplies 1% of elements by 20 before the rounding;
  * router logits fp32 N(0, 1); the skewed decode adds b_e = -1.1 ln(rank_e)
    with rank a seeded permutation of 1..E (Zipf(1.1) popularity);
  * post-expert norm: gain gamma ~ U[0.9, 1.1] stored as bf16(gamma - 1) with
    gain centre 1.0, applied before the norm, eps 1e-6.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np
import torch

SF_VEC = 16  # elements per NVFP4 block scale

_GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "tests", "golden", "scalars.json")


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # expert hidden width
    I: int          # intermediate width
    E: int          # experts
    K: int          # top-k
    tp: int = 1     # expert-TP slices run one after another
    zipf: float = 0.0
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0
    tile_m: int = 16
    eps: float = 1e-6
    gain_center: float = 1.0
    weight_before_norm: int = 1

    @property
    def routes(self) -> int:
        return self.T * self.K


WORKLOADS = {
    "tiny": Workload("tiny", T=4, H=256, I=128, E=8, K=2, tile_m=16),
    "decode_b8": Workload("decode_b8", T=8, H=2048, I=768, E=64, K=8, tile_m=16),
    "decode_b64_zipf": Workload("decode_b64_zipf", T=64, H=4096, I=1536, E=128, K=8,
                                zipf=1.1, tile_m=16),
    "prefill_t4096": Workload("prefill_t4096", T=4096, H=4096, I=1536, E=128, K=8,
                              outlier_p=0.01, outlier_scale=20.0, tile_m=128),
    "expert_tp8_b32": Workload("expert_tp8_b32", T=32, H=4096, I=2048, E=128, K=8,
                               tp=8, tile_m=16),
}
ORDER = ["tiny", "decode_b8", "decode_b64_zipf", "prefill_t4096", "expert_tp8_b32"]

_STREAMS = ["x", "outlier_mask", "logits", "zipf_perm", "w13_codes", "w13_sf",
            "w2_codes", "w2_sf", "g1_alphas", "g1_scale_c", "g2_alphas", "gamma",
            "router_x", "router_w", "gs_gate", "gs_up", "gs_w2", "bf16_w13", "bf16_w2"]


def _rng(seed: int, stream: str) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(_STREAMS.index(stream),))
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def stored_a2_gscale(name: str) -> float:
    with open(_GOLDEN) as f:
        table = json.load(f)
    entry = table["a2_gscale"][name]
    return float(np.frombuffer(bytes.fromhex(entry["fp32_hex"]), dtype=">f4")[0])


@dataclass
class Inputs:
    wl: Workload
    x_bf16: np.ndarray          # uint16 [T, H]
    logits: np.ndarray          # f32 [T, E]
    expert_bias: np.ndarray     # f32 [E]
    w13_codes: np.ndarray       # uint8 [E, 2I, H/2], logical rows: gate [0, I), up [I, 2I)
    w13_sf: np.ndarray          # uint8 (e4m3 bytes) [E, 2I, H/16]
    w2_codes: np.ndarray        # uint8 [E, H, I/2]
    w2_sf: np.ndarray           # uint8 [E, H, I/16]
    a1_gscale: np.ndarray       # f32 [1]
    g1_alphas: np.ndarray       # f32 [E]
    g1_scale_c: np.ndarray      # f32 [E]
    g2_alphas: np.ndarray       # f32 [E]
    norm_weight_bf16: np.ndarray  # uint16 [H], stores gamma - gain_center
    extra: dict = field(default_factory=dict)


def _scale_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    # e4m3 codes 0x30 (0.5) .. 0x40 (2.0): the codes whose values lie in [0.5, 2].
    return rng.integers(0x30, 0x41, size=shape, dtype=np.uint8)


def make_router_inputs(wl: Workload, seed: int | None = None, tokens: int | None = None):
    """The router's fp32 input [T, D] (N(0,1)) and weight [E, D] (N(0, 1/D), so
    that the logits are about N(0,1) like the workloads' direct logits), with
    D = H; `tokens` draws only the first rows of the input."""
    seed = wl.seed if seed is None else seed
    T = wl.T if tokens is None else tokens
    x = _rng(seed, "router_x").standard_normal((T, wl.H), dtype=np.float32)
    w = (_rng(seed, "router_w").standard_normal((wl.E, wl.H), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(wl.H))).astype(np.float32)
    return x, w


def make_weight_global_scales(wl: Workload, seed: int | None = None):
    """Per-expert fp32 weight global scales of the W4A16 variant: the gate and
    up halves of w13 and w2, each U[0.5, 1.5]."""
    seed = wl.seed if seed is None else seed
    return tuple(_rng(seed, s).uniform(0.5, 1.5, wl.E).astype(np.float32)
                 for s in ("gs_gate", "gs_up", "gs_w2"))


def make_bf16_weights(wl: Workload, seed: int | None = None):
    """bf16 expert weights for the BF16 expert layers, logical layout:
    w13 [E, 2I, H] (gate rows first) ~ N(0, 1/H), w2 [E, H, I] ~ N(0, 1/I)."""
    seed = wl.seed if seed is None else seed
    E, H, I = wl.E, wl.H, wl.I
    w13 = _rng(seed, "bf16_w13").standard_normal((E, 2 * I, H), dtype=np.float32) * np.float32(H ** -0.5)
    w2 = _rng(seed, "bf16_w2").standard_normal((E, H, I), dtype=np.float32) * np.float32(I ** -0.5)
    return to_bf16_bits(w13), to_bf16_bits(w2)


def make_weights(wl: Workload, seed: int | None = None):
    seed = wl.seed if seed is None else seed
    E, H, I = wl.E, wl.H, wl.I
    w13_codes = _rng(seed, "w13_codes").integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    w13_sf = _scale_bytes(_rng(seed, "w13_sf"), (E, 2 * I, H // SF_VEC))
    w2_codes = _rng(seed, "w2_codes").integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    w2_sf = _scale_bytes(_rng(seed, "w2_sf"), (E, H, I // SF_VEC))
    return w13_codes, w13_sf, w2_codes, w2_sf


def make_inputs(wl: Workload, seed: int | None = None, a2_gscale: float | None = None,
                with_weights: bool = True) -> Inputs:
    seed = wl.seed if seed is None else seed
    T, H, E = wl.T, wl.H, wl.E
    x = _rng(seed, "x").standard_normal((T, H), dtype=np.float32)
    if wl.outlier_p > 0:
        mask = _rng(seed, "outlier_mask").random((T, H)) < wl.outlier_p
        x = np.where(mask, x * np.float32(wl.outlier_scale), x).astype(np.float32)
    logits = _rng(seed, "logits").standard_normal((T, E), dtype=np.float32)
    if wl.zipf > 0:
        rank = _rng(seed, "zipf_perm").permutation(E) + 1
        logits = (logits + (-wl.zipf * np.log(rank)).astype(np.float32)[None, :]).astype(np.float32)
    if with_weights:
        w13_codes, w13_sf, w2_codes, w2_sf = make_weights(wl, seed)
    else:
        w13_codes = w13_sf = w2_codes = w2_sf = None
    if a2_gscale is None:
        a2_gscale = stored_a2_gscale(wl.name)
    a2 = np.float32(a2_gscale)
    g1_alphas = _rng(seed, "g1_alphas").uniform(0.5, 1.5, E).astype(np.float32)
    g1_scale_c = (_rng(seed, "g1_scale_c").uniform(0.5, 1.5, E).astype(np.float32) * a2).astype(np.float32)
    g2_alphas = (_rng(seed, "g2_alphas").uniform(0.5, 1.5, E).astype(np.float32) / a2).astype(np.float32)
    gamma = _rng(seed, "gamma").uniform(0.9, 1.1, H).astype(np.float32)
    norm_w = to_bf16_bits((gamma - np.float32(wl.gain_center)).astype(np.float32))
    return Inputs(
        wl=wl, x_bf16=to_bf16_bits(x), logits=logits,
        expert_bias=np.zeros(E, dtype=np.float32),
        w13_codes=w13_codes, w13_sf=w13_sf, w2_codes=w2_codes, w2_sf=w2_sf,
        a1_gscale=np.ones(1, dtype=np.float32),
        g1_alphas=g1_alphas, g1_scale_c=g1_scale_c, g2_alphas=g2_alphas,
        norm_weight_bf16=norm_w,
    )

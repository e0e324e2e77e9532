"""One MoE layer's routed-expert path through the C-ABI, with its buffers.

The step order is the model page's "_prepared_nvfp4_forward" and the runner
page's "MuseSparkTrtLlmNvFp4Experts.apply_routed" / "MusePostExpertFinalize":
route, quantize the expert input, experts up to the GEMM2 rows, finalize. This
module only allocates device buffers (torch) and calls the library; all
arithmetic runs in the HIP kernels.

Expert TP on one GPU (the expert_tp page): the tp slices of the converted
weights are byte views (``slice_weights``); each slice's experts write their
K-partial GEMM2 rows into ``rows[r]`` and the finalize sums them before the norm.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import native as N


def pack_weights(w13_codes, w13_sf, w2_codes, w2_sf, g1_alphas, g1_scale_c, g2_alphas,
                 stream=None) -> N.Weights:
    """Logical device tensors ([E, 2I, H/2], [E, 2I, H/16], [E, H, I/2], [E, H, I/16])
    -> converted weights (new device tensors, same byte counts)."""
    E, n2, half_h = w13_codes.shape
    I, H = n2 // 2, half_h * 2
    c13, s13 = torch.empty_like(w13_codes), torch.empty_like(w13_sf)
    c2, s2 = torch.empty_like(w2_codes), torch.empty_like(w2_sf)
    N.moe_pack_w13(w13_codes, w13_sf, E, I, H, c13, s13, stream)
    N.moe_pack_w2(w2_codes, w2_sf, E, H, I, c2, s2, stream)
    return N.Weights(
        w13=c13, w13_sf=s13, w2=c2, w2_sf=s2,
        w13_expert_stride=2 * I * H // 2, w13_pair_stride=(H // 64) * 1024,
        w13_sf_expert_stride=2 * I * H // 16, w13_sf_pair_stride=(H // 64) * 128,
        w2_expert_stride=H * I // 2, w2_pair_stride=(I // 64) * 1024,
        w2_sf_expert_stride=H * I // 16, w2_sf_pair_stride=(I // 64) * 128,
        g1_alphas=g1_alphas, g1_scale_c=g1_scale_c, g2_alphas=g2_alphas)


def slice_weights(full: N.Weights, r: int, tp: int, H: int, I: int) -> N.Weights:
    """Expert-TP slice r of tp as byte views (no copy): w13 row pairs
    [rI'/16, (r+1)I'/16), w2 k-tiles [rI'/64, (r+1)I'/64) of every row pair."""
    s = I // tp
    if s % 64:
        raise ValueError(f"slice width {s} is not a multiple of 64")
    p13 = s // 16 * r
    t2 = s // 64 * r
    return N.Weights(
        w13=full.w13, w13_sf=full.w13_sf, w2=full.w2, w2_sf=full.w2_sf,
        w13_expert_stride=full.w13_expert_stride, w13_pair_stride=full.w13_pair_stride,
        w13_sf_expert_stride=full.w13_sf_expert_stride, w13_sf_pair_stride=full.w13_sf_pair_stride,
        w2_expert_stride=full.w2_expert_stride, w2_pair_stride=full.w2_pair_stride,
        w2_sf_expert_stride=full.w2_sf_expert_stride, w2_sf_pair_stride=full.w2_sf_pair_stride,
        g1_alphas=full.g1_alphas, g1_scale_c=full.g1_scale_c, g2_alphas=full.g2_alphas,
        w13_offset=full.w13_offset + p13 * full.w13_pair_stride,
        w13_sf_offset=full.w13_sf_offset + p13 * full.w13_sf_pair_stride,
        w2_offset=full.w2_offset + t2 * 1024, w2_sf_offset=full.w2_sf_offset + t2 * 128)


@dataclass
class LayerShape:
    T: int
    H: int
    I: int
    E: int
    K: int
    tile_m: int
    tp: int = 1


class Buffers:
    """Every device buffer one layer call writes, sized once by moe_workspace_bytes
    and carved from one allocation (nothing is allocated per call, so the calls
    can be captured in a HIP graph)."""

    def __init__(self, shape: LayerShape, device="cuda"):
        s = self.shape = shape
        L = self.layout = N.moe_meta_layout_get(s.T, s.K, s.E, s.tile_m)
        W = self.ws_layout = N.moe_workspace_bytes(s.T, s.K, s.E, s.H, s.I, s.tile_m, s.tp)
        self.workspace = torch.empty((W.total_bytes,), dtype=torch.uint8, device=device)
        rm, I_slice = L.rows_max, s.I // s.tp

        def part(off, dtype, dims):
            n = 1
            for d in dims:
                n *= d
            nbytes = n * torch.empty((), dtype=dtype).element_size()
            return self.workspace[off:off + nbytes].view(dtype).view(dims)

        self.meta = part(W.meta, torch.int32, (L.total_ints,))
        self.meta.fill_(-1)
        self.ids = part(W.topk_ids, torch.int32, (s.T, s.K))
        self.weights = part(W.topk_weights, torch.float32, (s.T, s.K))
        self.a_codes = part(W.a_codes, torch.uint8, (s.T, s.H // 2))
        self.a_sf = part(W.a_sf, torch.uint8, (s.T, s.H // 16))
        if rm > 0:
            self.inter_codes = part(W.inter_codes, torch.uint8, (rm, I_slice // 2))
            self.inter_sf = part(W.inter_sf, torch.uint8, (rm, I_slice // 16))
            self.rows = part(W.rows, torch.int16, (s.tp, rm, s.H))
        else:                       # no routed rows: placeholders the calls never touch
            self.inter_codes = torch.empty((1, I_slice // 2), dtype=torch.uint8, device=device)
            self.inter_sf = torch.empty((1, I_slice // 16), dtype=torch.uint8, device=device)
            self.rows = torch.empty((s.tp, 1, s.H), dtype=torch.int16, device=device)
        self.out = torch.empty((s.T, s.H), dtype=torch.int16, device=device)

    def field(self, name: str, length: int) -> torch.Tensor:
        off = getattr(self.layout, name)
        return self.meta[off:off + length]

    @property
    def exp2perm(self) -> torch.Tensor:
        return self.field("exp2perm", self.shape.T * self.shape.K).view(self.shape.T, self.shape.K)

    @property
    def perm2tok(self) -> torch.Tensor:
        return self.field("perm2tok", self.layout.rows_max)

    def check_sync(self) -> None:
        """Raise if an expert step's bounded wait gave up (meta[sync_status] != 0:
        its rows are not valid) or left a tile, token or work-queue counter
        non-zero. Reads the metadata back, so the caller synchronizes the stream
        first."""
        L = self.layout
        status = int(self.meta[L.sync_status].item())
        counters = self.meta[L.sub_sync:L.sub_sync + 256 * L.subs_max].view(-1, 256)[:, :2]
        tok = self.meta[L.tok_sync:L.tok_sync + 32 * self.shape.T].view(-1, 32)[:, 0]
        queue = self.meta[L.queue:L.queue + 16]
        bad = int((counters != 0).sum().item()) + int((tok != 0).sum().item()) + int((queue != 0).sum().item())
        if status != 0 or bad:
            raise N.MoeError(f"expert step synchronization failed: sync_status={status}, "
                             f"non-zero counters={bad}; the rows and outputs are not valid")


def run_layer(bufs: Buffers, x_bf16, gscale, logits, expert_bias, is_padding, weights: N.Weights,
              norm_weight, gain_center: float, eps: float, weight_before_norm: bool,
              route_scale: float = 1.0, slices: list[N.Weights] | None = None, stream=None,
              fused_route_quant: bool = True, fused_finalize: bool = False, check: bool = False) -> None:
    """route -> quant -> experts (per TP slice) -> finalize, all enqueued on one stream.
    Route and quant run in one launch unless fused_route_quant is False. With
    fused_finalize the last (or only) slice's experts and the finalize run as one
    call (moe_experts_finalize: one launch at decode shapes; one launch fewer,
    which pays when launches are enqueued one by one, while replayed from a
    graph the separate finalize is as fast or faster). With check, waits for the
    stream and raises if an expert step's wait gave up."""
    s = bufs.shape
    if fused_route_quant:
        N.moe_route_quant(logits, expert_bias, is_padding, s.K, route_scale, s.tile_m, 0, s.E,
                          bufs.ids, bufs.weights, bufs.meta, x_bf16, gscale, bufs.a_codes,
                          bufs.a_sf, stream)
    else:
        N.moe_route(logits, expert_bias, is_padding, s.K, route_scale, s.tile_m, 0, s.E,
                    bufs.ids, bufs.weights, bufs.meta, stream)
        N.nvfp4_quant(x_bf16, gscale, bufs.a_codes, bufs.a_sf, stream)
    parts = slices if slices is not None else [weights]
    I_part = s.I // len(parts)
    n_sep = len(parts) - 1 if fused_finalize else len(parts)
    for r in range(n_sep):
        N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, parts[r], s.T, s.K, s.E, s.H, I_part,
                          s.tile_m, bufs.inter_codes, bufs.inter_sf, bufs.rows[r], stream)
    if fused_finalize:
        N.moe_experts_finalize(bufs.a_codes, bufs.a_sf, bufs.meta, parts[-1], s.T, s.K, s.E, s.H, I_part,
                               s.tile_m, bufs.inter_codes, bufs.inter_sf, bufs.rows, len(parts),
                               bufs.rows.stride(0), bufs.weights, norm_weight, gain_center, eps,
                               weight_before_norm, bufs.out, stream)
    else:
        N.moe_finalize(bufs.rows, len(parts), bufs.rows.stride(0), bufs.exp2perm, bufs.weights,
                       norm_weight, gain_center, eps, weight_before_norm, s.T, s.K, s.H, bufs.out, stream)
    if check:
        if stream is None:
            torch.cuda.current_stream().synchronize()
        else:
            stream.synchronize()
        bufs.check_sync()

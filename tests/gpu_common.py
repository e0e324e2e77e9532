"""Helpers of the GPU parity tests: run the HIP path through the C-ABI on a
workload's seeded inputs and bring the results back as numpy arrays."""
from __future__ import annotations

import sys

import numpy as np
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W

DEV = "cuda:0"


def say(*args):
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def sync_counters(meta: np.ndarray, L) -> np.ndarray:
    """The two sync counters of every 16-row tile in a metadata buffer."""
    return meta[L.sub_sync:L.sub_sync + 256 * L.subs_max].reshape(-1, 256)[:, :2]


def upload_weights(inp: W.Inputs) -> N.Weights:
    w13c, w13s, w2c, w2s = dev(inp.w13_codes), dev(inp.w13_sf), dev(inp.w2_codes), dev(inp.w2_sf)
    w = LY.pack_weights(w13c, w13s, w2c, w2s, dev(inp.g1_alphas), dev(inp.g1_scale_c),
                        dev(inp.g2_alphas))
    torch.cuda.synchronize()
    del w13c, w13s, w2c, w2s
    return w


def run_layer(inp: W.Inputs, weights: N.Weights | None = None, tile_m: int | None = None,
              is_padding: np.ndarray | None = None, tp: int = 1, bias: np.ndarray | None = None,
              fill_rows: int | None = None) -> dict:
    wl = inp.wl
    m = wl.tile_m if tile_m is None else tile_m
    if weights is None:
        weights = upload_weights(inp)
    shape = LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, m, tp)
    bufs = LY.Buffers(shape, DEV)
    if fill_rows is not None:
        bufs.rows.fill_(fill_rows)
    slices = None if tp == 1 else [LY.slice_weights(weights, r, tp, wl.H, wl.I) for r in range(tp)]
    say(f"layer {wl.name} T={wl.T} H={wl.H} I={wl.I} E={wl.E} K={wl.K} tile_m={m} tp={tp}")
    LY.run_layer(bufs, dev(inp.x_bf16), dev(inp.a1_gscale), dev(inp.logits),
                 None if bias is None else dev(bias),
                 None if is_padding is None else dev(is_padding.astype(np.uint8)),
                 weights, dev(inp.norm_weight_bf16), wl.gain_center, wl.eps,
                 bool(wl.weight_before_norm), slices=slices)
    torch.cuda.synchronize()
    L = bufs.layout
    meta = host(bufs.meta)
    res = dict(
        a_codes=host(bufs.a_codes), a_sf=host(bufs.a_sf), ids=host(bufs.ids),
        weights=host(bufs.weights), meta=meta, layout=L,
        num_tiles=int(meta[L.num_tiles]), total_rows=int(meta[L.total_rows]),
        offsets=meta[L.expert_offsets:L.expert_offsets + wl.E + 1],
        counts=meta[L.expert_counts:L.expert_counts + wl.E],
        exp2perm=meta[L.exp2perm:L.exp2perm + wl.T * wl.K].reshape(wl.T, wl.K),
        perm2tok=meta[L.perm2tok:L.perm2tok + L.rows_max],
        tile_expert=meta[L.tile_expert:L.tile_expert + L.tiles_max],
        sync_status=int(meta[L.sync_status]), sub_sync=sync_counters(meta, L),
        inter_codes=host(bufs.inter_codes), inter_sf=host(bufs.inter_sf),
        rows=host(bufs.rows), out=host(bufs.out))
    return res

"""A bounded wait of a one-launch expert step that gives up is reported, not
silent (through the C-ABI). One routed tile's ready counter is preset from the
host far below its target, so that the tile's GEMM2 workgroups poll until
their limit (2^20 polls, one to two seconds), set the metadata's sync_status
to 1 and finish; the tile's last GEMM2 workgroup still returns the counters to
0, the layer's check raises, and the next routing clears the status. Every
kernel exits normally."""
import dataclasses

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W

from .gpu_common import DEV, dev, host, say, sync_counters, token_counters, upload_weights

pytestmark = pytest.mark.gpu

UNREACHABLE = -(1 << 30)      # the first 16-row tile's ready counter; its GEMM1 workgroups add I/64


def test_expert_step_wait_gives_up():
    wl = W.WORKLOADS["decode_b8"]              # the one-launch W4A4 kernel
    inp = W.make_inputs(wl)
    w = upload_weights(inp)
    bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m, 1), DEV)
    L = bufs.layout
    logits, x, gs = dev(inp.logits), dev(inp.x_bf16), dev(inp.a1_gscale)

    def route():
        N.moe_route_quant(logits, None, None, wl.K, 1.0, wl.tile_m, 0, wl.E, bufs.ids, bufs.weights, bufs.meta,
                          x, gs, bufs.a_codes, bufs.a_sf)

    def experts():
        N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m,
                          bufs.inter_codes, bufs.inter_sf, bufs.rows[0])

    route()
    bufs.meta[L.sub_sync] = UNREACHABLE
    say("moe_experts_fwd decode_b8 with the first tile's ready counter preset out of reach")
    experts()
    torch.cuda.synchronize()
    meta = host(bufs.meta)
    assert meta[L.sync_status] == 1
    assert not sync_counters(meta, L).any()
    with pytest.raises(N.MoeError):
        bufs.check_sync()
    route()
    experts()
    torch.cuda.synchronize()
    bufs.check_sync()


def test_finalize_in_launch_wait_gives_up():
    """moe_experts_finalize's one-launch form: token 0's finalizer workgroups
    wait on its arrival counter (preset out of reach), give up, and the token's
    last finalizer still returns its counters to 0."""
    wl = W.WORKLOADS["decode_b8"]
    inp = W.make_inputs(wl)
    w = upload_weights(inp)
    bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m, 1), DEV)
    L = bufs.layout
    logits, x, gs, nw = dev(inp.logits), dev(inp.x_bf16), dev(inp.a1_gscale), dev(inp.norm_weight_bf16)

    def run(preset):
        N.moe_route_quant(logits, None, None, wl.K, 1.0, wl.tile_m, 0, wl.E, bufs.ids, bufs.weights, bufs.meta,
                          x, gs, bufs.a_codes, bufs.a_sf)
        if preset:
            bufs.meta[L.tok_sync] = UNREACHABLE
        N.moe_experts_finalize(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m,
                               bufs.inter_codes, bufs.inter_sf, bufs.rows, 1, bufs.rows.stride(0), bufs.weights, nw,
                               wl.gain_center, wl.eps, bool(wl.weight_before_norm), bufs.out)
        torch.cuda.synchronize()
        return host(bufs.meta)

    say("moe_experts_finalize decode_b8 with token 0's arrival counter preset out of reach")
    meta = run(True)
    assert meta[L.sync_status] == 1
    assert not sync_counters(meta, L).any() and not token_counters(meta, L, wl.T).any()
    with pytest.raises(N.MoeError):
        bufs.check_sync()
    meta = run(False)
    assert meta[L.sync_status] == 0
    bufs.check_sync()


def test_tiled_expert_step_wait_gives_up():
    """The persistent register-tiled kernel (many routes per expert): block 0's
    GEMM2 items wait on the same counter word (its first 16-row tile's)."""
    wl = dataclasses.replace(W.WORKLOADS["tiny"], name="tiled_wait", T=256, H=256, I=256, E=8, K=2, tile_m=128,
                             seed=19)                                   # T*K >= 32 E: the tiled kernel
    inp = W.make_inputs(wl, a2_gscale=1.0)                              # only the failure report is checked
    w = upload_weights(inp)
    bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m, 1), DEV)
    L = bufs.layout
    logits, x, gs = dev(inp.logits), dev(inp.x_bf16), dev(inp.a1_gscale)

    def route():
        N.moe_route_quant(logits, None, None, wl.K, 1.0, wl.tile_m, 0, wl.E, bufs.ids, bufs.weights, bufs.meta,
                          x, gs, bufs.a_codes, bufs.a_sf)

    def experts():
        N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m,
                          bufs.inter_codes, bufs.inter_sf, bufs.rows[0])

    route()
    bufs.meta[L.sub_sync] = UNREACHABLE
    say("moe_experts_fwd (tiled) T=256 H=256 I=256 E=8 with block 0's ready counter preset out of reach")
    experts()
    torch.cuda.synchronize()
    meta = host(bufs.meta)
    assert meta[L.sync_status] == 1
    assert not sync_counters(meta, L).any()
    assert not meta[L.queue:L.queue + 16].any()
    with pytest.raises(N.MoeError):
        bufs.check_sync()
    route()
    experts()
    torch.cuda.synchronize()
    bufs.check_sync()


def test_bf16_experts_wait_gives_up():
    wl = dataclasses.replace(W.WORKLOADS["tiny"], name="bf16_wait", T=8, H=256, I=256, E=8, K=2, tile_m=16,
                             seed=17)                                   # H, I % 256 == 0: one launch
    inp = W.make_inputs(wl, a2_gscale=1.0, with_weights=False)
    w13, w2 = W.make_bf16_weights(wl)
    T, H, I, E, K, m = wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m
    L = N.moe_meta_layout_get(T, K, E, m)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    wts = torch.empty((T, K), dtype=torch.float32, device=DEV)
    meta = torch.empty((L.total_ints,), dtype=torch.int32, device=DEV)
    inter = torch.zeros((L.rows_max, I), dtype=torch.int16, device=DEV)
    rows = torch.zeros((L.rows_max, H), dtype=torch.int16, device=DEV)
    xd, w13d, w2d, lg = dev(inp.x_bf16), dev(w13), dev(w2), dev(inp.logits)
    N.moe_route(lg, None, None, K, 1.0, m, 0, E, ids, wts, meta)
    meta[L.sub_sync] = UNREACHABLE
    say("moe_experts_fwd_bf16 with the first tile's ready counter preset out of reach")
    N.moe_experts_fwd_bf16(xd, meta, w13d, w2d, T, K, E, H, I, m, inter, rows)
    torch.cuda.synchronize()
    meta_h = host(meta)
    assert meta_h[L.sync_status] == 1
    assert not sync_counters(meta_h, L).any()
    N.moe_route(lg, None, None, K, 1.0, m, 0, E, ids, wts, meta)
    N.moe_experts_fwd_bf16(xd, meta, w13d, w2d, T, K, E, H, I, m, inter, rows)
    torch.cuda.synchronize()
    meta_h = host(meta)
    assert meta_h[L.sync_status] == 0 and not sync_counters(meta_h, L).any()

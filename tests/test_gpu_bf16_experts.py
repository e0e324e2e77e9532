"""Parity of the BF16 expert layers (moe_route, then moe_experts_fwd_bf16,
through the C-ABI) with the CPU oracle: GEMM2 rows and the finalized output
within rel-L2 1e-2, the bf16 intermediate within rel-L2 1e-3."""
import dataclasses

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W
from oracle import formats as F
from oracle.bf16_experts import experts_bf16
from oracle.finalize import finalize_routes
from oracle.layer import rel_l2
from oracle.routing import route as o_route

from .gpu_common import DEV, dev, host, say, sync_counters

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _compare(wl: W.Workload):
    inp = W.make_inputs(wl, a2_gscale=1.0, with_weights=False)
    w13, w2 = W.make_bf16_weights(wl)
    T, H, I, E, K, m = wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m
    L = N.moe_meta_layout_get(T, K, E, m)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    wts = torch.empty((T, K), dtype=torch.float32, device=DEV)
    meta = torch.empty((L.total_ints,), dtype=torch.int32, device=DEV)
    inter = torch.zeros((L.rows_max, I), dtype=torch.int16, device=DEV)
    rows = torch.full((L.rows_max, H), 0x3F3F, dtype=torch.int16, device=DEV)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    say(f"moe_experts_fwd_bf16 {wl.name} T={T} H={H} I={I} E={E} K={K} m={m}")
    N.moe_route(dev(inp.logits), None, None, K, 1.0, m, 0, E, ids, wts, meta)
    xd, w13d, w2d = dev(inp.x_bf16), dev(w13), dev(w2)
    N.moe_experts_fwd_bf16(xd, meta, w13d, w2d, T, K, E, H, I, m, inter, rows)
    first = host(rows)
    # a second call on the same metadata (the one-launch form's counters are
    # back at 0): the same rows bit for bit
    N.moe_experts_fwd_bf16(xd, meta, w13d, w2d, T, K, E, H, I, m, inter, rows)
    torch.cuda.synchronize()
    assert np.array_equal(host(rows), first)
    e2p_dev = meta[L.exp2perm:L.exp2perm + T * K]
    N.moe_finalize(rows, 1, 0, e2p_dev, wts, dev(inp.norm_weight_bf16), wl.gain_center, wl.eps,
                   bool(wl.weight_before_norm), T, K, H, out)
    torch.cuda.synchronize()
    meta_h, inter_h, rows_h, out_h = host(meta), host(inter), host(rows), host(out)
    assert meta_h[L.sync_status] == 0 and not sync_counters(meta_h, L).any()
    oids, ow = o_route(inp.logits, None, K)
    assert np.array_equal(host(ids), oids)
    p = meta_h[L.exp2perm:L.exp2perm + T * K]
    ref = experts_bf16(inp.x_bf16, np.repeat(np.arange(T), K), oids.reshape(-1), w13, w2)
    h_rel = rel_l2(F.bf16_to_f64(inter_h[p]), F.bf16_to_f64(ref["h"]))
    rows_rel = rel_l2(F.bf16_to_f64(rows_h[p]), F.bf16_to_f64(ref["rows"]))
    want = finalize_routes(ref["rows"].reshape(T, K, -1), np.ones((T, K), bool), ow, inp.norm_weight_bf16,
                           wl.gain_center, wl.eps, bool(wl.weight_before_norm))
    out_rel = rel_l2(F.bf16_to_f64(out_h), F.bf16_to_f64(want))
    say(f"{wl.name} BF16 layer: intermediate rel-L2 {h_rel:.2e}, rows rel-L2 {rows_rel:.2e}, "
        f"finalized rel-L2 {out_rel:.2e}")
    assert h_rel < 1e-3 and rows_rel < TOL and out_rel < TOL
    pad = meta_h[L.perm2tok:L.perm2tok + L.rows_max] < 0
    assert np.all(rows_h[pad] == 0x3F3F)                     # padding rows are not written


@pytest.mark.parametrize("name", ["tiny", "decode_b8"])
def test_bf16_layer_on_workload(name):
    _compare(W.WORKLOADS[name])


@pytest.mark.parametrize("T,H,I,E,K,m", [(6, 320, 192, 8, 2, 16), (5, 384, 256, 8, 3, 32),
                                         (40, 256, 128, 4, 2, 64), (3, 1024, 512, 4, 2, 16),
                                         (7, 512, 192, 8, 2, 16), (40, 512, 256, 4, 2, 64)])
def test_bf16_layer_shapes(T, H, I, E, K, m):
    """Per-wave kernels at pipeline depths 1 (H/64 = 5, I/64 = 3) and 2, and the
    LDS-staged workgroup kernels (K a multiple of 256); tiles of 16 to 64 rows.
    H and I both multiples of 256 take the one-launch form (H = 1024/I = 512,
    and H = 512/I = 256 with 64-row tiles)."""
    wl = dataclasses.replace(W.WORKLOADS["tiny"], name=f"bf16_{T}_{H}_{I}_{E}_{K}_{m}", T=T, H=H, I=I, E=E,
                             K=K, tile_m=m, seed=13)
    _compare(wl)

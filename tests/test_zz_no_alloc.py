"""moe_experts_fwd_noalloc, the expert step for callers that cannot allocate:
its intermediate lives in the library's static device memory. Two calls in a
row on one GPU, the second with a smaller layer, each against
moe_experts_fwd on the same routing and weights: the same rows bit for bit,
padding rows untouched, the tile counters back at zero."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W

from .gpu_common import DEV, dev, host, say, sync_counters, upload_weights

pytestmark = pytest.mark.gpu


def _both(name):
    inp = W.make_inputs(W.WORKLOADS[name])
    wl = inp.wl
    w = upload_weights(inp)
    bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m), DEV)
    N.moe_route_quant(dev(inp.logits), None, None, wl.K, 1.0, wl.tile_m, 0, wl.E, bufs.ids, bufs.weights,
                      bufs.meta, dev(inp.x_bf16), dev(inp.a1_gscale), bufs.a_codes, bufs.a_sf)
    say(f"moe_experts_fwd {name}")
    bufs.rows.fill_(0x3F3F)
    N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m,
                      bufs.inter_codes, bufs.inter_sf, bufs.rows[0])
    torch.cuda.synchronize()
    want = host(bufs.rows[0]).copy()
    rows = torch.full_like(bufs.rows[0], 0x3F3F)
    say(f"moe_experts_fwd_noalloc {name}")
    N.moe_experts_fwd_noalloc(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I, wl.tile_m,
                              rows)
    torch.cuda.synchronize()
    got = host(rows)
    meta = host(bufs.meta)
    L = bufs.layout
    valid = meta[L.perm2tok:L.perm2tok + L.rows_max] >= 0
    assert valid.any()
    assert np.array_equal(got[valid], want[valid]), name
    assert np.all(got[~valid] == 0x3F3F), name
    assert meta[L.sync_status] == 0 and not np.any(sync_counters(meta, L)), name


def test_noalloc_matches_experts_fwd_on_two_calls_in_a_row():
    _both("decode_b8")     # the one-launch kernel, 1024 permuted rows
    _both("tiny")          # smaller: the two-launch kernels, 128 rows

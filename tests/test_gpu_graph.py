"""The whole layer captured once into a HIP graph and replayed: every replay
equals the eager run bit for bit (routing, metadata and its sync counters,
intermediate, rows, output), with eager work and synchronizations between the
replays, and the routing's sync words end at zero after each replay."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import workloads as W

from .gpu_common import DEV, dev, host, queue_words, say, sync_counters, upload_weights

pytestmark = pytest.mark.gpu


def _inputs(name):
    if name in W.WORKLOADS:
        return W.make_inputs(W.WORKLOADS[name])
    # many routes per expert: the register-tiled GEMMs in one launch, GEMM2's
    # workgroups waiting on per-block counters that every replay must find at 0
    from oracle.layer import intermediate_amax
    wl = W.Workload(name, T=256, H=512, I=256, E=4, K=2, tile_m=128, seed=3)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    return W.make_inputs(wl, a2_gscale=float(np.float32(2688.0 / intermediate_amax(probe))))


@pytest.mark.parametrize("name", ["tiny", "decode_b8", "tiled_256"])
def test_graph_replays_equal_eager(name):
    inp = _inputs(name)
    wl = inp.wl
    w = upload_weights(inp)
    bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, wl.tile_m), DEV)
    x, gs, lg, nw = dev(inp.x_bf16), dev(inp.a1_gscale), dev(inp.logits), dev(inp.norm_weight_bf16)

    def step(stream=None):
        LY.run_layer(bufs, x, gs, lg, None, None, w, nw, wl.gain_center, wl.eps, bool(wl.weight_before_norm),
                     stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return {k: host(getattr(bufs, k)).copy() for k in ("ids", "weights", "meta", "rows", "out")}

    step()
    eager = snapshot()
    L = bufs.layout
    assert eager["meta"][L.sync_status] == 0 and not np.any(sync_counters(eager["meta"], L))
    assert not np.any(queue_words(eager["meta"], L))
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    say(f"graph of the {name} layer captured; replaying")
    for it in range(5):
        bufs.out.fill_(0x7F7F)                  # eager work between the replays
        bufs.rows.fill_(0x3F3F)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k, v in eager.items():
            if k == "rows":
                valid = eager["meta"][L.perm2tok:L.perm2tok + L.rows_max] >= 0
                assert np.array_equal(got[k][0][valid], v[0][valid]), (it, k)
            else:
                assert np.array_equal(got[k], v), (it, k)

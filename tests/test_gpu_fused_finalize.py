"""moe_experts_finalize (the expert step and the post-expert finalize in one
call; one launch at decode shapes, where the last GEMM2 workgroup to publish a
token's rows finalizes the token) against moe_experts_fwd followed by
moe_finalize on the same routing and weights: the same rows and the same
output bit for bit, the per-token and per-tile counters back at zero, on the
one-launch shapes (one and two output pairs a GEMM2 wave), the two-launch
shapes, padding tokens, an expert-parallel subset (tokens with no served
route), the expert-TP slices (the last slice's call finalizes all partials),
repeated calls and graph replays."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W
from oracle.layer import intermediate_amax

from .gpu_common import DEV, dev, host, say, sync_counters, token_counters, upload_weights

pytestmark = pytest.mark.gpu


def _inputs(name, shape=None):
    if shape is None:
        return W.make_inputs(W.WORKLOADS[name])
    T, H, I, E, K, m = shape
    wl = W.Workload(name, T=T, H=H, I=I, E=E, K=K, tile_m=m, seed=11)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    return W.make_inputs(wl, a2_gscale=float(np.float32(2688.0 / intermediate_amax(probe))))


class _Case:
    """One routing (moe_route_quant, optionally an expert-parallel subset and
    padding tokens) and the two ways to finish the layer on it."""

    def __init__(self, inp, offset=0, local=None, padding=None, tp=1, weights=None):
        wl = self.wl = inp.wl
        self.inp = inp
        self.local = wl.E if local is None else local
        self.offset = offset
        self.tp = tp
        self.w = upload_weights(inp) if weights is None else weights
        if offset or local is not None:   # the local experts' slice of the weights
            full = self.w
            self.w = N.Weights(**{**full.__dict__,
                                  "w13_offset": full.w13_offset + offset * full.w13_expert_stride,
                                  "w13_sf_offset": full.w13_sf_offset + offset * full.w13_sf_expert_stride,
                                  "w2_offset": full.w2_offset + offset * full.w2_expert_stride,
                                  "w2_sf_offset": full.w2_sf_offset + offset * full.w2_sf_expert_stride,
                                  "g1_alphas": full.g1_alphas[offset:], "g1_scale_c": full.g1_scale_c[offset:],
                                  "g2_alphas": full.g2_alphas[offset:]})
        self.bufs = LY.Buffers(LY.LayerShape(wl.T, wl.H, wl.I, self.local, wl.K, wl.tile_m, tp), DEV)
        self.x, self.gs = dev(inp.x_bf16), dev(inp.a1_gscale)
        self.nw = dev(inp.norm_weight_bf16)
        pad = None if padding is None else dev(padding.astype(np.uint8))
        N.moe_route_quant(dev(inp.logits), None, pad, wl.K, 1.0, wl.tile_m, offset, self.local, self.bufs.ids,
                          self.bufs.weights, self.bufs.meta, self.x, self.gs, self.bufs.a_codes, self.bufs.a_sf)
        self.parts = [self.w] if tp == 1 else [LY.slice_weights(self.w, r, tp, wl.H, wl.I) for r in range(tp)]
        torch.cuda.synchronize()

    def _experts(self, r, stream=None):
        wl, b = self.wl, self.bufs
        N.moe_experts_fwd(b.a_codes, b.a_sf, b.meta, self.parts[r], wl.T, wl.K, self.local, wl.H,
                          wl.I // self.tp, wl.tile_m, b.inter_codes, b.inter_sf, b.rows[r], stream)

    def two_calls(self):
        wl, b = self.wl, self.bufs
        b.rows.fill_(0x3F3F)
        b.out.fill_(0x7F7F)
        for r in range(self.tp):
            self._experts(r)
        N.moe_finalize(b.rows, self.tp, b.rows.stride(0), b.exp2perm, b.weights, self.nw, wl.gain_center, wl.eps,
                       bool(wl.weight_before_norm), wl.T, wl.K, wl.H, b.out)
        return self._snap()

    def fused(self, stream=None, clear=True):
        wl, b = self.wl, self.bufs
        if clear:
            b.rows.fill_(0x3F3F)
            b.out.fill_(0x7F7F)
        for r in range(self.tp - 1):
            self._experts(r, stream)
        N.moe_experts_finalize(b.a_codes, b.a_sf, b.meta, self.parts[-1], wl.T, wl.K, self.local, wl.H,
                               wl.I // self.tp, wl.tile_m, b.inter_codes, b.inter_sf, b.rows, self.tp,
                               b.rows.stride(0), b.weights, self.nw, wl.gain_center, wl.eps,
                               bool(wl.weight_before_norm), b.out, stream)
        return None if stream is not None else self._snap()

    def _snap(self):
        torch.cuda.synchronize()
        b, L = self.bufs, self.bufs.layout
        meta = host(b.meta)
        return dict(rows=host(b.rows).copy(), out=host(b.out).copy(), meta=meta,
                    valid=meta[L.perm2tok:L.perm2tok + L.rows_max] >= 0)

    def check(self, a, f, name):
        L = self.bufs.layout
        for r in range(self.tp):
            assert np.array_equal(a["rows"][r][a["valid"]], f["rows"][r][f["valid"]]), (name, r)
        assert np.array_equal(a["out"], f["out"]), name
        m = f["meta"]
        assert m[L.sync_status] == 0 and not np.any(sync_counters(m, L)), name
        assert not np.any(token_counters(m, L, self.wl.T)), name
        served = (m[L.exp2perm:L.exp2perm + self.wl.T * self.wl.K].reshape(self.wl.T, -1) >= 0).any(axis=1)
        say(f"{name}: out equal bit for bit; {int((~served).sum())} tokens with no served route")
        return served


@pytest.mark.parametrize("name,shape", [("tiny", None), ("decode_b8", None),
                                        ("fin_two_pairs", (6, 512, 256, 8, 2, 16)),
                                        ("fin_one_pair", (9, 1024, 512, 16, 4, 16)),
                                        ("fin_h4096", (5, 4096, 768, 16, 4, 32)),
                                        ("fin_two_launch", (7, 320, 192, 8, 2, 16)),
                                        # 512 tokens at H = 3072, one partial: the finalize takes 8
                                        # columns a thread, which the finalizer in the expert launch
                                        # does not, so the call runs the expert step, then moe_finalize
                                        ("fin_wide", (512, 3072, 256, 64, 2, 16))])
def test_experts_finalize_equals_two_calls(name, shape):
    c = _Case(_inputs(name, shape))
    c.check(c.two_calls(), c.fused(), name)


@pytest.mark.slow
def test_experts_finalize_decode_b64_zipf():
    c = _Case(_inputs("decode_b64_zipf"))
    c.check(c.two_calls(), c.fused(), "decode_b64_zipf")


def test_experts_finalize_padding_and_expert_parallel_subset():
    """Padding tokens and experts outside [16, 32) route nowhere: tokens with no
    served route get a zero output row, as moe_finalize gives them."""
    inp = _inputs("decode_b8")
    pad = np.zeros(inp.wl.T, bool)
    pad[[1, 6]] = True
    c = _Case(inp, padding=pad)
    served = c.check(c.two_calls(), c.fused(), "decode_b8 padded")
    assert not served[1] and not served[6]
    c = _Case(inp, offset=16, local=16)
    a, f = c.two_calls(), c.fused()
    served = c.check(a, f, "decode_b8 experts [16, 32)")
    assert np.all(f["out"][~served] == 0)


@pytest.mark.slow
def test_experts_finalize_expert_tp_slices():
    """The 8 slices of expert_tp8_b32: slices 0-6 by moe_experts_fwd, the last by
    moe_experts_finalize, which finalizes the fp32 sum of all 8 partials."""
    inp = _inputs("expert_tp8_b32")
    c = _Case(inp, tp=inp.wl.tp)
    c.check(c.two_calls(), c.fused(), "expert_tp8_b32 slices")


def test_experts_finalize_repeated_calls_and_graph_replays():
    inp = _inputs("decode_b8")
    c = _Case(inp)
    want = c.two_calls()
    for it in range(4):
        c.check(want, c.fused(), f"decode_b8 call {it}")
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        c.fused(stream=torch.cuda.current_stream(), clear=False)
    torch.cuda.synchronize()
    for it in range(5):
        c.bufs.out.fill_(0x7F7F)        # eager work between the replays
        c.bufs.rows.fill_(0x3F3F)
        torch.cuda.synchronize()
        g.replay()
        c.check(want, c._snap(), f"decode_b8 replay {it}")

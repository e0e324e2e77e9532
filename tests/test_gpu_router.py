"""Parity of the router logits (moe_router_logits) and the full routing chain
(moe_router_route), through the C-ABI, with the CPU oracle."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W
from oracle.permute import permute as o_permute
from oracle.router import router_logits
from oracle.routing import route as o_route

from .gpu_common import DEV, dev, host, say

pytestmark = pytest.mark.gpu


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp32 ulps (same-sign finite values)."""
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _gpu_logits(x: np.ndarray, w: np.ndarray, pad: int = 0) -> np.ndarray:
    T, D = x.shape
    xs = np.zeros((T, D + pad), np.float32)
    xs[:, :D] = x
    xt = dev(xs)[:, :D]
    out = torch.full((T, w.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    say(f"moe_router_logits T={T} D={D} E={w.shape[0]} stride={D + pad}")
    N.moe_router_logits(xt, dev(w), out)
    torch.cuda.synchronize()
    return host(out)


def _check_logits(got: np.ndarray, want: np.ndarray, name: str):
    """Each logit is the rounded exact product; the kernel's fp64 sums may move
    a value that lies within a few fp64 ulps of an fp32 rounding boundary by one
    fp32 ulp, and nothing else."""
    d = _ulps(got, want)
    say(f"{name}: {int(np.count_nonzero(d))} of {d.size} logits differ from the oracle, max {int(d.max())} ulp")
    assert d.max() <= 1 and np.count_nonzero(d) <= max(1, d.size // 10000)


@pytest.mark.parametrize("name", ["tiny", "decode_b8", "decode_b64_zipf", "expert_tp8_b32"])
def test_router_logits_on_workload(name):
    wl = W.WORKLOADS[name]
    x, w = W.make_router_inputs(wl)
    _check_logits(_gpu_logits(x, w), router_logits(x, w), name)


def test_router_logits_prefill_sampled():
    """4096 tokens on the GPU; the oracle computes 24 sampled tokens."""
    wl = W.WORKLOADS["prefill_t4096"]
    x, w = W.make_router_inputs(wl)
    got = _gpu_logits(x, w)
    tok = np.concatenate([np.random.default_rng(0).choice(wl.T, 22, replace=False), [0, wl.T - 1]])
    _check_logits(got[tok], router_logits(x[tok], w), "prefill_t4096 sampled")


@pytest.mark.parametrize("T,D,E,pad", [(1, 4, 1, 0), (7, 60, 3, 4), (8, 256, 64, 0), (9, 2052, 257, 8),
                                       (33, 4096, 128, 0), (5, 6144, 16, 4), (40, 512, 7, 4),
                                       (100, 1000, 130, 4), (256, 2052, 65, 0), (300, 1000, 100, 4),
                                       (257, 64, 64, 0), (320, 4100, 130, 0)])
def test_router_logits_shapes(T, D, E, pad):
    """Up to 256 tokens the kernel of 8-token groups whose waves split D (1, 2
    or 4 experts a workgroup as T grows: partial token groups, expert groups
    and 256-column rounds), beyond it the LDS-tiled one (partial token, expert
    and column tiles)."""
    rng = np.random.default_rng(T * D + E)
    x = rng.standard_normal((T, D)).astype(np.float32)
    w = (rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    _check_logits(_gpu_logits(x, w, pad), router_logits(x, w), f"T={T} D={D} E={E}")


@pytest.mark.parametrize("name", ["tiny", "decode_b8", "decode_b64_zipf"])
def test_router_route_chain(name):
    """moe_router_route = moe_router_logits + moe_route, bit for bit; its ids,
    weights and metadata are the oracle's routing of the logits it produced
    (both sides take the top-k decision from the same fp32 logits), and the
    logits match the oracle's."""
    wl = W.WORKLOADS[name]
    x, w = W.make_router_inputs(wl)
    T, E, K, m = wl.T, wl.E, wl.K, wl.tile_m
    rng = np.random.default_rng(2)
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    L = N.moe_meta_layout_get(T, K, E, m)

    def bufs():
        return (torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV),
                torch.full((T, K), 12345, dtype=torch.int32, device=DEV),
                torch.full((T, K), 7.0, dtype=torch.float32, device=DEV),
                torch.full((L.total_ints,), -777, dtype=torch.int32, device=DEV))

    xt, wt, bt = dev(x), dev(w), dev(bias)
    lg, ids, wts, meta = bufs()
    say(f"moe_router_route {name} T={T} D={wl.H} E={E} K={K}")
    N.moe_router_route(xt, wt, bt, None, K, 1.0, m, 0, E, lg, ids, wts, meta)
    lg2, ids2, wts2, meta2 = bufs()
    N.moe_router_logits(xt, wt, lg2)
    N.moe_route(lg2, bt, None, K, 1.0, m, 0, E, ids2, wts2, meta2)
    torch.cuda.synchronize()
    for a, b in ((lg, lg2), (ids, ids2), (wts, wts2), (meta, meta2)):
        assert np.array_equal(host(a).view(np.uint32) if a.dtype == torch.float32 else host(a),
                              host(b).view(np.uint32) if b.dtype == torch.float32 else host(b))
    glog = host(lg)
    _check_logits(glog, router_logits(x, w), name)
    oids, ow = o_route(glog, bias, K)
    assert np.array_equal(host(ids), oids)
    assert np.array_equal(host(wts).view(np.uint32), ow.view(np.uint32))
    om = o_permute(oids, 0, E, m)
    hm = host(meta)
    assert np.array_equal(hm[L.exp2perm:L.exp2perm + T * K], om["exp2perm"].reshape(-1))
    assert np.array_equal(hm[L.perm2tok:L.perm2tok + L.rows_max], om["perm2tok"])


def test_router_zero_tokens():
    x = torch.zeros((0, 64), dtype=torch.float32, device=DEV)
    w = torch.zeros((8, 64), dtype=torch.float32, device=DEV)
    out = torch.zeros((0, 8), dtype=torch.float32, device=DEV)
    N.moe_router_logits(x, w, out)
    torch.cuda.synchronize()

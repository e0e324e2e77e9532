"""Parity of nvfp4_norm_quant (the pre-expert RMSNorm inside the NVFP4 input
quantizer, through the C-ABI) with the CPU oracle: codes and block scales bit
for bit."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W
from oracle import formats as F
from oracle.norm_quant import norm_quant

from .gpu_common import DEV, dev, host, say

pytestmark = pytest.mark.gpu


def _gpu_norm_quant(xb: np.ndarray, w, center: float, eps: float, gscale: float, pad: int = 0):
    T, H = xb.shape
    xs = np.zeros((T, H + pad), np.uint16)
    xs[:, :H] = xb
    x = dev(xs)[:, :H]
    codes = torch.full((T, H // 2), 0xAB, dtype=torch.uint8, device=DEV)
    sf = torch.full((T, H // 16), 0xCD, dtype=torch.uint8, device=DEV)
    g = torch.tensor([gscale], dtype=torch.float32, device=DEV)
    say(f"nvfp4_norm_quant T={T} H={H} stride={H + pad} weight={'yes' if w is not None else 'no'} "
        f"centre={center} eps={eps} gscale={gscale}")
    N.nvfp4_norm_quant(x, None if w is None else dev(w), center, eps, g, codes, sf)
    torch.cuda.synchronize()
    return host(codes), host(sf)


def _check(xb, w, center, eps, gscale, pad=0):
    c, s = _gpu_norm_quant(xb, w, center, eps, gscale, pad)
    oc, os_ = norm_quant(xb, w, center, eps, gscale)
    bad_s = int(np.count_nonzero(s != os_))
    bad_c = int(np.count_nonzero(c != oc))
    assert bad_s == 0 and bad_c == 0, f"{bad_s} scales and {bad_c} code bytes differ"


def _weight(H, seed):
    rng = np.random.default_rng(seed)
    return F.f32_to_bf16(rng.uniform(-0.1, 0.1, H).astype(np.float32))


@pytest.mark.parametrize("name", W.ORDER)
def test_norm_quant_bit_exact_on_workload_activations(name):
    """Each workload's activations (its token count and width; prefill with its
    1% outliers) with a zero-centred weight around 1, eps 1e-6."""
    inp = W.make_inputs(W.WORKLOADS[name])
    _check(inp.x_bf16, _weight(inp.wl.H, 1), 1.0, 1e-6, float(inp.a1_gscale[0]))


@pytest.mark.parametrize("T,H,pad", [(1, 16, 0), (3, 48, 8), (5, 1024, 0), (2, 1040, 16), (4, 2048, 0),
                                     (7, 4096, 8), (3, 4112, 0), (2, 8192, 0), (3, 16384, 8), (9, 2000, 0)])
def test_norm_quant_shapes(T, H, pad):
    """Rows held in registers (H up to 4096: 1, 2 or 4 blocks a lane, partial
    last rounds) and rows read twice (wider), padded row strides, partial last
    workgroups."""
    rng = np.random.default_rng(T * H)
    xb = F.f32_to_bf16((rng.standard_normal((T, H)) * 3).astype(np.float32))
    _check(xb, _weight(H, H), 1.0, 1e-6, 1.0, pad)
    _check(xb, None, 0.0, 1e-5, 2.5, pad)


def test_norm_quant_edge_rows():
    """A zero row, one spike, values near the top and bottom of the bf16 range
    (fp32 mean square overflowing to inf or underflowing to 0), constant rows,
    and mixed magnitudes in one row; several global scales."""
    H = 256
    rng = np.random.default_rng(9)
    rows = [np.zeros(H), np.eye(1, H, 17)[0] * 1000.0, np.full(H, 3.0e38), np.full(H, -1.0e-38),
            np.full(H, 1.0e-20), np.where(np.arange(H) % 2, 1e30, 1e-30), np.full(H, 1.0),
            rng.standard_normal(H) * np.logspace(-8, 8, H)]
    xb = F.f32_to_bf16(np.array(rows, dtype=np.float32))
    for g in (1.0, 0.37, 448.0, 1e-3):
        _check(xb, _weight(H, 4), 1.0, 1e-6, g)
        _check(xb, None, 0.0, 0.5, g)


def test_norm_quant_zero_tokens():
    x = torch.zeros((0, 64), dtype=torch.int16, device=DEV)
    codes = torch.zeros((0, 32), dtype=torch.uint8, device=DEV)
    sf = torch.zeros((0, 4), dtype=torch.uint8, device=DEV)
    N.nvfp4_norm_quant(x, None, 1.0, 1e-6, torch.ones(1, device=DEV), codes, sf)
    torch.cuda.synchronize()

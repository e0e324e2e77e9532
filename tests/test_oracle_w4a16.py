"""Pins of the oracle's W4A16 expert variant (oracle/w4a16.py): the scalar
folding against the unfolded layer, GEMM1 against the exact W4A4 GEMM1 on
NVFP4-representable inputs, rational brute force on a tiny case."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle.experts import gemm1 as w4a4_gemm1, silu64
from oracle.quant import dequantize_nvfp4
from oracle.w4a16 import experts_w4a16, fold_scalars


def _weights(E, H, I, seed):
    rng = np.random.default_rng(seed)
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w13s = rng.integers(0x30, 0x41, (E, 2 * I, H // 16), dtype=np.uint8)
    w2s = rng.integers(0x30, 0x41, (E, H, I // 16), dtype=np.uint8)
    return w13c, w13s, w2c, w2s


def _x(T, H, seed):
    return F.f32_to_bf16(np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32))


def test_folding_equals_the_unfolded_layer():
    """Without the bf16 rounding of h, GEMM1 with the gate's scale on both
    halves and GEMM2 with w2 * up / gate give the rows of the layer with each
    half's own scale: h_true = silu(g * gate) * (u * up), rows = (h_true . w2) * w2_gs.
    An inverted ratio would be off by (up / gate)^2."""
    E, H, I, T = 3, 64, 32, 5
    w13c, w13s, w2c, w2s = _weights(E, H, I, 1)
    rng = np.random.default_rng(2)
    gate, up, w2g = (rng.uniform(0.5, 1.5, E).astype(np.float32) for _ in range(3))
    x = _x(T, H, 3)
    tokens = np.array([0, 1, 2, 3, 4, 0])
    experts = np.array([0, 1, 2, 0, 1, 2])
    s13, s2 = fold_scalars(gate, up, w2g)
    got = experts_w4a16(x, tokens, experts, w13c, w13s, w2c, w2s, s13, s2, round_h=False)["rows64"]
    want = np.zeros_like(got)
    for r, (t, e) in enumerate(zip(tokens, experts)):
        w13 = dequantize_nvfp4(w13c[e], w13s[e])
        acc = w13 @ F.bf16_to_f64(x[t])
        h = silu64(acc[:I] * float(gate[e])) * (acc[I:] * float(up[e]))
        want[r] = (dequantize_nvfp4(w2c[e], w2s[e]) @ h) * float(w2g[e])
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-9 * np.abs(want).max())
    assert np.array_equal(s13, gate)


def test_gemm1_equals_the_w4a4_gemm1_on_nvfp4_inputs():
    """Activations that are NVFP4 values (e2m1 x e4m3, exact in bf16): GEMM1 of
    the W4A16 path equals the exact W4A4 GEMM1 on their codes and scales."""
    E, H, I, T = 2, 128, 64, 4
    w13c, w13s, w2c, w2s = _weights(E, H, I, 4)
    rng = np.random.default_rng(5)
    ac = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    asf = rng.integers(0x30, 0x41, (T, H // 16), dtype=np.uint8)
    a = dequantize_nvfp4(ac, asf)
    xb = F.f64_to_bf16(a)
    assert np.array_equal(F.bf16_to_f64(xb), a)
    tokens = np.array([0, 1, 2, 3, 1])
    experts = np.array([0, 0, 1, 1, 1])
    ones = np.ones(E, np.float32)
    got = experts_w4a16(xb, tokens, experts, w13c, w13s, w2c, w2s, ones, ones)["acc1"]
    want = w4a4_gemm1(ac, asf, tokens, experts, w13c, w13s)
    assert np.array_equal(got, want)


def test_tiny_case_against_rationals():
    """One route, H = 32, I = 16: acc1 and acc2 equal their exact rational sums,
    h is the bf16 nearest to silu(g) * u, and the row is the bf16 nearest to
    acc2 * s2."""
    E, H, I = 1, 32, 16
    w13c, w13s, w2c, w2s = _weights(E, H, I, 6)
    x = _x(1, H, 7)
    s13 = np.array([0.75], np.float32)
    s2 = np.array([1.25], np.float32)
    out = experts_w4a16(x, [0], [0], w13c, w13s, w2c, w2s, s13, s2)
    xv = [Fraction(v) for v in F.bf16_to_f64(x[0])]
    w13 = dequantize_nvfp4(w13c[0], w13s[0])
    acc1 = [sum(xv[k] * Fraction(w13[n, k]) for k in range(H)) for n in range(2 * I)]
    assert [Fraction(v) for v in out["acc1"][0]] == acc1
    g = np.array([float(acc1[n] * Fraction(0.75)) for n in range(I)])
    u = np.array([float(acc1[I + n] * Fraction(0.75)) for n in range(I)])
    h64 = g / (1.0 + np.exp(-g)) * u
    hb = F.bf16_to_f64(out["h"][0])
    step = np.spacing(np.abs(hb).astype(np.float32)).astype(np.float64) * 2 ** 16   # bf16 ulp
    assert np.all(np.abs(hb - h64) <= 0.5 * step + 1e-300)
    w2 = dequantize_nvfp4(w2c[0], w2s[0])
    acc2 = [sum(Fraction(hb[i]) * Fraction(w2[n, i]) for i in range(I)) for n in range(H)]
    assert [Fraction(v) for v in out["acc2"][0]] == acc2
    assert np.array_equal(out["rows"][0], F.f64_to_bf16(np.array([float(v * Fraction(1.25)) for v in acc2])))


@pytest.mark.parametrize("seed", [0, 1])
def test_fold_scalars_in_fp32(seed):
    rng = np.random.default_rng(seed)
    gate, up, w2 = (rng.uniform(0.5, 1.5, 8).astype(np.float32) for _ in range(3))
    s13, s2 = fold_scalars(gate, up, w2)
    assert s2.dtype == np.float32 and np.array_equal(s2, w2 * (up / gate))
    np.testing.assert_allclose(s2, w2.astype(np.float64) * up / gate, rtol=2.5e-7)

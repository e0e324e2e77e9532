"""Pins of the oracle's BF16 expert layers (oracle/bf16_experts.py): integer
products, and the W4A16 oracle on weights that are NVFP4 values."""
import numpy as np

from oracle import formats as F
from oracle.bf16_experts import experts_bf16
from oracle.experts import silu64
from oracle.quant import dequantize_nvfp4
from oracle.w4a16 import experts_w4a16


def test_integer_weights_give_integer_products():
    """Small-integer activations and weights (E, H, I, T all different): acc1 is
    the integer matrix product (gate rows first in w13), h the bf16 SwiGLU of
    it, acc2 the exact product of h with w2 (to fp64 rounding)."""
    rng = np.random.default_rng(1)
    E, H, I, T = 3, 40, 8, 5
    x = rng.integers(-3, 4, (T, H)).astype(np.float64)
    w13 = rng.integers(-2, 3, (E, 2 * I, H)).astype(np.float64)
    w2 = rng.integers(-2, 3, (E, H, I)).astype(np.float64)
    tokens = np.array([0, 1, 2, 3, 4, 2])
    experts = np.array([2, 0, 1, 1, 0, 2])
    out = experts_bf16(F.f64_to_bf16(x), tokens, experts, F.f64_to_bf16(w13), F.f64_to_bf16(w2))
    for r, (t, e) in enumerate(zip(tokens, experts)):
        acc = w13[e].astype(np.int64) @ x[t].astype(np.int64)
        assert np.array_equal(out["acc1"][r], acc)
        h = F.bf16_to_f64(F.f64_to_bf16(silu64(acc[:I].astype(np.float64)) * acc[I:]))
        assert np.array_equal(F.bf16_to_f64(out["h"][r]), h)
        from fractions import Fraction
        exact = [float(sum(Fraction(int(w2[e, n, i])) * Fraction(h[i]) for i in range(I))) for n in range(H)]
        np.testing.assert_allclose(out["acc2"][r], exact, rtol=1e-15, atol=1e-300)


def test_nvfp4_valued_weights_reduce_to_w4a16():
    """bf16 weights equal to dequantized NVFP4 weights (exact in bf16) and unit
    global scales: the BF16 layer is the W4A16 variant, bit for bit."""
    rng = np.random.default_rng(2)
    E, H, I, T = 2, 64, 32, 4
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = rng.integers(0x30, 0x41, (E, 2 * I, H // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(0x30, 0x41, (E, H, I // 16), dtype=np.uint8)
    w13 = np.stack([F.f64_to_bf16(dequantize_nvfp4(w13c[e], w13s[e])) for e in range(E)])
    w2 = np.stack([F.f64_to_bf16(dequantize_nvfp4(w2c[e], w2s[e])) for e in range(E)])
    x = F.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    tokens, experts = np.array([0, 1, 2, 3, 0]), np.array([0, 1, 1, 0, 1])
    a = experts_bf16(x, tokens, experts, w13, w2)
    ones = np.ones(E, np.float32)
    b = experts_w4a16(x, tokens, experts, w13c, w13s, w2c, w2s, ones, ones)
    for k in ("acc1", "h", "acc2", "rows"):
        assert np.array_equal(a[k], b[k]), k

"""Pins of the oracle's pre-expert RMSNorm + NVFP4 quantizer (oracle/norm_quant.py)
against closed forms, invariants and the textbook RMSNorm."""
import numpy as np
import pytest

from oracle import formats as F
from oracle.norm_quant import gamma, norm_quant, norm_scale, normalize
from oracle.quant import quantize_nvfp4


def _bf16(a) -> np.ndarray:
    return F.f32_to_bf16(np.asarray(a, dtype=np.float32))


def _rows(T, H, seed, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    if outliers:
        x = np.where(rng.random((T, H)) < 0.01, x * 20, x).astype(np.float32)
    return _bf16(x)


@pytest.mark.parametrize("H,eps", [(64, 1e-6), (2048, 1e-6), (4096, 1e-5), (320, 0.0)])
def test_normalize_is_textbook_rmsnorm(H, eps):
    """No weight and a zero gain centre: y = x / sqrt(mean(x^2) + eps), the
    textbook RMSNorm, here in fp64 through numpy's vector norm (eps inside the
    root), to within the four fp32 roundings of the definition."""
    xb = _rows(6, H, seed=H, outliers=True)
    y = normalize(xb, None, 0.0, eps)
    x = F.bf16_to_f64(xb)
    ref = x / np.sqrt(np.linalg.norm(x, axis=1, keepdims=True) ** 2 / H + np.float32(eps))
    np.testing.assert_allclose(y, ref, rtol=4e-7, atol=0)


def test_eps_sits_inside_the_root():
    """Rows of mean square near eps: eps changes the scale by sqrt(2), as only
    eps inside the square root does."""
    x = np.full((1, 64), 1e-3, dtype=np.float32)
    xb = _bf16(x)
    xv = float(F.bf16_to_f64(xb)[0, 0])
    eps = xv * xv                                   # mean square == eps
    r = float(norm_scale(xb, eps)[0])
    assert r == pytest.approx(1.0 / np.sqrt(2.0 * xv * xv), rel=3e-7)


def test_weight_applies_after_the_norm():
    """gamma multiplies the normalized row: y(w) = gamma * y(no weight, centre 0)
    elementwise, to one rounding; a weight applied before the norm would also
    rescale each row by rms(x)/rms(gamma*x)."""
    H = 1024
    xb = _rows(4, H, seed=7)
    rng = np.random.default_rng(8)
    w = _bf16(rng.uniform(-0.5, 0.5, H))              # zero-centred weight
    yw = normalize(xb, w, 1.0, 1e-6)
    y1 = normalize(xb, None, 0.0, 1e-6)
    g = gamma(w, 1.0, H)
    np.testing.assert_allclose(yw, y1 * g, rtol=1.2e-7, atol=0)
    assert np.array_equal(g, (F.bf16_to_f64(w) + 1.0).astype(np.float32))
    assert np.array_equal(gamma(None, 0.0, H), np.ones(H, np.float32))


def test_unit_mean_square_reduces_to_the_plain_quantizer():
    """Rows whose mean square is exactly 1 (values 2, 1/2 and 1 in the ratio
    4 : 16 : 12, random signs and order), eps 0 and gamma 1: r = 1 exactly, so
    the fused op equals the plain quantizer on the same values."""
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(8):
        v = np.array([2.0] * 4 + [0.5] * 16 + [1.0] * 12) * rng.choice([-1.0, 1.0], 32)
        rows.append(rng.permutation(v))
    x = np.concatenate([np.array(rows)] * 4, axis=1).astype(np.float32)   # H = 128
    xb = _bf16(x)
    assert np.all(norm_scale(xb, 0.0) == 1.0)
    for g in (1.0, 0.37, 6.0):
        c, s = norm_quant(xb, None, 0.0, 0.0, g)
        oc, os_ = quantize_nvfp4(x, g)
        assert np.array_equal(c, oc) and np.array_equal(s, os_)


def test_constant_row_closed_form():
    """A constant row of +-1 (eps 0, gamma 1, gscale 1): y = +-1, the block
    scale is e4m3(1/6) = 0.171875 (code 0x23) and every code is the e2m1
    magnitude 6 (x / 0.171875 = 5.82 rounds to 6): nibble 0x7, or 0xF negative."""
    x = np.ones((2, 32), np.float32)
    x[1] *= -1
    c, s = norm_quant(_bf16(x), None, 0.0, 0.0, 1.0)
    assert np.all(s == 0x23)
    assert np.all(c[0] == 0x77) and np.all(c[1] == 0xFF)


def test_zero_row_gives_zero_codes_and_scales():
    x = np.zeros((1, 64), np.uint16)
    c, s = norm_quant(x, None, 1.0, 1e-6, 1.0)
    assert not np.any(c) and not np.any(s)


@pytest.mark.parametrize("k", [-20, -3, 1, 9])
def test_power_of_two_scaling_leaves_the_output_unchanged(k):
    """With eps 0, scaling a row by 2^k scales its squares by 2^2k exactly, its
    mean square, root and reciprocal by exact powers of two: y, the codes and
    the scales are unchanged (bit for bit)."""
    xb = _rows(5, 512, seed=abs(k) + 1, outliers=True)
    x = F.bf16_to_f64(xb)
    xs = _bf16(x * 2.0 ** k)
    assert np.array_equal(F.bf16_to_f64(xs), x * 2.0 ** k)            # exact in bf16
    w = _bf16(np.random.default_rng(3).uniform(-0.1, 0.1, 512))
    a = norm_quant(xb, w, 1.0, 0.0, 2.5)
    b = norm_quant(xs, w, 1.0, 0.0, 2.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fsum_is_the_exact_sum():
    """The oracle's sum of squares is the correctly rounded exact sum: for
    bf16 inputs whose squares span few binades it equals an exact integer sum."""
    xb = _rows(3, 256, seed=5)
    bits = xb.astype(np.int64)
    # every bf16 here is normal: value = m * 2^(e - 134), m in [128, 255]
    e = (bits >> 7) & 0xFF
    m = (bits & 0x7F) | 0x80
    assert np.all(e > 0)
    emin = int(e.min())
    exact = [sum(int(mm) ** 2 << (2 * (int(ee) - emin)) for mm, ee in zip(m[t], e[t])) for t in range(3)]
    from fractions import Fraction
    for t in range(3):
        s = Fraction(exact[t]) * Fraction(2) ** (2 * (emin - 134))
        ms = np.float32(float(s / 256))
        want = np.float32(np.float32(1.0) / np.float32(np.sqrt(np.float32(ms + np.float32(1e-6)))))
        assert norm_scale(xb[t:t + 1], 1e-6)[0] == want

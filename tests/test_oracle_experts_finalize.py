"""Pins of the oracle's grouped GEMMs (exact-rational triple loop, integer
special case), gated activation, GEMM2 rounding, finalize (textbook RMSNorm,
invariants), converted layout (per-element address formula) and the expert-TP
slice identity (exact)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import experts as ex
from oracle import formats as F
from oracle import layout as LY
from oracle.finalize import finalize, finalize_routes, sum_partials
from oracle.layer import rel_l2
from oracle.quant import quantize_nvfp4


def _rand_nvfp4(rng, rows, n):
    codes = rng.integers(0, 256, (rows, n // 2), dtype=np.uint8)
    sf = rng.integers(0x28, 0x48, (rows, n // 16), dtype=np.uint8)
    return codes, sf


# ------------------------------------------------------------------ GEMMs
def test_gemm1_against_rational_triple_loop():
    rng = np.random.default_rng(0)
    T, H, I, E = 3, 64, 32, 2
    a_codes, a_sf = _rand_nvfp4(rng, T, H)
    w_codes = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w_sf = rng.integers(0x01, 0x7E, (E, 2 * I, H // 16), dtype=np.uint8)
    tokens = np.array([0, 1, 2, 2])
    experts = np.array([1, 0, 0, 1])
    acc = ex.gemm1(a_codes, a_sf, tokens, experts, w_codes, w_sf)
    A = F.unpack_nibbles(a_codes)
    Wn = F.unpack_nibbles(w_codes)
    e2m1 = [Fraction(v) for v in F.E2M1]
    e4m3 = [Fraction(v) if np.isfinite(v) else None for v in F.E4M3]
    for r, (t, e) in enumerate(zip(tokens, experts)):
        for n in range(2 * I):
            tot = Fraction(0)
            for h in range(H):
                tot += (e2m1[A[t, h]] * e4m3[a_sf[t, h // 16]]
                        * e2m1[Wn[e, n, h]] * e4m3[w_sf[e, n, h // 16]])
            assert Fraction(acc[r, n]) == tot


def test_gemm_unit_scales_is_integer_matmul():
    rng = np.random.default_rng(1)
    M, N, K = 5, 48, 256
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    w_codes = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    one = np.full((M, K // 16), 0x38, np.uint8)               # e4m3 1.0
    wone = np.full((1, N, K // 16), 0x38, np.uint8)
    acc = ex.gemm1(a_codes, one, np.arange(M), np.zeros(M, np.int64), w_codes, wone)
    half_units = np.rint(F.E2M1 * 2).astype(np.int64)          # e2m1 values in units of 1/2
    ai = half_units[F.unpack_nibbles(a_codes)]
    wi = half_units[F.unpack_nibbles(w_codes[0])]
    assert np.array_equal(acc * 4, (ai @ wi.T).astype(np.float64))


def test_gemm2_against_rational_triple_loop():
    """GEMM2 of routes whose experts interleave (2, 0, 1, 0, 2): every route's
    intermediate row against its own expert's w2, summed as rationals. A row
    gathered from the wrong route or the wrong expert's weights fails it."""
    rng = np.random.default_rng(8)
    R, H, I, E = 5, 32, 64, 3
    h_codes, h_sf = _rand_nvfp4(rng, R, I)
    w_codes = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w_sf = rng.integers(0x01, 0x7E, (E, H, I // 16), dtype=np.uint8)
    experts = np.array([2, 0, 1, 0, 2])
    acc = ex.gemm2(h_codes, h_sf, experts, w_codes, w_sf)
    Hn = F.unpack_nibbles(h_codes)
    Wn = F.unpack_nibbles(w_codes)
    e2m1 = [Fraction(v) for v in F.E2M1]
    e4m3 = [Fraction(v) if np.isfinite(v) else None for v in F.E4M3]
    for r, e in enumerate(experts):
        for n in range(H):
            tot = Fraction(0)
            for i in range(I):
                tot += (e2m1[Hn[r, i]] * e4m3[h_sf[r, i // 16]]
                        * e2m1[Wn[e, n, i]] * e4m3[w_sf[e, n, i // 16]])
            assert Fraction(acc[r, n]) == tot


def test_gemm2_unit_scales_is_integer_matmul_per_expert():
    """Unit scales: each route's row is the integer product of its own
    intermediate codes with its expert's w2 codes (experts interleaved)."""
    rng = np.random.default_rng(9)
    R, N, K, E = 7, 40, 128, 3
    h_codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    w_codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    one = np.full((R, K // 16), 0x38, np.uint8)
    wone = np.full((E, N, K // 16), 0x38, np.uint8)
    experts = np.array([1, 2, 0, 1, 0, 2, 1])
    acc = ex.gemm2(h_codes, one, experts, w_codes, wone)
    half_units = np.rint(F.E2M1 * 2).astype(np.int64)
    hi = half_units[F.unpack_nibbles(h_codes)]
    for r, e in enumerate(experts):
        wi = half_units[F.unpack_nibbles(w_codes[e])]
        assert np.array_equal(acc[r] * 4, (wi @ hi[r]).astype(np.float64))


def test_experts_forward_gathers_tokens_per_route():
    """Routes whose tokens differ from their index and repeat (3, 0, 3, 1):
    each route's rows equal those of the same (token, expert) run alone."""
    rng = np.random.default_rng(10)
    T, H, I, E = 4, 128, 64, 2
    a_codes, a_sf = _rand_nvfp4(rng, T, H)
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = rng.integers(0x30, 0x41, (E, 2 * I, H // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(0x30, 0x41, (E, H, I // 16), dtype=np.uint8)
    g1a = rng.uniform(0.5, 1.5, E).astype(np.float32)
    g1c = (rng.uniform(0.5, 1.5, E) * 0.05).astype(np.float32)
    g2a = rng.uniform(0.5, 1.5, E).astype(np.float32)
    tokens = np.array([3, 0, 3, 1])
    experts = np.array([1, 0, 0, 1])
    fw = ex.experts_forward(a_codes, a_sf, tokens, experts, w13c, w13s, w2c, w2s, g1a, g1c, g2a)
    for r, (t, e) in enumerate(zip(tokens, experts)):
        one = ex.experts_forward(a_codes[t:t + 1], a_sf[t:t + 1], [0], [0], w13c[e:e + 1],
                                 w13s[e:e + 1], w2c[e:e + 1], w2s[e:e + 1], g1a[e:e + 1],
                                 g1c[e:e + 1], g2a[e:e + 1])
        assert np.array_equal(fw["acc1"][r], one["acc1"][0])
        assert np.array_equal(fw["h_codes"][r], one["h_codes"][0])
        assert np.array_equal(fw["acc2"][r], one["acc2"][0])
        assert np.array_equal(fw["rows"][r], one["rows"][0])
    # the two routes of token 3 go to different experts: different rows
    assert not np.array_equal(fw["acc1"][0], fw["acc1"][2])


def test_exactness_guard_raises():
    a = np.full((1, 4096), 2688.0)
    with pytest.raises(ArithmeticError):
        ex._exact_matmul(a, a)


def test_silu_against_library_sigmoid():
    g = np.linspace(-50, 50, 10001)
    want = g * torch.sigmoid(torch.from_numpy(g)).numpy()
    assert np.allclose(ex.silu64(g), want, rtol=1e-14, atol=1e-300)
    assert ex.silu64(np.array([0.0]))[0] == 0.0


def test_swiglu_requant_sides():
    # gate side scaled by g1_alphas before the SiLU, up side by g1_scale_c after
    acc = np.array([[2.0, -1.0, 3.0, 4.0] * 8 + [1.0, 2.0, 0.5, -2.0] * 8])   # I = 32
    h, codes, sf = ex.swiglu_requant(acc, np.array([0]), np.array([0.5], np.float32),
                                     np.array([2.0], np.float32))
    g = acc[0, :32] * 0.5
    u = acc[0, 32:] * 2.0
    want = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(h[0], want)
    c2, s2 = quantize_nvfp4(want[None, :], 1.0)
    assert np.array_equal(codes, c2) and np.array_equal(sf, s2)


def test_gemm2_rows_round_once():
    acc2 = np.array([[1.0 + 2.0 ** -8 + 2.0 ** -40, -3.0]])
    rows = ex.gemm2_rows_bf16(acc2, np.array([0]), np.array([1.0], np.float32))
    assert F.bf16_to_f64(rows).tolist() == [[1.0 + 2.0 ** -7, -3.0]]


# ------------------------------------------------------------------ finalize
def test_finalize_k1_is_textbook_rmsnorm():
    rng = np.random.default_rng(2)
    T, H = 6, 128
    rows = F.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32) * 3)
    gamma = rng.uniform(0.9, 1.1, H).astype(np.float32)
    w_bf16 = F.f32_to_bf16(gamma)                               # gain centre 0
    out = finalize(rows, np.arange(T)[:, None], np.ones((T, 1), np.float32), w_bf16, 0.0, 1e-6, False)
    x = torch.from_numpy(F.bf16_to_f64(rows))
    g = torch.from_numpy(F.bf16_to_f64(w_bf16))
    ref = torch.nn.functional.rms_norm(x, (H,), g, eps=float(np.float32(1e-6))).numpy()
    assert np.array_equal(out, F.f64_to_bf16(ref.astype(np.float32).astype(np.float64)))


def test_finalize_weight_before_norm_closed_form():
    """A unit row under a gain alternating 2, 0: with the weight applied before
    the norm, z = (2, 0, 2, 0, ...) has mean square 2 and y = sqrt(2) on the even
    columns; with the weight after it, r / rms(r) = 1 and y = 2. Normalizing by
    the rms of r instead of that of gamma * r gives 2, not sqrt(2)."""
    H = 64
    rows = F.f32_to_bf16(np.ones((1, H), np.float32))
    gamma = np.tile(np.array([2.0, 0.0], np.float32), H // 2)
    w_bf16 = F.f32_to_bf16(gamma)                                   # gain centre 0
    e2p = np.zeros((1, 1), np.int64)
    wk = np.ones((1, 1), np.float32)
    before = F.bf16_to_f64(finalize(rows, e2p, wk, w_bf16, 0.0, 0.0, True))[0]
    after = F.bf16_to_f64(finalize(rows, e2p, wk, w_bf16, 0.0, 0.0, False))[0]
    assert np.all(before[1::2] == 0) and np.all(after[1::2] == 0)
    assert np.all(before[0::2] == F.bf16_to_f64(F.f64_to_bf16(np.array([np.sqrt(2.0)])))[0])
    assert np.all(after[0::2] == 2.0)


def test_finalize_weight_before_norm_is_textbook_rmsnorm_of_the_weighted_row():
    """With the weight before the norm, K = 1 and w = 1, the output is the
    library RMSNorm (no weight) of gamma * r, gamma = stored weight + centre."""
    rng = np.random.default_rng(12)
    T, H = 5, 256
    rows = F.f32_to_bf16((rng.standard_normal((T, H)) * 7).astype(np.float32))
    nw = F.f32_to_bf16(rng.uniform(-0.5, 0.5, H).astype(np.float32))
    out = finalize(rows, np.arange(T)[:, None], np.ones((T, 1), np.float32), nw, 1.0, 1e-6, True)
    gamma = (F.bf16_to_f64(nw).astype(np.float32) + np.float32(1.0)).astype(np.float64)
    z = torch.from_numpy(F.bf16_to_f64(rows) * gamma)
    ref = torch.nn.functional.rms_norm(z, (H,), None, eps=float(np.float32(1e-6))).numpy()
    assert np.array_equal(out, F.f64_to_bf16(ref.astype(np.float32).astype(np.float64)))


def test_finalize_weight_before_norm_scale_invariant_and_masking():
    rng = np.random.default_rng(3)
    T, K, H = 4, 3, 64
    rows = F.f32_to_bf16(rng.standard_normal((T * K, H)).astype(np.float32))
    rows2 = F.f32_to_bf16(F.bf16_to_f64(rows) * 4.0)            # exact power-of-two scaling
    e2p = np.arange(T * K).reshape(T, K).astype(np.int64)
    e2p[1, 2] = -1                                              # not served: reads zero
    w = rng.uniform(0, 1, (T, K)).astype(np.float32)
    nw = F.f32_to_bf16(rng.uniform(-0.1, 0.1, H).astype(np.float32))
    o1 = F.bf16_to_f64(finalize(rows, e2p, w, nw, 1.0, 1e-6, True))
    o2 = F.bf16_to_f64(finalize(rows2, e2p, w, nw, 1.0, 1e-6, True))
    assert rel_l2(o2, o1) < 1e-5
    e2p_b = e2p.copy()
    e2p_b[1, 2] = 5
    w_b = w.copy()
    w_b[1, 2] = 0.0
    assert np.array_equal(finalize(rows, e2p, w, nw, 1.0, 1e-6, True),
                          finalize(rows, e2p_b, w_b, nw, 1.0, 1e-6, True))
    zero = np.zeros_like(rows)
    assert np.all(F.bf16_to_f64(finalize(zero, e2p, w, nw, 1.0, 1e-6, True)) == 0)


def test_partials_sum_in_fp32_then_bf16():
    a = F.f32_to_bf16(np.array([[1.0, 256.0]], np.float32))
    b = F.f32_to_bf16(np.array([[2.0 ** -9, 1.0]], np.float32))
    s = sum_partials([a, b, b])
    # fp32 sum 1 + 2^-8 is the bf16 midpoint -> ties to even 1.0; 258 is a bf16 value
    assert F.bf16_to_f64(s).tolist() == [[1.0, 258.0]]


def test_rel_l2_closed_form():
    b = np.random.default_rng(4).standard_normal(1000)
    assert rel_l2(b * 1.01, b) == pytest.approx(0.01, rel=1e-9)


# ------------------------------------------------------------------ layout
def test_converted_layout_addresses():
    rng = np.random.default_rng(5)
    E, N, K = 2, 64, 128
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 256, (E, N, K // 16), dtype=np.uint8)
    cc = LY.convert_codes(codes).reshape(E, -1)
    cs = LY.convert_scales(sf).reshape(E, -1)
    nib = F.unpack_nibbles(codes)
    tiles_k = K // 64
    for e in range(E):
        for row in range(N):
            p, h, n = row // 32, (row % 32) // 16, row % 16
            for k in range(K):
                t, q, i = k // 64, (k % 64) // 16, k % 16
                byte = (p * tiles_k + t) * 1024 + ((q * 16 + n) * 2 + h) * 8 + i // 2
                v = (cc[e, byte] >> (4 * (i & 1))) & 15
                assert v == nib[e, row, k]
            for b in range(K // 16):
                t, q = b // 4, b % 4
                byte = (p * tiles_k + t) * 128 + (q * 16 + n) * 2 + h
                assert cs[e, byte] == sf[e, row, b]


def test_gate_up_interleave_rows():
    E, I = 1, 64
    rows = np.arange(2 * I).reshape(E, 2 * I)
    conv = LY.interleave_gate_up(rows)[0]
    for rho in range(2 * I):
        c, w = rho // 32, rho % 32
        want = 16 * c + w if w < 16 else I + 16 * c + (w - 16)
        assert conv[rho] == want


@pytest.mark.parametrize("tp", [2, 4])
def test_tp_slices_are_byte_views_of_converted_layout(tp):
    rng = np.random.default_rng(6)
    E, H, I = 3, 128, 64 * tp
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = rng.integers(0, 256, (E, 2 * I, H // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(0, 256, (E, H, I // 16), dtype=np.uint8)
    full13 = LY.convert_w13(w13c, w13s)
    full2 = LY.convert_w2(w2c, w2s)
    for r in range(tp):
        sl13 = LY.convert_w13(*LY.logical_slice_w13(w13c, w13s, r, tp))
        sl2 = LY.convert_w2(*LY.logical_slice_w2(w2c, w2s, r, tp))
        assert np.array_equal(sl13[0], LY.view_slice_w13(full13[0], r, tp))
        assert np.array_equal(sl13[1], LY.view_slice_w13(full13[1], r, tp))
        assert np.array_equal(sl2[0], LY.view_slice_w2(full2[0], r, tp))
        assert np.array_equal(sl2[1], LY.view_slice_w2(full2[1], r, tp))
        # views, not copies
        assert np.shares_memory(LY.view_slice_w2(full2[0], r, tp), full2[0])


def test_tp_slice_sum_is_exact():
    """Summing the K-partial GEMM2 accumulators of tp intermediate slices gives
    the full-width accumulator exactly (before g2_alphas); each slice's
    intermediate is the matching columns of the full intermediate."""
    rng = np.random.default_rng(7)
    T, H, I, E, tp = 6, 128, 256, 3, 4
    a_codes, a_sf = _rand_nvfp4(rng, T, H)
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = rng.integers(0x30, 0x41, (E, 2 * I, H // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(0x30, 0x41, (E, H, I // 16), dtype=np.uint8)
    g1a = rng.uniform(0.5, 1.5, E).astype(np.float32)
    g1c = (rng.uniform(0.5, 1.5, E) * 0.01).astype(np.float32)
    g2a = rng.uniform(0.5, 1.5, E).astype(np.float32)
    tokens = np.repeat(np.arange(T), 2)
    experts = np.tile(np.arange(2), T) % E
    full = ex.experts_forward(a_codes, a_sf, tokens, experts, w13c, w13s, w2c, w2s, g1a, g1c, g2a)
    s = I // tp
    total = np.zeros_like(full["acc2"])
    for r in range(tp):
        c13, s13 = LY.logical_slice_w13(w13c, w13s, r, tp)
        c2, s2 = LY.logical_slice_w2(w2c, w2s, r, tp)
        part = ex.experts_forward(a_codes, a_sf, tokens, experts, c13, s13, c2, s2, g1a, g1c, g2a)
        assert np.array_equal(part["h_codes"], full["h_codes"][:, r * s // 2:(r + 1) * s // 2])
        assert np.array_equal(part["h_sf"], full["h_sf"][:, r * s // 16:(r + 1) * s // 16])
        total += part["acc2"]
    assert np.array_equal(total, full["acc2"])

"""Pins of the oracle's NVFP4 quantizer, sigmoid, top-k routing and permutation
metadata against closed forms, error bounds, exhaustive brute force and
invariants."""
import itertools

import numpy as np
import pytest

from oracle import formats as F
from oracle.permute import permute, rows_max
from oracle.quant import dequantize_nvfp4, quantize_nvfp4
from oracle.routing import exp32, route, sigmoid32


# ------------------------------------------------------------------ quantizer
def test_quant_exact_grid_roundtrip():
    # A block whose values are e2m1 grid points times 2^k and whose amax is 6 * 2^k
    # has scale 2^k exactly; the codes reproduce the values exactly.
    rng = np.random.default_rng(0)
    for k in range(-6, 7):
        codes = rng.integers(0, 16, (8, 64)).astype(np.uint8)
        codes[:, ::16] = 7                                   # amax 6 in every block
        x = (F.decode_e2m1(codes) * 2.0 ** k).astype(np.float32)
        c, s = quantize_nvfp4(x, 1.0)
        assert np.all(F.decode_e4m3(s) == 2.0 ** k)
        assert np.array_equal(dequantize_nvfp4(c, s), x.astype(np.float64))


def test_quant_error_bound_and_layout():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((32, 256)) * np.exp2(rng.integers(-8, 8, (32, 1)))).astype(np.float32)
    g = np.float32(3.0)
    c, s = quantize_nvfp4(x, float(g))
    assert c.shape == (32, 128) and s.shape == (32, 16)
    d = F.decode_e4m3(s)
    deq = dequantize_nvfp4(c, s).reshape(32, 16, 16)
    xs = x.astype(np.float64).reshape(32, 16, 16) * float(g)
    # the scale is the e4m3 rounding of amax * g / 6: within half a step of the e4m3
    # grid (relative 1/16 for normal values, 2^-10 absolute in the subnormal range)
    amax = np.abs(xs).max(-1)
    half_step = np.maximum(amax / 6 / 16, 2.0 ** -10)
    assert np.all(np.abs(d - amax / 6) <= half_step * (1 + 1e-6))
    # each element is within half a grid step of the scaled value, measured in
    # units of the block scale, except where the scaled value exceeds 6 (saturated)
    u = xs / d[..., None]
    step = np.where(np.abs(u) < 2, 0.5, np.where(np.abs(u) < 4, 1.0, 2.0))
    err = np.abs(u - deq / d[..., None])
    sat = np.abs(u) > 6
    assert np.all(err[~sat] <= step[~sat] / 2 * (1 + 1e-5))
    assert np.all(np.abs(deq[sat] / d[..., None].repeat(16, -1)[sat]) == 6)


def test_quant_special_blocks():
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 16] = 5.0                                   # single spike
    x[0, 32:48] = -1e-20                             # scale underflows to 0 -> zero codes
    x[0, 48:64] = np.float32(2.0 ** -9 * 6)          # smallest subnormal scale
    c, s = quantize_nvfp4(x, 1.0)
    assert s[0, 0] == 0 and np.all(c[0, 0:8] == 0)   # all-zero block
    assert F.decode_e4m3(s[0, 1]) == pytest.approx(5.0 / 6, rel=1 / 16)
    assert s[0, 2] == 0 and np.all(c[0, 16:24] == 0)
    assert s[0, 3] == 0x01 and np.all(F.unpack_nibbles(c[0, 24:32]) == 7)


def test_quant_saturating_scale():
    x = np.full((1, 16), 3000.0, dtype=np.float32)   # amax / 6 = 500 > 448
    c, s = quantize_nvfp4(x, 1.0)
    assert s[0, 0] == 0x7E
    assert np.all(F.unpack_nibbles(c) == 7)          # 3000 / 448 = 6.7 -> saturates to 6


# ------------------------------------------------------------------ sigmoid
def _ulp_err(got32, ref64):
    ref32 = ref64.astype(np.float32)
    ulp = np.abs(np.nextafter(ref32, np.float32(np.inf)) - ref32).astype(np.float64)
    return np.abs(got32.astype(np.float64) - ref64) / ulp


def test_exp32_accuracy():
    x = np.linspace(-20, 80, 2000001).astype(np.float32)
    e = _ulp_err(exp32(x), np.exp(x.astype(np.float64)))
    assert e.max() <= 2.0, e.max()


def test_sigmoid32_accuracy_and_special_values():
    bits = np.arange(0, 2 ** 32, 509, dtype=np.uint64).astype(np.uint32).view(np.float32)
    l = bits[np.isfinite(bits) & (np.abs(bits) <= 30)]
    ref = 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    assert _ulp_err(sigmoid32(l), ref).max() <= 3.0
    assert sigmoid32(np.array([0.0], np.float32))[0] == 0.5
    assert sigmoid32(np.array([100.0], np.float32))[0] == 1.0
    assert sigmoid32(np.array([-100.0], np.float32))[0] == 0.0
    wide = np.linspace(-79, 79, 100001).astype(np.float32)
    refw = 1.0 / (1.0 + np.exp(-wide.astype(np.float64)))
    assert _ulp_err(sigmoid32(wide), refw).max() <= 3.0


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_topk_exhaustive_with_ties(K):
    """Every key vector over a 4-value alphabet (ties everywhere) for E = 8,
    against a textbook sort by (-key, index)."""
    E = 8
    # Every token takes one of 4^8 logit vectors over a 4-letter alphabet, so the
    # sigmoid keys tie in every possible pattern.
    idx = np.array(list(itertools.product(range(4), repeat=E)), dtype=np.int64)
    lvals = np.array([-3.0, -1.0, 1.0, 3.0], dtype=np.float32)
    logits = lvals[idx]
    ids, w = route(logits, None, K)
    s = sigmoid32(lvals)
    T = idx.shape[0]
    for t in range(T):
        keys = s[idx[t]]
        want = sorted(range(E), key=lambda e: (-float(keys[e]), e))[:K]
        if ids[t].tolist() != want:
            raise AssertionError((idx[t].tolist(), ids[t].tolist(), want))


def test_topk_bias_selects_only():
    logits = np.array([[0.0, 0.1, -0.1, 0.2]], dtype=np.float32)
    bias = np.array([0.0, 0.0, 1.0, 0.0], dtype=np.float32)
    ids, w = route(logits, bias, 2)
    assert ids.tolist() == [[2, 3]]
    s = sigmoid32(logits[0])
    want = (s[[2, 3]] / np.float32(np.float32(s[2] + s[3]) + np.float32(1e-15))).astype(np.float32)
    assert np.array_equal(w[0], want)
    ids2, w2 = route(logits, bias, 2, bias_in_weights=True)
    assert ids2.tolist() == [[2, 3]] and not np.array_equal(w2, w)


def test_route_weights_renormalize_and_padding():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((300, 64)).astype(np.float32)
    pad = np.zeros(300, dtype=bool)
    pad[[3, 77]] = True
    ids, w = route(logits, None, 8, 1.0, pad)
    assert np.all(ids[pad] == -1) and np.all(w[pad] == 0)
    ok = ~pad
    assert np.all(np.abs(w[ok].astype(np.float64).sum(1) - 1) < 8 * 2 ** -23)
    s = sigmoid32(logits)
    chosen = np.take_along_axis(s[ok], ids[ok].astype(np.int64), 1).astype(np.float64)
    assert np.allclose(w[ok], chosen / chosen.sum(1, keepdims=True), rtol=4e-7, atol=0)
    # K = 1: the single weight is s / (s + 1e-15), i.e. 1 for any s >> 1e-15
    ids1, w1 = route(logits, None, 1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(ids1[:, 0], np.argmax(s, 1))


def test_route_scale_multiplies():
    logits = np.random.default_rng(4).standard_normal((10, 16)).astype(np.float32)
    _, w = route(logits, None, 4, 1.0)
    _, w2 = route(logits, None, 4, 2.5)
    assert np.array_equal(w2, (w * np.float32(2.5)).astype(np.float32))


# ------------------------------------------------------------------ permutation
def _check_meta(ids, off, nloc, m):
    meta = permute(ids, off, nloc, m)
    T, K = ids.shape
    flat = ids.reshape(-1)
    loc = flat - off
    valid = (flat >= 0) & (loc >= 0) & (loc < nloc)
    e2p = meta["exp2perm"].reshape(-1)
    p2t = meta["perm2tok"]
    assert np.all(e2p[~valid] == -1)
    pos = e2p[valid]
    assert len(set(pos.tolist())) == pos.size                      # injective
    assert np.array_equal(np.sort(np.nonzero(p2t >= 0)[0]), np.sort(pos))  # onto non-pad rows
    assert np.all(p2t[pos] == np.nonzero(valid)[0] // K)
    # library sort as a second construction: stable sort of routes by expert
    order = np.argsort(loc[valid], kind="stable")
    r_sorted = np.nonzero(valid)[0][order]
    e_sorted = loc[valid][order]
    expect = np.empty(r_sorted.size, dtype=np.int64)
    for e in np.unique(e_sorted):
        sel = e_sorted == e
        expect[sel] = meta["offsets"][e] + np.arange(sel.sum())
    assert np.array_equal(e2p[r_sorted], expect)
    assert np.all(meta["offsets"] % m == 0)
    assert meta["total_rows"] == meta["offsets"][-1] <= rows_max(T, K, nloc, m) == meta["rows_max"]
    for tile in range(meta["num_tiles"]):
        e = meta["tile_expert"][tile]
        assert meta["offsets"][e] <= tile * m < meta["offsets"][e + 1]
    assert np.all(meta["tile_expert"][meta["num_tiles"]:] == -1)
    return meta


def test_permute_invariants_random():
    rng = np.random.default_rng(3)
    for T, E, K, m in [(4, 8, 2, 16), (8, 64, 8, 16), (64, 128, 8, 16), (300, 16, 4, 128), (1, 4, 4, 1)]:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        _check_meta(ids, 0, E, m)


def test_permute_ep_and_padding_tokens():
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(32)[:4] for _ in range(50)]).astype(np.int32)
    ids[7] = -1
    meta = _check_meta(ids, 8, 8, 16)
    assert np.all(meta["exp2perm"][7] == -1)


def test_rows_max_bound_is_reached():
    # E_local experts with one route each, the rest on expert 0: the bound is tight.
    T, K, E, m = 16, 4, 8, 16
    R = T * K
    ids = np.zeros((T, K), dtype=np.int32)
    flat = ids.reshape(-1)
    flat[:E] = np.arange(E)
    # distinct experts per token are not needed by the metadata itself
    meta = permute(flat.reshape(T, K), 0, E, m)
    # expert 0 holds 1 + (R - E) routes, every other expert one
    assert meta["total_rows"] == (-(-(R - E + 1) // m) + E - 1) * m
    assert meta["total_rows"] <= rows_max(T, K, E, m)
    # exactly tight when (R - E) is a multiple of m
    T2 = 6
    ids2 = np.zeros((T2, K), dtype=np.int32).reshape(-1)
    ids2[:E] = np.arange(E)
    meta2 = permute(ids2.reshape(T2, K), 0, E, m)
    assert meta2["total_rows"] == rows_max(T2, K, E, m)

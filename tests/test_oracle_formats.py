"""Pins of the oracle's codecs against exact-rational brute force and against
torch's own float8_e4m3fn / bfloat16 conversions (library routines)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

# The e2m1 magnitudes as the OCP microscaling format lists them.
E2M1_LISTED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_is_the_listed_format():
    assert list(F.E2M1[:8]) == E2M1_LISTED
    assert list(F.E2M1[8:]) == [-v for v in E2M1_LISTED]


def _brute_e2m1(v: float) -> int:
    """Nearest e2m1 magnitude by exact rational distance, ties to the even code,
    saturating at 6; sign bit from the input's sign."""
    if np.isnan(v):
        return 0
    sign = 8 if np.signbit(v) else 0
    a = abs(v)
    if a >= 6.0:
        return sign | 7
    fa = Fraction(a)
    best = None
    for code, g in enumerate(E2M1_LISTED):
        d = abs(fa - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return sign | best[1]


def _breakpoint_values(points):
    out = []
    for p in points:
        x = np.float32(p)
        for _ in range(4):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(9):
            out.append(x)
            x = np.nextafter(x, np.float32(np.inf))
    vals = np.array(out, dtype=np.float32)
    return np.concatenate([vals, -vals])


def test_e2m1_encode_named_cases():
    cases = [(0.0, 0), (-0.0, 8), (0.25, 0), (0.2500001, 1), (0.75, 2), (1.25, 2), (1.75, 4),
             (2.5, 4), (3.5, 6), (5.0, 6), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e30, 7),
             (-1e30, 15), (-0.75, 10), (float("inf"), 7), (float("-inf"), 15), (-1e-30, 8)]
    for v, want in cases:
        assert int(F.encode_e2m1(np.array([v], dtype=np.float32))[0]) == want, v
    assert int(F.encode_e2m1(np.array([np.nan], dtype=np.float32))[0]) == 0


def test_e2m1_encode_against_rational_brute_force():
    bf16_all = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf16_all = bf16_all[~np.isnan(bf16_all)]
    mids = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rand = rand[~np.isnan(rand)]
    near = (rng.uniform(-7, 7, 50000)).astype(np.float32)
    vals = np.concatenate([bf16_all, _breakpoint_values(mids), rand, near])
    got = F.encode_e2m1(vals)
    want = np.array([_brute_e2m1(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_monotone_on_sorted_sweep():
    x = np.sort(np.random.default_rng(3).uniform(0, 8, 200000).astype(np.float32))
    mags = F.decode_e2m1(F.encode_e2m1(x))
    assert np.all(np.diff(mags) >= 0)


def test_nibble_packing_low_first():
    codes = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    assert F.pack_nibbles(codes).tolist() == [[0x21, 0x43]]
    assert F.unpack_nibbles(F.pack_nibbles(codes)).tolist() == codes.tolist()


def test_e4m3_table_matches_torch_float8_e4m3fn():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.E4M3
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(both_nan, np.isnan(ref))
    assert np.array_equal(ref[~both_nan], mine[~both_nan])
    assert F.E4M3[0x7E] == 448.0 and F.E4M3[0x01] == 2.0 ** -9 and F.E4M3[0x08] == 2.0 ** -6


def _torch_e4m3(vals: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    bf16_all = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    rand_bits = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    pts = [F.E4M3[c] for c in range(127)]
    mids = [(F.E4M3[c] + F.E4M3[c + 1]) / 2 for c in range(126)]
    vals = np.concatenate([bf16_all, rand_bits, _breakpoint_values(pts + mids),
                           rng.uniform(-500, 500, 100000).astype(np.float32)])
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    got = F.encode_e4m3(vals)
    want = _torch_e4m3(vals)
    # torch keeps the sign of zero like the oracle does
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_saturates_and_nan():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e9, np.inf, -1e9, -np.inf, np.nan],
                 dtype=np.float32)
    assert F.encode_e4m3(v).tolist() == [0x7E] * 7 + [0xFE, 0xFE, 0x7F]


def test_bf16_from_fp32_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 2 ** 32, 500000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f32_to_bf16(x)
    assert np.array_equal(got, want)


def _brute_bf16(x: float) -> float:
    """Nearest bf16 by exact rational search over the two candidates."""
    f = Fraction(x)
    b = np.float32(x).view(np.uint32) & np.uint32(0xFFFF0000)
    lo = np.array([b], dtype=np.uint32).view(np.float32)[0]
    cands = []
    for d in (-1, 0, 1, 2):
        bits = np.uint32(int(b) + d * 0x10000)
        v = np.array([bits], dtype=np.uint32).view(np.float32)[0]
        if np.isfinite(v):
            cands.append((abs(Fraction(float(v)) - f), (int(bits) >> 16) & 1, float(v)))
    cands.sort(key=lambda c: (c[0], c[1]))
    return cands[0][2]


def test_bf16_from_fp64_rounds_once():
    # Just above the midpoint between 1 and 1 + 2^-7: one rounding gives 1 + 2^-7,
    # rounding through fp32 first would land on the midpoint and tie to 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([x])))[0] == 1.0 + 2.0 ** -7
    rng = np.random.default_rng(9)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    got = F.bf16_to_f64(F.f64_to_bf16(vals))
    want = np.array([_brute_bf16(float(v)) for v in vals])
    assert np.array_equal(got, want)

"""Number formats of NVFP4: e2m1 element codes, e4m3 block scales, bf16 rows.

Test infrastructure (see ``oracle/__init__``).

NVFP4 stores two e2m1 codes per byte and one e4m3 ("float8_e4m3fn") scale per
16 elements (the expert_tp page, "StockNvfp4": uint8 [.., H/2] codes and e4m3
[.., H/16] scales). The pages do not state the nibble order, the rounding mode
or the overflow behaviour; the readings taken here are:

  * element 2j sits in the low nibble of byte j, 2j+1 in the high nibble;
  * encoding rounds to the nearest representable value, ties to the code with
    an even last mantissa bit, and saturates to the largest finite magnitude
    (6 for e2m1, 448 for e4m3) instead of producing inf/NaN;
  * the sign bit of an encoded zero is the sign bit of the input;
  * NaN encodes to e2m1 +0 and to the e4m3 NaN code 0x7F.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------- e2m1
def _e2m1_table() -> np.ndarray:
    """The 16 e2m1 values from the format: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    vals = np.zeros(16, dtype=np.float64)
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        vals[code] = -mag if s else mag
    return vals


E2M1 = _e2m1_table()
E2M1_MAX = 6.0


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    return E2M1[np.asarray(nibbles, dtype=np.int64) & 15]


def _nearest_even(mags: np.ndarray, table_vals: np.ndarray, table_codes: np.ndarray,
                  vmax: float) -> np.ndarray:
    """Index into a sorted table of non-negative values: nearest value, ties to the
    code with an even last bit, saturating at vmax. ``mags`` is float64, >= 0."""
    mags = np.minimum(mags, vmax)
    hi = np.clip(np.searchsorted(table_vals, mags, side="left"), 1, len(table_vals) - 1)
    lo = hi - 1
    d_lo = mags - table_vals[lo]
    d_hi = table_vals[hi] - mags
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((table_codes[hi] & 1) == 0))
    return np.where(pick_hi, hi, lo)


_E2M1_POS_VALS = E2M1[:8].copy()           # 0, .5, 1, 1.5, 2, 3, 4, 6 (increasing)
_E2M1_POS_CODES = np.arange(8, dtype=np.int64)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e2m1 nibbles (uint8 0..15)."""
    v = np.asarray(v, dtype=np.float32)
    nan = np.isnan(v)
    mags = np.abs(v.astype(np.float64))
    mags = np.where(nan, 0.0, mags)
    idx = _nearest_even(mags, _E2M1_POS_VALS, _E2M1_POS_CODES, E2M1_MAX)
    sign = np.where(nan, 0, np.signbit(v).astype(np.int64))
    return (_E2M1_POS_CODES[idx] | (sign << 3)).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] nibbles -> [..., n] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------- e4m3
def _e4m3_table() -> np.ndarray:
    """OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; subnormals m * 2^-9."""
    vals = np.zeros(256, dtype=np.float64)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            vals[code] = np.nan
            continue
        mag = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -mag if s else mag
    return vals


E4M3 = _e4m3_table()
E4M3_MAX = 448.0
_E4M3_POS_VALS = E4M3[:127].copy()          # codes 0x00 .. 0x7E, increasing
_E4M3_POS_CODES = np.arange(127, dtype=np.int64)


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    return E4M3[np.asarray(b, dtype=np.int64) & 255]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3fn bytes (round to nearest even, saturate to +-448)."""
    v = np.asarray(v, dtype=np.float32)
    nan = np.isnan(v)
    mags = np.where(nan, 0.0, np.abs(v.astype(np.float64)))
    idx = _nearest_even(mags, _E4M3_POS_VALS, _E4M3_POS_CODES, E4M3_MAX)
    code = _E4M3_POS_CODES[idx] | (np.signbit(v).astype(np.int64) << 7)
    return np.where(nan, 0x7F, code).astype(np.uint8)


# --------------------------------------------------------------------- bf16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits, 8 exponent bits), to
    nearest, ties to even, directly from the fp64 value (no fp32 step).
    Overflow goes to inf, as round-to-nearest does."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                                  # xf = m * 2^e, 0.5 <= |m| < 1
    q_exp = np.maximum(e - 8, -133)                      # quantum: 8 significant bits, subnormal floor
    r = np.ldexp(np.rint(np.ldexp(xf, -q_exp)), q_exp)   # rint = round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[finite] = r
    out[~finite] = x[~finite]
    f32 = out.astype(np.float32)                         # exact: every value is a bf16 value
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    return f64_to_bf16(np.asarray(x, dtype=np.float32).astype(np.float64))

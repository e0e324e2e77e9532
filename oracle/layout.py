"""The converted NVFP4 weight layout and its expert-TP slice views.
Test infrastructure (see ``oracle/__init__``); the GPU path has its own
converter, and tests compare the two byte for byte.

The pages need one property of the layout the kernels read (the expert_tp
page, module docstring, "slice_views", "unsupported"): a tensor-parallel slice
of the converted weights is, byte for byte, the converted layout of the slice,
so each slice is a view. For w13 [E, 2I, H/2] the gated interleave puts slice
r's 2I' rows on contiguous rows [2rI', 2(r+1)I'); for w2 [E, H, I/2] slice r is
columns [rI'/2, (r+1)I'/2) of every row, and the block scales keep whole
k-tiles of I/64. The vendor's own shuffle is not on the pages; this layout is
this project's own, chosen for the MI355X kernels, and keeps that property
whenever I' % 64 == 0.

Layout, per expert, of an NVFP4 matrix with N rows and K columns
(N % 16 == 0, K % 64 == 0):
  * codes: [N/16 row groups][K/64 k-tiles][512 bytes]. Element (n, k) of a tile
    (n < 16, k < 64) is nibble (j & 1) of byte ((q * 16 + n) * 2 + s) * 4 + j / 2
    with s = k / 32, q = (k % 32) / 8, j = k % 8 (low nibble for even j);
  * scales: [N/16][K/64][64 bytes]. Block b = k / 16 of row n is byte
    ((b % 2) * 16 + n) * 2 + b / 2;
  * w13 only: converted row 32c + w is logical row 16c + w for w < 16 (gate)
    and I + 16c + (w - 16) for w >= 16 (up), so every 32 rows hold the gate
    and up rows of the same 16 intermediates.
"""
from __future__ import annotations

import numpy as np

from .formats import pack_nibbles, unpack_nibbles

ROWS = 16        # rows per row group
KTILE = 64       # elements per k-tile


def interleave_gate_up(rows: np.ndarray) -> np.ndarray:
    """[E, 2I, ...] logical (gate, then up) -> [E, 2I, ...] converted row order."""
    E, n2 = rows.shape[:2]
    I = n2 // 2
    gate = rows[:, :I].reshape((E, I // ROWS, ROWS) + rows.shape[2:])
    up = rows[:, I:].reshape((E, I // ROWS, ROWS) + rows.shape[2:])
    return np.stack([gate, up], axis=2).reshape(rows.shape)


def convert_codes(codes: np.ndarray) -> np.ndarray:
    """[E, N, K/2] bytes -> [E, N/16, K/64, 512] bytes."""
    E, N, half = codes.shape
    K = half * 2
    nib = unpack_nibbles(codes).reshape(E, N // ROWS, ROWS, K // KTILE, 2, 4, 8)
    #                                   e  g         n     t           s  q  j
    t = nib.transpose(0, 1, 3, 5, 2, 4, 6).reshape(E, N // ROWS, K // KTILE, 1024)
    return pack_nibbles(t)


def convert_scales(sf: np.ndarray) -> np.ndarray:
    """[E, N, K/16] bytes -> [E, N/16, K/64, 64] bytes."""
    E, N, nb = sf.shape
    K = nb * 16
    s = sf.reshape(E, N // ROWS, ROWS, K // KTILE, 2, 2)
    #                e  g         n     t          b/2 b%2
    return np.ascontiguousarray(s.transpose(0, 1, 3, 5, 2, 4)).reshape(E, N // ROWS, K // KTILE, 64)


def convert_w13(codes, sf):
    return convert_codes(interleave_gate_up(codes)), convert_scales(interleave_gate_up(sf))


def convert_w2(codes, sf):
    return convert_codes(codes), convert_scales(sf)


# ------------------------------------------------------------- TP slices
def logical_slice_w13(codes, sf, r: int, tp: int):
    """Slice r of tp of the logical w13: gate rows [rI', (r+1)I') and the same up rows."""
    I = codes.shape[1] // 2
    s = I // tp
    rows = np.r_[r * s:(r + 1) * s, I + r * s:I + (r + 1) * s]
    return codes[:, rows], sf[:, rows]


def logical_slice_w2(codes, sf, r: int, tp: int):
    """Slice r of tp of the logical w2: intermediate columns [rI', (r+1)I')."""
    I = codes.shape[2] * 2
    s = I // tp
    return codes[:, :, r * s // 2:(r + 1) * s // 2], sf[:, :, r * s // 16:(r + 1) * s // 16]


def view_slice_w13(conv: np.ndarray, r: int, tp: int) -> np.ndarray:
    """Byte view of slice r of converted w13 codes or scales [E, 2I/16, H/64, b]."""
    g = conv.shape[1] // tp
    return conv[:, r * g:(r + 1) * g]


def view_slice_w2(conv: np.ndarray, r: int, tp: int) -> np.ndarray:
    """Byte view of slice r of converted w2 codes or scales [E, H/16, I/64, b]."""
    t = conv.shape[2] // tp
    return conv[:, :, r * t:(r + 1) * t]

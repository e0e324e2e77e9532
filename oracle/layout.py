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
(N % 32 == 0, K % 64 == 0). Rows come in pairs of 16-row groups (32 rows);
row rho of a pair is row n = rho % 16 of half h = rho // 16. Per pair, the
K/64 k-tiles follow each other; a k-tile holds 64 slots s = q * 16 + n, one
per (16-column block q = k // 16 of the tile, row n), and each slot holds that
block for both halves:
  * codes: [N/32 pairs][K/64 k-tiles][1024 bytes]. Element (rho, k) of a tile
    (k < 64, i = k % 16) is nibble (i & 1) of byte (s * 2 + h) * 8 + i // 2
    (low nibble for even i);
  * scales: [N/32][K/64][128 bytes]. The scale of block q of row rho is byte
    s * 2 + h;
  * w13 only: converted row 32c + w is logical row 16c + w for w < 16 (gate)
    and I + 16c + (w - 16) for w >= 16 (up), so pair c holds the gate rows
    (half 0) and the up rows (half 1) of intermediates [16c, 16c + 16).
"""
from __future__ import annotations

import numpy as np

from .formats import pack_nibbles, unpack_nibbles

ROWS = 16        # rows per group; two groups per pair
KTILE = 64       # elements per k-tile
BLOCK = 16       # elements per scale block


def interleave_gate_up(rows: np.ndarray) -> np.ndarray:
    """[E, 2I, ...] logical (gate, then up) -> [E, 2I, ...] converted row order."""
    E, n2 = rows.shape[:2]
    I = n2 // 2
    gate = rows[:, :I].reshape((E, I // ROWS, ROWS) + rows.shape[2:])
    up = rows[:, I:].reshape((E, I // ROWS, ROWS) + rows.shape[2:])
    return np.stack([gate, up], axis=2).reshape(rows.shape)


def convert_codes(codes: np.ndarray) -> np.ndarray:
    """[E, N, K/2] bytes -> [E, N/32, K/64, 1024] bytes."""
    E, N, half = codes.shape
    K = half * 2
    nib = unpack_nibbles(codes).reshape(E, N // 32, 2, ROWS, K // KTILE, 4, BLOCK)
    #                                   e  p        h  n     c           q  i
    t = nib.transpose(0, 1, 4, 5, 3, 2, 6).reshape(E, N // 32, K // KTILE, 2048)
    return pack_nibbles(t)


def convert_scales(sf: np.ndarray) -> np.ndarray:
    """[E, N, K/16] bytes -> [E, N/32, K/64, 128] bytes."""
    E, N, nb = sf.shape
    K = nb * BLOCK
    s = sf.reshape(E, N // 32, 2, ROWS, K // KTILE, 4)
    #                e  p        h  n     c           q
    return np.ascontiguousarray(s.transpose(0, 1, 4, 5, 3, 2)).reshape(E, N // 32, K // KTILE, 128)


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
    """Byte view of slice r of converted w13 codes or scales [E, 2I/32, H/64, b]."""
    p = conv.shape[1] // tp
    return conv[:, r * p:(r + 1) * p]


def view_slice_w2(conv: np.ndarray, r: int, tp: int) -> np.ndarray:
    """Byte view of slice r of converted w2 codes or scales [E, H/32, I/64, b]."""
    t = conv.shape[2] // tp
    return conv[:, :, r * t:(r + 1) * t]

"""Routing metadata: routes grouped per expert, padded to the GEMM tile.
Test infrastructure (see ``oracle/__init__``).

The pages fix what the metadata is for, not its exact form (the flashinfer_ops
page, module docstring and "FlashInferOps.slot": the routing kernel writes the
expanded-to-permuted and permuted-to-token maps, per-expert counts and the
tile-to-expert maps; "gemm2_rows": the GEMM2 rows are the padded permuted rows;
"FlashInferOps.prepare_from_metadata": the metadata buffer is filled with -1 so
that unwritten rows stay defined; the expert_tp page, "route_rows": a route not
served here has permuted index -1).

Reading taken (the plain counting sort):
  * experts in ascending local index; within an expert, routes in ascending
    expanded index t * K + k; each expert's rows padded up to a multiple of the
    tile m; padding rows map to token -1;
  * a route whose expert is not local (outside [offset, offset + local)) or
    whose id is -1 has permuted index -1;
  * rows_max(T, K, E_local, m) = (min(E_local, R) + (R - min(E_local, R)) // m) * m
    with R = T * K, the bound of "gemm2_rows" without the op's 128 KiB floor.
"""
from __future__ import annotations

import numpy as np


def rows_max(T: int, K: int, E_local: int, m: int) -> int:
    R = T * K
    filled = min(E_local, R)
    return (filled + (R - filled) // m) * m


def permute(ids: np.ndarray, local_offset: int, local_num: int, m: int) -> dict:
    ids = np.asarray(ids, dtype=np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    local = flat - local_offset
    valid = (flat >= 0) & (local >= 0) & (local < local_num)
    counts = np.zeros(local_num, dtype=np.int64)
    for e in local[valid]:
        counts[e] += 1
    padded = -(-counts // m) * m
    offsets = np.zeros(local_num + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    total = int(offsets[-1])
    rmax = rows_max(T, K, local_num, m)
    assert total <= rmax
    exp2perm = np.full(T * K, -1, dtype=np.int64)
    perm2tok = np.full(rmax, -1, dtype=np.int64)
    seen = np.zeros(local_num, dtype=np.int64)
    for r in range(T * K):                       # ascending expanded index
        if not valid[r]:
            continue
        e = local[r]
        p = offsets[e] + seen[e]
        seen[e] += 1
        exp2perm[r] = p
        perm2tok[p] = r // K
    num_tiles = total // m
    tile_expert = np.full(rmax // m, -1, dtype=np.int64)
    for e in range(local_num):
        tile_expert[offsets[e] // m: offsets[e + 1] // m] = e
    return dict(
        counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
        exp2perm=exp2perm.reshape(T, K).astype(np.int32), perm2tok=perm2tok.astype(np.int32),
        tile_expert=tile_expert.astype(np.int32), num_tiles=num_tiles, total_rows=total,
        rows_max=rmax, tile_m=m,
    )

"""The C-ABI library loads, exports every function include/moe_nvfp4.h declares,
and its host-side sizing and validation behave as documented. No GPU: every
call here returns before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from nvfp4_block_scaled_route_amd import native as N
from oracle.permute import rows_max as oracle_rows_max

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert set(decl) == set(N.EXPORTS), decl


def test_library_exports_every_declared_symbol():
    L = N.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 8


@pytest.mark.parametrize("T,K,E,m", [(4, 2, 8, 16), (8, 8, 64, 16), (64, 8, 128, 16),
                                     (4096, 8, 128, 128), (32, 8, 128, 16), (1, 1, 1, 16),
                                     (0, 8, 8, 16), (3, 5, 1000, 256)])
def test_rows_max_matches_oracle(T, K, E, m):
    assert N.moe_rows_max(T, K, E, m) == oracle_rows_max(T, K, E, m)
    lay = N.moe_meta_layout_get(T, K, E, m)
    assert lay.rows_max == oracle_rows_max(T, K, E, m) and lay.tiles_max * m == lay.rows_max
    assert lay.subs_max * 16 == lay.rows_max
    fields = [lay.expert_offsets, lay.expert_counts, lay.exp2perm, lay.perm2tok, lay.tile_expert,
              lay.sub_sync, lay.tok_sync, lay.perm_counts]
    sizes = [E + 1, E, T * K, lay.rows_max, lay.tiles_max, 256 * lay.subs_max, 32 * T, -(-T * K // 512) * E]
    assert all(f % 64 == 0 for f in fields)
    for (f, n), nxt in zip(zip(fields, sizes), fields[1:] + [lay.total_ints]):
        assert f + n <= nxt
    header = {lay.num_tiles, lay.total_rows, lay.sync_status}
    assert len(header) == 3 and max(header) < 64
    # the 16 work-queue words sit in the header too, clear of its other words
    assert max(header) < lay.queue and lay.queue + 16 <= 64


def test_invalid_sizes_are_refused():
    L = N.lib()
    f = ctypes.c_float
    assert L.moe_rows_max(-1, 8, 8, 16) == -1
    with pytest.raises(N.MoeError):
        N.moe_meta_layout_get(8, 8, 64, 24)            # tile not a multiple of 16
    cases = [
        (L.moe_route, (None, 8, None, None, 4, 8, 9, f(1.0), 16, 0, 8, None, None, None, None), N.MOE_EUNSUPPORTED),  # K > E
        (L.moe_route, (None, 8, None, None, 4, 2000, 2, f(1.0), 16, 0, 8, None, None, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_route, (None, 8, None, None, 4, 8, 2, f(1.0), 8, 0, 8, None, None, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_route, (None, 4, None, None, 4, 8, 2, f(1.0), 16, 0, 8, None, None, None, None), N.MOE_EINVAL),  # stride < E
        (L.nvfp4_quant, (None, 24, None, 4, 24, None, None, None), N.MOE_EUNSUPPORTED),   # H % 16
        (L.nvfp4_quant, (None, 32, None, 4, 32, None, None, None), N.MOE_EINVAL),         # NULL
        (L.nvfp4_norm_quant, (None, 24, None, f(1.0), f(1e-6), None, 4, 24, None, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_router_logits, (None, 64, None, 4, 62, 8, None, None), N.MOE_EUNSUPPORTED),        # D % 4
        (L.moe_router_logits, (None, 64, None, 4, 64, 8, None, None), N.MOE_EINVAL),              # NULL
        (L.moe_router_logits, (16, 60, 16, 4, 64, 8, 16, None), N.MOE_EINVAL),                    # stride < D
        (L.moe_router_route, (16, 64, 16, 64, None, None, 4, 8, 9, f(1.0), 16, 0, 8, 16, 16, 16, 16, None),
         N.MOE_EUNSUPPORTED),                                                                       # K > E
        (L.moe_router_route, (16, 64, 16, 64, None, None, 4, 8, 2, f(1.0), 16, 0, 8, 16, 16, 16, None, None),
         N.MOE_EINVAL),                                                                             # NULL meta
        (L.nvfp4_norm_quant, (None, 32, None, f(1.0), f(1e-6), None, 4, 32, None, None, None), N.MOE_EINVAL),
        (L.nvfp4_norm_quant, (16, 32, None, f(1.0), f(0.0), 16, 4, 32, 16, 16, None), N.MOE_EINVAL),   # eps 0
        (L.nvfp4_norm_quant, (16, 32 * 1024, None, f(1.0), f(1e-6), 16, 4, 32 * 1024, 16, 16, None), N.MOE_EUNSUPPORTED),
        (L.moe_route_quant, (None, 8, None, None, 4, 8, 2, f(1.0), 16, 0, 8, None, None, None,
                             None, 24, None, 24, None, None, None), N.MOE_EUNSUPPORTED),   # H % 16
        (L.moe_route_quant, (None, 8, None, None, 4, 8, 9, f(1.0), 16, 0, 8, None, None, None,
                             None, 32, None, 32, None, None, None), N.MOE_EINVAL),         # NULL x
        (L.moe_pack_w13, (None, None, 2, 24, 64, None, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_pack_w2, (None, None, 2, 64, 96, None, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_pack_w2, (None, None, 2, 48, 64, None, None, None), N.MOE_EUNSUPPORTED),   # H % 32
        (L.moe_finalize, (None, 64, 1, 0, None, None, None, f(1.0), f(1e-6), 1, 4, 2, 60, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_finalize, (None, 64, 17, 0, None, None, None, f(1.0), f(1e-6), 1, 4, 2, 64, None, None), N.MOE_EUNSUPPORTED),
        (L.moe_finalize, (None, 64, 1, 0, None, None, None, f(1.0), f(1e-6), 1, 4, 2, 64, None, None), N.MOE_EINVAL),
    ]
    for fn, args, want in cases:
        assert fn(*args) == want, (fn.__name__, L.moe_last_error())
        assert L.moe_last_error()


def test_experts_refusals():
    L = N.lib()
    w = N.MoeNvfp4Weights()
    args = lambda H, I, m: (None, None, None, ctypes.byref(w), 4, 2, 8, H, I, m, None, None, None, H, None)
    assert L.moe_experts_fwd(*args(96, 128, 16)) == N.MOE_EUNSUPPORTED     # H % 64
    assert L.moe_experts_fwd(*args(256, 96, 16)) == N.MOE_EUNSUPPORTED     # I % 64
    assert L.moe_experts_fwd(*args(256, 128, 48 + 1)) == N.MOE_EUNSUPPORTED
    assert L.moe_experts_fwd(*args(256, 128, 16)) == N.MOE_EINVAL          # NULL pointers
    assert L.moe_experts_fwd(None, None, None, None, 4, 2, 8, 256, 128, 16, None, None, None, 256, None) == N.MOE_EINVAL
    assert L.moe_experts_fwd(*args(256, 16384 + 64, 16)) == N.MOE_EUNSUPPORTED   # I above the limit
    assert L.moe_experts_fwd(*args(16384 + 64, 128, 16)) == N.MOE_EUNSUPPORTED   # H above the limit
    # strides too small for the shape: checked before any launch
    w.w13 = w.w13_sf = w.w2 = w.w2_sf = 256
    w.g1_alphas = w.g1_scale_c = w.g2_alphas = 256
    assert L.moe_experts_fwd(256, 256, 256, ctypes.byref(w), 4, 2, 8, 256, 128, 16, 256, 256, 256, 256, None) == N.MOE_EINVAL
    assert b"stride" in L.moe_last_error()


def test_experts_w4a16_refusals():
    L = N.lib()
    w = N.MoeNvfp4Weights()
    args = lambda H, I, m: (None, H, None, ctypes.byref(w), 4, 2, 8, H, I, m, None, None, H, None)
    assert L.moe_experts_fwd_w4a16(*args(96, 128, 16)) == N.MOE_EUNSUPPORTED     # H % 64
    assert L.moe_experts_fwd_w4a16(*args(256, 96, 16)) == N.MOE_EUNSUPPORTED     # I % 64
    assert L.moe_experts_fwd_w4a16(*args(256, 128, 24)) == N.MOE_EUNSUPPORTED    # tile
    assert L.moe_experts_fwd_w4a16(*args(256, 128, 16)) == N.MOE_EINVAL          # NULL pointers
    assert L.moe_experts_fwd_w4a16(None, 256, None, None, 4, 2, 8, 256, 128, 16, None, None, 256, None) == N.MOE_EINVAL


def test_experts_bf16_refusals():
    L = N.lib()
    args = lambda H, I, m: (None, H, None, None, None, 4, 2, 8, H, I, m, None, None, H, None)
    assert L.moe_experts_fwd_bf16(*args(96, 128, 16)) == N.MOE_EUNSUPPORTED     # H % 64
    assert L.moe_experts_fwd_bf16(*args(256, 96, 16)) == N.MOE_EUNSUPPORTED     # I % 64
    assert L.moe_experts_fwd_bf16(*args(256, 128, 16)) == N.MOE_EINVAL          # NULL meta
    assert L.moe_experts_fwd_bf16(16, 256, 16, None, 16, 4, 2, 8, 256, 128, 16, 16, 16, 256, None) == N.MOE_EINVAL


def test_zero_tokens_is_a_no_op_without_device():
    L = N.lib()
    assert L.nvfp4_quant(None, 64, None, 0, 64, None, None, None) == N.MOE_OK
    assert L.moe_finalize(None, 64, 1, 0, None, None, None, ctypes.c_float(1.0), ctypes.c_float(1e-6), 1, 0, 2, 64, None, None) == N.MOE_OK


def _weights_struct(H, I, E, base=1 << 20, **override):
    """A descriptor of full-width converted weights at fake, aligned addresses
    (never dereferenced: moe_validate_weights reads no device memory)."""
    w = N.MoeNvfp4Weights()
    w.w13, w.w13_sf, w.w2, w.w2_sf = base, 2 * base, 3 * base, 4 * base
    w.g1_alphas, w.g1_scale_c, w.g2_alphas = 5 * base, 6 * base, 7 * base
    w.w13_pair_stride_bytes = (H // 64) * 1024
    w.w13_sf_pair_stride_bytes = (H // 64) * 128
    w.w13_expert_stride_bytes = (I // 16) * w.w13_pair_stride_bytes
    w.w13_sf_expert_stride_bytes = (I // 16) * w.w13_sf_pair_stride_bytes
    w.w2_pair_stride_bytes = (I // 64) * 1024
    w.w2_sf_pair_stride_bytes = (I // 64) * 128
    w.w2_expert_stride_bytes = (H // 32) * w.w2_pair_stride_bytes
    w.w2_sf_expert_stride_bytes = (H // 32) * w.w2_sf_pair_stride_bytes
    for k, v in override.items():
        setattr(w, k, v)
    return w


def test_validate_weights_accepts_the_workloads_and_their_tp_cuts():
    L = N.lib()
    for (H, I, E, tp) in [(256, 128, 8, 1), (2048, 768, 64, 1), (4096, 1536, 128, 1),
                          (4096, 2048, 128, 8), (4096, 2048, 128, 2), (1024, 512, 4, 4)]:
        w = _weights_struct(H, I, E)
        assert L.moe_validate_weights(ctypes.byref(w), E, H, I, tp) == N.MOE_OK, L.moe_last_error()


def test_validate_weights_refusals():
    """The expert_tp page's "unsupported": tp must divide I, the slice I/tp be a
    multiple of 64 and H of 128; and the descriptor's pointers and strides."""
    L = N.lib()
    H, I, E = 4096, 2048, 128
    ok = _weights_struct(H, I, E)
    cases = [
        ((ok, E, H, I, 3), N.MOE_EUNSUPPORTED, b"split"),           # 2048 % 3
        ((ok, E, H, I, 64), N.MOE_EUNSUPPORTED, b"multiples"),      # slice 32
        ((_weights_struct(64 * 23, I, E), E, 64 * 23, I, 8), N.MOE_EUNSUPPORTED, b"multiples"),     # H % 128
        ((ok, E, H, I, 0), N.MOE_EINVAL, b"tp"),
        ((ok, 0, H, I, 1), N.MOE_EINVAL, b"E_local"),
        ((ok, E, H + 32, I, 1), N.MOE_EUNSUPPORTED, b"multiples of 64"),
        ((_weights_struct(H, I, E, w2=0), E, H, I, 1), N.MOE_EINVAL, b"NULL"),
        ((_weights_struct(H, I, E, g1_scale_c=8), E, H, I, 1), N.MOE_EINVAL, b"aligned"),
        ((_weights_struct(H, I, E, w13_pair_stride_bytes=1024), E, H, I, 1), N.MOE_EINVAL, b"pair strides"),
        ((_weights_struct(H, I, E, w2_sf_pair_stride_bytes=(I // 64) * 128 + 8), E, H, I, 1), N.MOE_EINVAL,
         b"pair strides"),
        ((_weights_struct(H, I, E, w2_expert_stride_bytes=1024), E, H, I, 1), N.MOE_EINVAL, b"expert strides"),
    ]
    for (w, e, h, i, tp), want, msg in cases:
        assert L.moe_validate_weights(ctypes.byref(w), e, h, i, tp) == want, (tp, L.moe_last_error())
        assert msg in L.moe_last_error(), L.moe_last_error()
    assert L.moe_validate_weights(None, E, H, I, 1) == N.MOE_EINVAL


@pytest.mark.parametrize("T,K,E,H,I,m,tp", [(4, 2, 8, 256, 128, 16, 1), (8, 8, 64, 2048, 768, 16, 1),
                                            (64, 8, 128, 4096, 1536, 16, 1),
                                            (4096, 8, 128, 4096, 1536, 128, 1),
                                            (32, 8, 128, 4096, 2048, 16, 8), (0, 8, 8, 64, 64, 16, 1)])
def test_workspace_layout(T, K, E, H, I, m, tp):
    """Every buffer of one layer call at a 256-byte aligned offset of one
    allocation, none overlapping, each of the size its call needs."""
    lay = N.moe_workspace_bytes(T, K, E, H, I, m, tp)
    meta = N.moe_meta_layout_get(T, K, E, m)
    rm = oracle_rows_max(T, K, E, m)
    Is = I // tp
    need = [("meta", 4 * meta.total_ints), ("topk_ids", 4 * T * K), ("topk_weights", 4 * T * K),
            ("a_codes", T * H // 2), ("a_sf", T * H // 16), ("inter_codes", rm * Is // 2),
            ("inter_sf", rm * Is // 16), ("rows", tp * rm * H * 2)]
    spans = []
    for name, nbytes in need:
        off = getattr(lay, name)
        assert off % 256 == 0, name
        spans.append((off, off + nbytes))
    spans.sort()
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= lay.total_bytes < spans[-1][1] + 256 * len(need)
    assert N.lib().moe_workspace_bytes(T, K, E, H, I, m, tp, None) == lay.total_bytes


def test_workspace_refusals():
    L = N.lib()
    assert L.moe_workspace_bytes(4, 0, 8, 256, 128, 16, 1, None) == -1
    assert L.moe_workspace_bytes(4, 2, 8, 256, 128, 24, 1, None) == -1
    assert L.moe_workspace_bytes(4, 2, 8, 256, 128, 16, 3, None) == -1       # 128 % 3
    assert L.moe_last_error()


def test_noalloc_refusals():
    """moe_experts_fwd_noalloc refuses, before touching the device, an
    intermediate larger than its static memory, and the usual bad shapes."""
    L = N.lib()
    w = N.MoeNvfp4Weights()
    big = (None, None, None, ctypes.byref(w), 65536, 8, 128, 4096, 4096, 128, None, 4096, None)
    assert L.moe_experts_fwd_noalloc(*big) == N.MOE_EUNSUPPORTED
    assert b"static scratch" in L.moe_last_error()
    assert L.moe_experts_fwd_noalloc(None, None, None, ctypes.byref(w), 4, 2, 8, 96, 128, 16, None, 96, None) \
        == N.MOE_EUNSUPPORTED                                               # H % 64
    assert L.moe_experts_fwd_noalloc(None, None, None, None, 4, 2, 8, 256, 128, 16, None, 256, None) == N.MOE_EINVAL


def test_experts_finalize_refusals():
    """moe_experts_finalize: the expert step's checks and the finalize's, before
    any launch."""
    L = N.lib()
    w = N.MoeNvfp4Weights()
    f = ctypes.c_float

    def call(H=256, I=128, m=16, nparts=1, pstride=0, rows=16, tw=16, out=16, meta=16):
        return L.moe_experts_finalize(16, 16, meta, ctypes.byref(w), 4, 2, 8, H, I, m, 16, 16, rows, H, nparts,
                                      pstride, tw, None, f(1.0), f(1e-6), 1, out, None)
    assert call(H=96) == N.MOE_EUNSUPPORTED
    assert call(m=24) == N.MOE_EUNSUPPORTED
    assert call(nparts=17) == N.MOE_EUNSUPPORTED
    assert call(nparts=0) == N.MOE_EUNSUPPORTED
    assert call(out=0) == N.MOE_EINVAL
    assert call(tw=0) == N.MOE_EINVAL
    assert call(tw=8) == N.MOE_EINVAL                  # alignment
    assert call(nparts=2, pstride=12) == N.MOE_EINVAL   # partial stride % 8
    assert call() == N.MOE_EINVAL                      # NULL weight pointers (checked with the expert step)
    assert L.moe_last_error()

"""ctypes binding of libmoe_nvfp4.so (include/moe_nvfp4.h): the same entry
points, argument marshalling only. Tensors are torch device tensors (PyTorch
provides device memory and streams); every computation runs in the library's
HIP kernels. There is no fallback: without the built library, or on a failed
call, this raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_nvfp4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ELAUNCH = 0, -1, -2, -3

# Every symbol include/moe_nvfp4.h declares.
EXPORTS = ("moe_abi_version", "moe_last_error", "moe_rows_max", "moe_meta_layout_get",
           "moe_route", "nvfp4_quant", "moe_route_quant", "moe_pack_w13", "moe_pack_w2",
           "moe_experts_fwd", "moe_finalize", "nvfp4_norm_quant", "moe_router_logits",
           "moe_router_route", "moe_experts_fwd_w4a16", "moe_experts_fwd_bf16",
           "moe_validate_weights", "moe_workspace_bytes", "moe_experts_fwd_noalloc",
           "moe_experts_finalize")


class MoeMetaLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_tiles", "total_rows", "expert_offsets", "expert_counts", "exp2perm", "perm2tok",
        "tile_expert", "total_ints", "rows_max", "tiles_max", "sync_status", "sub_sync", "subs_max", "perm_counts",
        "tok_sync", "fin_part", "queue")]


class MoeNvfp4Weights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_sf", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p)] + \
               [(n, ctypes.c_int64) for n in (
                   "w13_expert_stride_bytes", "w13_pair_stride_bytes",
                   "w13_sf_expert_stride_bytes", "w13_sf_pair_stride_bytes",
                   "w2_expert_stride_bytes", "w2_pair_stride_bytes",
                   "w2_sf_expert_stride_bytes", "w2_sf_pair_stride_bytes")] + \
               [("g1_alphas", ctypes.c_void_p), ("g1_scale_c", ctypes.c_void_p),
                ("g2_alphas", ctypes.c_void_p)]


class MoeWorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "meta", "topk_ids", "topk_weights", "a_codes", "a_sf", "inter_codes", "inter_sf", "rows",
        "total_bytes")]


class MoeError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run python -m nvfp4_block_scaled_route_amd.build")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    sig = {
        "moe_abi_version": (i32, []),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_rows_max": (i64, [i32, i32, i32, i32]),
        "moe_meta_layout_get": (i32, [i32, i32, i32, i32, ctypes.POINTER(MoeMetaLayout)]),
        "moe_route": (i32, [vp, i64, vp, vp, i32, i32, i32, f32, i32, i32, i32, vp, vp, vp, vp]),
        "nvfp4_quant": (i32, [vp, i64, vp, i32, i32, vp, vp, vp]),
        "nvfp4_norm_quant": (i32, [vp, i64, vp, f32, f32, vp, i32, i32, vp, vp, vp]),
        "moe_router_logits": (i32, [vp, i64, vp, i32, i32, i32, vp, vp]),
        "moe_experts_fwd_bf16": (i32, [vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i64, vp]),
        "moe_experts_fwd_w4a16": (i32, [vp, i64, vp, ctypes.POINTER(MoeNvfp4Weights), i32, i32, i32, i32,
                                        i32, i32, vp, vp, i64, vp]),
        "moe_router_route": (i32, [vp, i64, vp, i32, vp, vp, i32, i32, i32, f32, i32, i32, i32, vp, vp,
                                   vp, vp, vp]),
        "moe_route_quant": (i32, [vp, i64, vp, vp, i32, i32, i32, f32, i32, i32, i32, vp, vp, vp,
                                  vp, i64, vp, i32, vp, vp, vp]),
        "moe_pack_w13": (i32, [vp, vp, i32, i32, i32, vp, vp, vp]),
        "moe_pack_w2": (i32, [vp, vp, i32, i32, i32, vp, vp, vp]),
        "moe_experts_fwd": (i32, [vp, vp, vp, ctypes.POINTER(MoeNvfp4Weights), i32, i32, i32,
                                  i32, i32, i32, vp, vp, vp, i64, vp]),
        "moe_finalize": (i32, [vp, i64, i32, i64, vp, vp, vp, f32, f32, i32, i32, i32, i32, vp, vp]),
        "moe_experts_fwd_noalloc": (i32, [vp, vp, vp, ctypes.POINTER(MoeNvfp4Weights), i32, i32, i32,
                                          i32, i32, i32, vp, i64, vp]),
        "moe_experts_finalize": (i32, [vp, vp, vp, ctypes.POINTER(MoeNvfp4Weights), i32, i32, i32, i32, i32,
                                       i32, vp, vp, vp, i64, i32, i64, vp, vp, f32, f32, i32, vp, vp]),
        "moe_validate_weights": (i32, [ctypes.POINTER(MoeNvfp4Weights), i32, i32, i32, i32]),
        "moe_workspace_bytes": (i64, [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(MoeWorkspaceLayout)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc: int, name: str) -> None:
    if rc != MOE_OK:
        msg = lib().moe_last_error().decode(errors="replace")
        raise MoeError(f"{name} failed ({rc}): {msg}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ sizing
def moe_rows_max(T: int, K: int, E_local: int, tile_m: int) -> int:
    return int(lib().moe_rows_max(T, K, E_local, tile_m))


def moe_workspace_bytes(T: int, K: int, E_local: int, H: int, I: int, tile_m: int,
                        tp: int = 1) -> MoeWorkspaceLayout:
    out = MoeWorkspaceLayout()
    n = lib().moe_workspace_bytes(T, K, E_local, H, I, tile_m, tp, ctypes.byref(out))
    if n < 0:
        _check(MOE_EINVAL, "moe_workspace_bytes")
    return out


def moe_meta_layout_get(T: int, K: int, E_local: int, tile_m: int) -> MoeMetaLayout:
    out = MoeMetaLayout()
    _check(lib().moe_meta_layout_get(T, K, E_local, tile_m, ctypes.byref(out)), "moe_meta_layout_get")
    return out


# ------------------------------------------------------------------ entry points
def moe_route(logits, expert_bias, is_padding, K, route_scale, tile_m, local_expert_offset,
              local_num_experts, topk_ids, topk_weights, meta, stream=None) -> None:
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits), logits.stride(0), _ptr(expert_bias), _ptr(is_padding),
                           T, E, K, float(route_scale), tile_m, local_expert_offset,
                           local_num_experts, _ptr(topk_ids), _ptr(topk_weights), _ptr(meta),
                           _stream(stream)), "moe_route")


def nvfp4_quant(x, gscale, codes, sf, stream=None) -> None:
    T, H = x.shape
    _check(lib().nvfp4_quant(_ptr(x), x.stride(0), _ptr(gscale), T, H, _ptr(codes), _ptr(sf),
                             _stream(stream)), "nvfp4_quant")


def nvfp4_norm_quant(x, norm_weight, gain_center, eps, gscale, codes, sf, stream=None) -> None:
    T, H = x.shape
    _check(lib().nvfp4_norm_quant(_ptr(x), x.stride(0), _ptr(norm_weight), gain_center, eps,
                                  _ptr(gscale), T, H, _ptr(codes), _ptr(sf), _stream(stream)),
           "nvfp4_norm_quant")


def moe_router_logits(x, w_router, logits, stream=None) -> None:
    T, D = x.shape
    _check(lib().moe_router_logits(_ptr(x), x.stride(0), _ptr(w_router), T, D, w_router.shape[0],
                                   _ptr(logits), _stream(stream)), "moe_router_logits")


def moe_router_route(x, w_router, expert_bias, is_padding, K, route_scale, tile_m, local_expert_offset,
                     local_num_experts, logits, topk_ids, topk_weights, meta, stream=None) -> None:
    T, D = x.shape
    _check(lib().moe_router_route(_ptr(x), x.stride(0), _ptr(w_router), D, _ptr(expert_bias),
                                  _ptr(is_padding), T, w_router.shape[0], K, route_scale, tile_m,
                                  local_expert_offset, local_num_experts, _ptr(logits), _ptr(topk_ids),
                                  _ptr(topk_weights), _ptr(meta), _stream(stream)), "moe_router_route")


def moe_route_quant(logits, expert_bias, is_padding, K, route_scale, tile_m, local_expert_offset,
                    local_num_experts, topk_ids, topk_weights, meta, x, gscale, codes, sf,
                    stream=None) -> None:
    T, E = logits.shape
    H = x.shape[1]
    _check(lib().moe_route_quant(_ptr(logits), logits.stride(0), _ptr(expert_bias),
                                 _ptr(is_padding), T, E, K, float(route_scale), tile_m,
                                 local_expert_offset, local_num_experts, _ptr(topk_ids),
                                 _ptr(topk_weights), _ptr(meta), _ptr(x), x.stride(0),
                                 _ptr(gscale), H, _ptr(codes), _ptr(sf), _stream(stream)),
           "moe_route_quant")


def moe_pack_w13(codes, sf, E, I, H, out_codes, out_sf, stream=None) -> None:
    _check(lib().moe_pack_w13(_ptr(codes), _ptr(sf), E, I, H, _ptr(out_codes), _ptr(out_sf),
                              _stream(stream)), "moe_pack_w13")


def moe_pack_w2(codes, sf, E, H, I, out_codes, out_sf, stream=None) -> None:
    _check(lib().moe_pack_w2(_ptr(codes), _ptr(sf), E, H, I, _ptr(out_codes), _ptr(out_sf),
                             _stream(stream)), "moe_pack_w2")


@dataclass
class Weights:
    """Converted experts (device tensors) plus the strides the kernels read them with."""
    w13: torch.Tensor
    w13_sf: torch.Tensor
    w2: torch.Tensor
    w2_sf: torch.Tensor
    w13_expert_stride: int
    w13_pair_stride: int
    w13_sf_expert_stride: int
    w13_sf_pair_stride: int
    w2_expert_stride: int
    w2_pair_stride: int
    w2_sf_expert_stride: int
    w2_sf_pair_stride: int
    g1_alphas: torch.Tensor
    g1_scale_c: torch.Tensor
    g2_alphas: torch.Tensor
    w13_offset: int = 0       # byte offsets of a view into the tensors above
    w13_sf_offset: int = 0
    w2_offset: int = 0
    w2_sf_offset: int = 0

    def struct(self) -> MoeNvfp4Weights:
        return MoeNvfp4Weights(
            _ptr(self.w13) + self.w13_offset, _ptr(self.w13_sf) + self.w13_sf_offset,
            _ptr(self.w2) + self.w2_offset, _ptr(self.w2_sf) + self.w2_sf_offset,
            self.w13_expert_stride, self.w13_pair_stride, self.w13_sf_expert_stride,
            self.w13_sf_pair_stride, self.w2_expert_stride, self.w2_pair_stride,
            self.w2_sf_expert_stride, self.w2_sf_pair_stride,
            _ptr(self.g1_alphas), _ptr(self.g1_scale_c), _ptr(self.g2_alphas))


def moe_validate_weights(weights: Weights, E_local: int, H: int, I: int, tp: int = 1) -> None:
    """Host-only check of the descriptor (and of its cut into tp slices); raises MoeError."""
    ws = weights.struct()
    _check(lib().moe_validate_weights(ctypes.byref(ws), E_local, H, I, tp), "moe_validate_weights")


def moe_experts_fwd(a_codes, a_sf, meta, weights: Weights, T, K, E_local, H, I, tile_m,
                    inter_codes, inter_sf, rows, stream=None) -> None:
    ws = weights.struct()
    _check(lib().moe_experts_fwd(_ptr(a_codes), _ptr(a_sf), _ptr(meta), ctypes.byref(ws), T, K,
                                 E_local, H, I, tile_m, _ptr(inter_codes), _ptr(inter_sf),
                                 _ptr(rows), rows.stride(0), _stream(stream)), "moe_experts_fwd")


def moe_experts_finalize(a_codes, a_sf, meta, weights: Weights, T, K, E_local, H, I, tile_m,
                         inter_codes, inter_sf, rows, n_partials, partial_stride, topk_weights, norm_weight,
                         gain_center, eps, weight_before_norm, out, stream=None) -> None:
    """rows: the partials' base (partial q at rows + q * partial_stride elements);
    this call writes partial n_partials - 1 and finalizes into out."""
    ws = weights.struct()
    _check(lib().moe_experts_finalize(_ptr(a_codes), _ptr(a_sf), _ptr(meta), ctypes.byref(ws), T, K, E_local,
                                      H, I, tile_m, _ptr(inter_codes), _ptr(inter_sf), _ptr(rows),
                                      rows.stride(-2), n_partials, partial_stride, _ptr(topk_weights),
                                      _ptr(norm_weight), float(gain_center), float(eps),
                                      int(weight_before_norm), _ptr(out), _stream(stream)),
           "moe_experts_finalize")


def moe_experts_fwd_noalloc(a_codes, a_sf, meta, weights: Weights, T, K, E_local, H, I, tile_m,
                            rows, stream=None) -> None:
    ws = weights.struct()
    _check(lib().moe_experts_fwd_noalloc(_ptr(a_codes), _ptr(a_sf), _ptr(meta), ctypes.byref(ws), T, K,
                                         E_local, H, I, tile_m, _ptr(rows), rows.stride(0), _stream(stream)),
           "moe_experts_fwd_noalloc")


def moe_experts_fwd_w4a16(x, meta, weights: Weights, T, K, E_local, H, I, tile_m, inter, rows,
                          stream=None) -> None:
    ws = weights.struct()
    _check(lib().moe_experts_fwd_w4a16(_ptr(x), x.stride(0), _ptr(meta), ctypes.byref(ws), T, K, E_local, H,
                                       I, tile_m, _ptr(inter), _ptr(rows), rows.stride(0), _stream(stream)),
           "moe_experts_fwd_w4a16")


def moe_experts_fwd_bf16(x, meta, w13, w2, T, K, E_local, H, I, tile_m, inter, rows, stream=None) -> None:
    _check(lib().moe_experts_fwd_bf16(_ptr(x), x.stride(0), _ptr(meta), _ptr(w13), _ptr(w2), T, K, E_local, H, I,
                                      tile_m, _ptr(inter), _ptr(rows), rows.stride(0), _stream(stream)),
           "moe_experts_fwd_bf16")


def moe_finalize(rows, n_partials, partial_stride, exp2perm, topk_weights, norm_weight,
                 gain_center, eps, weight_before_norm, T, K, H, out, stream=None) -> None:
    _check(lib().moe_finalize(_ptr(rows), rows.stride(-2), n_partials, partial_stride,
                              _ptr(exp2perm), _ptr(topk_weights), _ptr(norm_weight),
                              float(gain_center), float(eps), int(weight_before_norm), T, K, H,
                              _ptr(out), _stream(stream)), "moe_finalize")

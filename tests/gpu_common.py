"""Helpers of the GPU parity tests: run the HIP path through the C-ABI on a
workload's seeded inputs and bring the results back as numpy arrays."""
from __future__ import annotations

import sys

import numpy as np
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W

DEV = "cuda:0"


def say(*args):
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def sync_counters(meta: np.ndarray, L) -> np.ndarray:
    """The two sync counters of every 16-row tile in a metadata buffer."""
    return meta[L.sub_sync:L.sub_sync + 256 * L.subs_max].reshape(-1, 256)[:, :2]


def queue_words(meta: np.ndarray, L) -> np.ndarray:
    """The register-tiled expert step's work-queue counters (zero between calls)."""
    return meta[L.queue:L.queue + 16]


def token_counters(meta: np.ndarray, L, T: int) -> np.ndarray:
    """The arrival counter of every token (moe_experts_finalize's one-launch form)."""
    return meta[L.tok_sync:L.tok_sync + 32 * T].reshape(-1, 32)[:, 0]


def upload_weights(inp: W.Inputs) -> N.Weights:
    w13c, w13s, w2c, w2s = dev(inp.w13_codes), dev(inp.w13_sf), dev(inp.w2_codes), dev(inp.w2_sf)
    w = LY.pack_weights(w13c, w13s, w2c, w2s, dev(inp.g1_alphas), dev(inp.g1_scale_c),
                        dev(inp.g2_alphas))
    torch.cuda.synchronize()
    del w13c, w13s, w2c, w2s
    return w


def run_layer(inp: W.Inputs, weights: N.Weights | None = None, tile_m: int | None = None,
              is_padding: np.ndarray | None = None, tp: int = 1, bias: np.ndarray | None = None,
              fill_rows: int | None = None, fused_finalize: bool = False) -> dict:
    wl = inp.wl
    m = wl.tile_m if tile_m is None else tile_m
    if weights is None:
        weights = upload_weights(inp)
    shape = LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, m, tp)
    bufs = LY.Buffers(shape, DEV)
    if fill_rows is not None:
        bufs.rows.fill_(fill_rows)
    slices = None if tp == 1 else [LY.slice_weights(weights, r, tp, wl.H, wl.I) for r in range(tp)]
    say(f"layer {wl.name} T={wl.T} H={wl.H} I={wl.I} E={wl.E} K={wl.K} tile_m={m} tp={tp}")
    LY.run_layer(bufs, dev(inp.x_bf16), dev(inp.a1_gscale), dev(inp.logits),
                 None if bias is None else dev(bias),
                 None if is_padding is None else dev(is_padding.astype(np.uint8)),
                 weights, dev(inp.norm_weight_bf16), wl.gain_center, wl.eps,
                 bool(wl.weight_before_norm), slices=slices, fused_finalize=fused_finalize)
    torch.cuda.synchronize()
    L = bufs.layout
    meta = host(bufs.meta)
    res = dict(
        a_codes=host(bufs.a_codes), a_sf=host(bufs.a_sf), ids=host(bufs.ids),
        weights=host(bufs.weights), meta=meta, layout=L,
        num_tiles=int(meta[L.num_tiles]), total_rows=int(meta[L.total_rows]),
        offsets=meta[L.expert_offsets:L.expert_offsets + wl.E + 1],
        counts=meta[L.expert_counts:L.expert_counts + wl.E],
        exp2perm=meta[L.exp2perm:L.exp2perm + wl.T * wl.K].reshape(wl.T, wl.K),
        perm2tok=meta[L.perm2tok:L.perm2tok + L.rows_max],
        tile_expert=meta[L.tile_expert:L.tile_expert + L.tiles_max],
        sync_status=int(meta[L.sync_status]), sub_sync=sync_counters(meta, L),
        tok_sync=token_counters(meta, L, wl.T),
        inter_codes=host(bufs.inter_codes), inter_sf=host(bufs.inter_sf),
        rows=host(bufs.rows), out=host(bufs.out))
    return res


# ------------------------------------------------------------------ requantized intermediate
U32 = 2.0 ** -24      # fp32 unit roundoff


def abs_gemm1(a_codes, a_sf, tokens, experts, w13_codes, w13_sf) -> np.ndarray:
    """sum_h |a[t, h] w13[e, n, h]| per route and column: the oracle's exact GEMM1
    on the magnitudes (sign bits cleared), the scale of an accumulation's error."""
    from oracle import experts as ex
    return ex.gemm1(a_codes & 0x77, a_sf & 0x7F, tokens, experts, w13_codes & 0x77, w13_sf & 0x7F)


def h_error_bound(acc1, abs_acc1, experts, g1_alphas, g1_scale_c, h, K) -> np.ndarray:
    """A bound on |h_kernel - h_oracle| per element of the gated activation.

    The kernels accumulate exact f16 products in fp32 through a chain of at most
    K/16 matrix instructions, each adding at most 32 terms, so the accumulator's
    error is at most (K/16 + 32) u sum|a w| to first order (u = 2^-24, any
    summation order of that depth). It propagates into h = silu(g) u through
    |d h / d acc_gate| = |ga silu'(g) u| and |d h / d acc_up| = |uc silu(g)|,
    silu'(g) = s (1 + g (1 - s)) with s the logistic of g, taken at g (the
    accumulator's relative error is far below what moves it); the scalar
    products, the exponential (about (|g| + 4) u relative for exp2 of a rounded
    argument), the reciprocal or division and the final product add at most
    (|g| + 12) u |h|. Doubled for safety."""
    I = h.shape[1]
    ga = np.asarray(g1_alphas, np.float64)[experts][:, None]
    uc = np.asarray(g1_scale_c, np.float64)[experts][:, None]
    g = acc1[:, :I] * ga
    up = acc1[:, I:] * uc
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    depth = K / 16 + 32
    eps_g = depth * U32 * abs_acc1[:, :I] * np.abs(ga)
    eps_u = depth * U32 * abs_acc1[:, I:] * np.abs(uc)
    hv = np.abs(h.astype(np.float64))
    return 2.0 * (dsilu * np.abs(up) * eps_g + np.abs(silu) * eps_u + (np.abs(g) + 12.0) * U32 * hv) + 1e-38


def check_requant(got_codes, got_sf, h, ref_codes, ref_sf, eb_of, name, max_frac=1e-3):
    """The kernel's requantized intermediate (codes [R, I/2], scales [R, I/16])
    against the oracle's, where several results are correct: every differing
    scale byte is the adjacent e4m3 code, with the oracle's amax / 6 within
    (the block's error bound) / 6 of the midpoint between the two; every code
    that differs, after quantizing the oracle's h with the kernel's scale, is
    the adjacent e2m1 value of the same sign (or a zero of the other sign),
    with the oracle's h within its error bound of the boundary between the two.
    At most max_frac of the codes and of the scales may differ. eb_of(routes)
    gives the error bound [len(routes), I] of those routes' h (h_error_bound),
    asked for only where something differs."""
    from oracle import formats as F
    R, nb = got_sf.shape
    sf_diff = got_sf != ref_sf
    code_diff = got_codes != ref_codes
    say(f"{name}: requant scale diff {sf_diff.mean():.2e}, code byte diff {code_diff.mean():.2e}")
    assert sf_diff.mean() <= max_frac and code_diff.mean() <= max_frac, name
    bad = np.nonzero(sf_diff.any(axis=1) | code_diff.any(axis=1))[0]
    if bad.size == 0:
        return
    eb = eb_of(bad)
    hb = h[bad].astype(np.float32).reshape(bad.size, nb, 16)
    ebb = eb.reshape(bad.size, nb, 16)
    gsf, rsf = got_sf[bad], ref_sf[bad]
    # scales: adjacent codes, amax / 6 at their midpoint within the bound
    rr, bb = np.nonzero(gsf != rsf)
    for r, b in zip(rr, bb):
        g, o = int(gsf[r, b]), int(rsf[r, b])
        assert abs(g - o) == 1 and max(g, o) < 0x7F, (name, bad[r], b, g, o)
        mid = (F.E4M3[g] + F.E4M3[o]) / 2.0
        amax = float(np.max(np.abs(hb[r, b]).astype(np.float64)))
        assert abs(amax / 6.0 - mid) <= float(ebb[r, b].max()) / 6.0 + 2 * U32 * amax, (name, bad[r], b)
    # codes, against the oracle's h quantized with the kernel's scale
    gn = F.unpack_nibbles(got_codes[bad]).astype(np.int64)
    d = F.decode_e4m3(gsf).astype(np.float32)
    with np.errstate(divide="ignore"):
        recip = np.where(d == 0, np.float32(0), (np.float32(1) / d).astype(np.float32)).astype(np.float32)
    want = F.encode_e2m1((hb * recip[..., None]).astype(np.float32)).reshape(bad.size, -1).astype(np.int64)
    want = np.where(np.repeat(d == 0, 16, axis=1), 0, want)
    rr, ii = np.nonzero(gn != want)
    hv = h[bad].astype(np.float64)
    for r, i in zip(rr, ii):
        g, o = int(gn[r, i]), int(want[r, i])
        dd = float(d[r, i // 16])
        mg, mo = g & 7, o & 7
        if mg == 0 and mo == 0:             # a zero of the other sign: h within the bound of 0
            assert abs(hv[r, i]) <= eb[r, i], (name, bad[r], i)
            continue
        assert (g >> 3) == (o >> 3) or min(mg, mo) == 0, (name, bad[r], i, g, o)
        assert abs(mg - mo) == 1, (name, bad[r], i, g, o)
        mid = (abs(F.E2M1[g]) + abs(F.E2M1[o])) / 2.0 * dd * np.sign(hv[r, i])
        assert abs(hv[r, i] - mid) <= eb[r, i] + 4 * U32 * abs(hv[r, i]), (name, bad[r], i, hv[r, i], mid)

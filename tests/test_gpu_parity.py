"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bit-exact: the NVFP4 quantizer's codes and scales, the routing ids and weights,
every field of the permutation metadata, the weight converter. Floating point:
the final bf16 outputs and the GEMM2 route rows within rel-L2 1e-2 (the
pages' rel-L2 probe criterion, the expert_tp page, "probe_rel_l2"); the
requantized intermediate is reported, and its scale bytes and codes must agree
except at rare fp32 rounding boundaries (several results are correct there)."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_route_amd import layer as LY
from nvfp4_block_scaled_route_amd import native as N
from nvfp4_block_scaled_route_amd import workloads as W
from oracle import formats as F
from oracle import layout as OL
from oracle.finalize import finalize as o_finalize
from oracle.layer import layer as o_layer, layer_sampled, quantize_input, rel_l2
from oracle.permute import permute as o_permute
from oracle.quant import quantize_nvfp4
from oracle.routing import route as o_route

from .gpu_common import (DEV, abs_gemm1, check_requant, dev, h_error_bound, host, queue_words, run_layer, say,
                         sync_counters, upload_weights)

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache[name] = W.make_inputs(W.WORKLOADS[name])
        return cache[name]
    return get


# ------------------------------------------------------------------ quantizer
def _gpu_quant(x_bf16: np.ndarray, gscale: float):
    T, H = x_bf16.shape
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=DEV)
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device=DEV)
    say(f"nvfp4_quant T={T} H={H} gscale={gscale}")
    N.nvfp4_quant(dev(x_bf16), dev(np.array([gscale], np.float32)), codes, sf)
    torch.cuda.synchronize()
    return host(codes), host(sf)


@pytest.mark.parametrize("name", W.ORDER)
def test_quant_bit_exact_on_workload(inputs, name):
    inp = inputs(name)
    codes, sf = _gpu_quant(inp.x_bf16, float(inp.a1_gscale[0]))
    oc, osf = quantize_input(inp)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)


def _edge_rows():
    rng = np.random.default_rng(11)
    rows = []
    z = np.zeros(64, np.float32)
    rows.append(z.copy())                                       # all zero
    r = z.copy(); r[5] = 7.0; rows.append(r)                    # single spike
    rows.append(np.full(64, -0.0, np.float32))                  # negative zeros
    rows.append(np.full(64, 3e-40, np.float32))                 # underflowing scale
    rows.append(np.array([2.0 ** -9 * 6 * (i % 3) for i in range(64)], np.float32))
    r = (F.E2M1[rng.integers(0, 16, 64)] * 0.75).astype(np.float32); r[::16] = 6 * 0.75
    rows.append(r)                                              # exact grid
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    r = np.tile(np.concatenate([mids, -mids]), 4); r[::16] = 6.0
    rows.append(r)                                              # ties
    rows.append(np.full(64, 3.0e38, np.float32))                # huge
    rows.append((rng.standard_normal(64) * 1e4).astype(np.float32))
    rows.append((rng.standard_normal(64) * 1e-6).astype(np.float32))
    x = np.stack(rows)
    return F.f32_to_bf16(x)


@pytest.mark.parametrize("gscale", [1.0, 0.37, 3.5, 448.0, 1e-3])
def test_quant_bit_exact_edge_blocks(gscale):
    x = _edge_rows()
    rng = np.random.default_rng(5)
    extra = F.f32_to_bf16((rng.standard_normal((37, 64 * 3)) *
                           np.exp2(rng.integers(-20, 20, (37, 1)))).astype(np.float32))
    for xb in (x, extra):
        codes, sf = _gpu_quant(xb, gscale)
        oc, osf = quantize_nvfp4(F.bf16_to_f64(xb).astype(np.float32), gscale)
        assert np.array_equal(sf, osf)
        assert np.array_equal(codes, oc)


def test_quant_all_bf16_patterns():
    """Every finite bf16 value passes through the quantizer, in blocks that
    mix magnitudes, at several global scales."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    bits = bits[np.isfinite(v)]
    rng = np.random.default_rng(2)
    for trial in range(3):
        perm = rng.permutation(bits.size)
        n = (bits.size // 64) * 64
        xb = bits[perm][:n].reshape(-1, 64)
        for g in (1.0, 2.0 ** -100, 5.25):
            codes, sf = _gpu_quant(xb, g)
            oc, osf = quantize_nvfp4(F.bf16_to_f64(xb).astype(np.float32), g)
            assert np.array_equal(sf, osf) and np.array_equal(codes, oc)


# ------------------------------------------------------------------ routing
def _gpu_route(logits, bias, K, tile_m, offset=0, local=None, padding=None, route_scale=1.0):
    T, E = logits.shape
    local = E if local is None else local
    L = N.moe_meta_layout_get(T, K, local, tile_m)
    ids = torch.full((T, K), 12345, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), 7.0, dtype=torch.float32, device=DEV)
    meta = torch.full((L.total_ints + 64,), -777, dtype=torch.int32, device=DEV)
    say(f"moe_route T={T} E={E} K={K} m={tile_m} local=[{offset},+{local})")
    N.moe_route(dev(logits), None if bias is None else dev(bias),
                None if padding is None else dev(padding.astype(np.uint8)), K, route_scale,
                tile_m, offset, local, ids, w, meta)
    torch.cuda.synchronize()
    return host(ids), host(w), host(meta), L


def _check_route(logits, bias, K, tile_m, offset=0, local=None, padding=None, route_scale=1.0):
    T, E = logits.shape
    local = E if local is None else local
    ids, w, meta, L = _gpu_route(logits, bias, K, tile_m, offset, local, padding, route_scale)
    oids, ow = o_route(logits, bias, K, route_scale, padding)
    assert np.array_equal(ids, oids)
    assert np.array_equal(w.view(np.uint32), ow.view(np.uint32))
    om = o_permute(oids, offset, local, tile_m)
    assert meta[L.num_tiles] == om["num_tiles"] and meta[L.total_rows] == om["total_rows"]
    assert np.array_equal(meta[L.expert_offsets:L.expert_offsets + local + 1], om["offsets"])
    assert np.array_equal(meta[L.expert_counts:L.expert_counts + local], om["counts"])
    assert np.array_equal(meta[L.exp2perm:L.exp2perm + T * K], om["exp2perm"].reshape(-1))
    assert np.array_equal(meta[L.perm2tok:L.perm2tok + L.rows_max], om["perm2tok"])
    assert np.array_equal(meta[L.tile_expert:L.tile_expert + L.tiles_max], om["tile_expert"])
    assert meta[L.sync_status] == 0 and not np.any(sync_counters(meta, L))
    assert not np.any(queue_words(meta, L))
    assert np.all(meta[L.total_ints:] == -777)                   # nothing written past the buffer
    return ids, w, meta


@pytest.mark.parametrize("name", W.ORDER)
def test_route_bit_exact_on_workload(inputs, name):
    inp = inputs(name)
    _check_route(inp.logits, inp.expert_bias, inp.wl.K, inp.wl.tile_m)


@pytest.mark.parametrize("T,E,K,m", [(1, 8, 1, 16), (7, 100, 5, 32), (9, 64, 8, 16),
                                     (300, 256, 6, 64), (33, 1024, 32, 256), (2048, 16, 4, 128)])
def test_route_shapes_bias_padding(T, E, K, m):
    rng = np.random.default_rng(T * 131 + E)
    logits = (rng.standard_normal((T, E)) * 8).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    pad = rng.random(T) < 0.1
    _check_route(logits, bias, K, m, padding=pad, route_scale=1.5)


def test_route_ties_and_wide_logits():
    rng = np.random.default_rng(3)
    T, E, K = 4096, 64, 8
    logits = rng.choice(np.array([-30, -1, 0, 0.5, 2, 30], np.float32), (T, E))
    _check_route(logits, None, K, 16)
    wide = rng.uniform(-90, 90, (T, E)).astype(np.float32)
    _check_route(wide, None, K, 16)


def test_route_sigmoid_bits_many_tokens():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((65536, 32)) * 6).astype(np.float32)
    _check_route(logits, None, 8, 128)


@pytest.mark.parametrize("T", [40, 600])
def test_route_expert_parallel_subset(T):
    """Experts outside [16, 32) are not served here: their routes map to -1
    (one-workgroup permutation at 320 routes, the grid-wide one at 4800)."""
    rng = np.random.default_rng(6 + T)
    logits = rng.standard_normal((T, 64)).astype(np.float32)
    _, _, meta = _check_route(logits, None, 8, 16, offset=16, local=16)


def test_route_zero_tokens():
    L = N.moe_meta_layout_get(0, 8, 64, 16)
    meta = torch.full((L.total_ints,), -5, dtype=torch.int32, device=DEV)
    ids = torch.empty((0, 8), dtype=torch.int32, device=DEV)
    w = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    N.moe_route(torch.empty((0, 64), dtype=torch.float32, device=DEV), None, None, 8, 1.0, 16, 0,
                64, ids, w, meta)
    torch.cuda.synchronize()
    m = host(meta)
    assert m[L.num_tiles] == 0 and m[L.total_rows] == 0
    assert np.all(m[L.expert_offsets:L.expert_offsets + 65] == 0)


@pytest.mark.parametrize("T,E,K,m", [(5, 256, 8, 16), (20, 512, 6, 32), (32, 128, 8, 16),
                                     (16, 3, 3, 16), (33, 200, 7, 16), (6, 48, 8, 16),
                                     (8, 100, 24, 16), (12, 64, 8, 16)])
def test_route_tied_keys_both_paths(T, E, K, m):
    """Many equal keys: the rank count (E <= 64) and the arg-max rounds (E > 64,
    2, 4 or 16 experts a lane) must both take ties to the lower index, in one
    workgroup (T <= 8) and in the top-k grid (T > 8); and the permutation by
    one wave (up to 128 routes), by the workgroup (8 tokens x 24: 192 routes,
    from the top-k ids in LDS) and after the grid (from global memory)."""
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.choice(np.array([-3, -0.5, 0, 0.25, 1, 4], np.float32), (T, E))
    bias = rng.choice(np.array([0.0, -0.0, 0.125], np.float32), E)
    pad = rng.random(T) < 0.15
    _check_route(logits, bias, K, m, padding=pad)


@pytest.mark.parametrize("T,H,E,K", [(8, 2048, 64, 8), (300, 256, 128, 8), (1, 64, 8, 2),
                                     (40, 4096, 300, 4)])
def test_route_quant_equals_separate_calls(T, H, E, K):
    rng = np.random.default_rng(T + H)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = W.to_bf16_bits((rng.standard_normal((T, H)) * 3).astype(np.float32))
    gscale = np.array([0.5], np.float32)
    pad = rng.random(T) < 0.2
    ids0, w0, meta0, L = _gpu_route(logits, None, K, 16, padding=pad)
    codes0, sf0 = _gpu_quant(x, float(gscale[0]))
    ids = torch.full((T, K), 12345, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), 7.0, dtype=torch.float32, device=DEV)
    meta = torch.full((L.total_ints + 64,), -777, dtype=torch.int32, device=DEV)
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=DEV)
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device=DEV)
    say(f"moe_route_quant T={T} H={H} E={E} K={K}")
    N.moe_route_quant(dev(logits), None, dev(pad.astype(np.uint8)), K, 1.0, 16, 0, E, ids, w,
                      meta, dev(x), dev(gscale), codes, sf)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids), ids0)
    assert np.array_equal(host(w).view(np.uint32), w0.view(np.uint32))
    assert np.array_equal(host(meta), meta0)
    assert np.array_equal(host(codes), codes0) and np.array_equal(host(sf), sf0)


# ------------------------------------------------------------------ weight converter
@pytest.mark.parametrize("E,H,I", [(3, 256, 128), (4, 512, 256), (2, 2048, 768), (1, 64, 64)])
def test_pack_bit_exact(E, H, I):
    rng = np.random.default_rng(E * H + I)
    w13c = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = rng.integers(0, 256, (E, 2 * I, H // 16), dtype=np.uint8)
    w2c = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = rng.integers(0, 256, (E, H, I // 16), dtype=np.uint8)
    say(f"moe_pack E={E} H={H} I={I}")
    w = LY.pack_weights(dev(w13c), dev(w13s), dev(w2c), dev(w2s),
                        *(torch.ones(E, device=DEV) for _ in range(3)))
    torch.cuda.synchronize()
    o13 = OL.convert_w13(w13c, w13s)
    o2 = OL.convert_w2(w2c, w2s)
    assert np.array_equal(host(w.w13).reshape(-1), o13[0].reshape(-1))
    assert np.array_equal(host(w.w13_sf).reshape(-1), o13[1].reshape(-1))
    assert np.array_equal(host(w.w2).reshape(-1), o2[0].reshape(-1))
    assert np.array_equal(host(w.w2_sf).reshape(-1), o2[1].reshape(-1))


# ------------------------------------------------------------------ finalize
@pytest.mark.parametrize("wbn,npart,use_norm", [(1, 1, True), (0, 1, True), (1, 8, True),
                                                (1, 1, False), (0, 3, False)])
def test_finalize_against_oracle(wbn, npart, use_norm):
    _finalize_case(wbn, npart, use_norm, 37, 8, 4096)


@pytest.mark.parametrize("K,H,npart", [(20, 16384, 1), (32, 2048, 1), (3, 64, 2), (9, 8200, 1)])
def test_finalize_batches_and_widths(K, H, npart):
    """More than one batch of 8 routes, two chunks per thread (H > 8192), a
    single-wave workgroup (H = 64), a width that leaves the last wave partial."""
    _finalize_case(1, npart, True, 5, K, H)


def _finalize_case(wbn, npart, use_norm, T, K, H):
    rng = np.random.default_rng(7 + npart + K + H)
    R = 400
    parts = [F.f32_to_bf16((rng.standard_normal((R, H)) * rng.uniform(0.1, 50)).astype(np.float32))
             for _ in range(npart)]
    e2p = rng.integers(-1, R, (T, K)).astype(np.int32)
    wts = rng.uniform(0, 1, (T, K)).astype(np.float32)
    nw = F.f32_to_bf16(rng.uniform(-0.1, 0.1, H).astype(np.float32)) if use_norm else None
    rows = torch.stack([dev(p) for p in parts])
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    say(f"moe_finalize T={T} K={K} H={H} partials={npart} wbn={wbn}")
    N.moe_finalize(rows, npart, rows.stride(0), dev(e2p), dev(wts),
                   None if nw is None else dev(nw), 1.0, 1e-6, wbn, T, K, H, out)
    torch.cuda.synchronize()
    got = F.bf16_to_f64(host(out))
    if npart > 1:
        want = o_finalize(None, e2p, wts, nw, 1.0, 1e-6, wbn, partials=parts)
    else:
        want = o_finalize(parts[0], e2p, wts, nw, 1.0, 1e-6, wbn)
    want = F.bf16_to_f64(want)
    assert rel_l2(got, want) < 1e-3
    # fp32 against fp64 norm arithmetic: at most one bf16 step of the row's
    # magnitude apart (the k-sum can cancel, so not of each element's own)
    scale = np.abs(want).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - want) <= scale * 2.0 ** -7)


# ------------------------------------------------------------------ whole layer
def _check_sync_words(res):
    """The expert step's waits all ended normally and its per-tile counters
    are back at zero (the next call on this metadata starts from them)."""
    assert res["sync_status"] == 0
    assert not np.any(res["sub_sync"])
    assert not np.any(res["tok_sync"])


def _compare_requant(res, ref, inp, rows_got, tokens, experts, name, a_codes=None, a_sf=None):
    """The kernel's intermediate at permuted rows rows_got against the oracle's
    for the same routes in the same order (ref: h, acc1, h_codes, h_sf), by the
    one-grid-step rule at rounding boundaries (the error bound is computed for
    the routes that differ only)."""
    if a_codes is None:
        a_codes, a_sf = quantize_input(inp)

    def eb_of(sel):
        abs_acc1 = abs_gemm1(a_codes, a_sf, tokens[sel], experts[sel], inp.w13_codes, inp.w13_sf)
        return h_error_bound(ref["acc1"][sel], abs_acc1, experts[sel], inp.g1_alphas, inp.g1_scale_c,
                             ref["h"][sel], inp.wl.H)

    check_requant(res["inter_codes"][rows_got], res["inter_sf"][rows_got], ref["h"], ref["h_codes"],
                  ref["h_sf"], eb_of, name)


def _compare_layer(res, ref, name, inp, tile_m=None):
    _check_sync_words(res)
    p = ref["rows_idx"]
    m = inp.wl.tile_m if tile_m is None else tile_m
    # routing and metadata: bit-exact
    assert np.array_equal(res["ids"], ref["ids"])
    assert np.array_equal(res["weights"].view(np.uint32), ref["weights"].view(np.uint32))
    assert np.array_equal(res["exp2perm"], ref["meta"]["exp2perm"])
    assert np.array_equal(res["perm2tok"], ref["meta"]["perm2tok"])
    assert np.array_equal(res["a_codes"], ref["a_codes"]) and np.array_equal(res["a_sf"], ref["a_sf"])
    # intermediate: equal except one grid step at fp32 rounding boundaries
    tokens = ref["meta"]["perm2tok"][p]
    experts = ref["meta"]["tile_expert"][p // m]
    _compare_requant(res, ref, inp, p, tokens, experts, name, ref["a_codes"], ref["a_sf"])
    got_rows, want_rows = F.bf16_to_f64(res["rows"][0][p]), F.bf16_to_f64(ref["rows"][p])
    rows_rel = rel_l2(got_rows, want_rows)
    out_rel = rel_l2(F.bf16_to_f64(res["out"]), F.bf16_to_f64(ref["out"]))
    # every block of up to 128 permuted rows (a tiled kernel's row block, a few
    # streaming tiles) on its own, so that one wrong block cannot hide in the total
    blk = p // 128
    worst = max(rel_l2(got_rows[blk == b], want_rows[blk == b]) for b in np.unique(blk))
    say(f"{name}: rows rel-L2 {rows_rel:.2e} (worst 128-row block {worst:.2e}), out rel-L2 {out_rel:.2e}")
    assert worst < TOL
    assert rows_rel < TOL
    assert out_rel < TOL
    return out_rel


@pytest.mark.parametrize("name", ["tiny", "decode_b8"])
def test_layer_parity_full_oracle(inputs, name):
    inp = inputs(name)
    res = run_layer(inp)
    ref = o_layer(inp)
    _compare_layer(res, ref, name, inp)


@pytest.mark.parametrize("T,H,I,E,K,m", [(256, 512, 256, 4, 2, 128), (200, 256, 512, 6, 3, 256),
                                         (96, 1024, 256, 3, 2, 128), (128, 768, 256, 2, 2, 128)])
def test_layer_parity_tiled_path(T, H, I, E, K, m):
    """Many routes per expert: the register-tiled MFMA kernels (every 128-row
    block of one expert, padding rows in every expert's last block, 1 to 4
    routed row tiles per block, column groups that do not fill a workgroup),
    whole layer against the oracle."""
    from oracle.layer import intermediate_amax
    wl = W.Workload(f"tiled_{T}_{H}_{I}_{E}_{K}_{m}", T=T, H=H, I=I, E=E, K=K, tile_m=m, seed=3)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    a2 = float(np.float32(2688.0 / intermediate_amax(probe)))
    inp = W.make_inputs(wl, a2_gscale=a2)
    assert T * K >= 32 * E                      # the tiled path's dispatch condition
    res = run_layer(inp)
    ref = o_layer(inp)
    _compare_layer(res, ref, wl.name, inp)


@pytest.mark.parametrize("T,H,I,E,K,m", [(6, 320, 192, 8, 2, 16), (5, 384, 256, 8, 3, 16),
                                         (7, 512, 768, 16, 4, 32), (3, 1024, 512, 4, 2, 16),
                                         (4, 512, 320, 8, 2, 16), (9, 768, 1280, 8, 3, 16),
                                         (6, 512, 256, 8, 2, 16), (5, 1024, 256, 8, 3, 32)])
def test_layer_parity_streaming_kernel_choices(T, H, I, E, K, m):
    """Few routes per expert, shapes that take each expert kernel: GEMM1 on the
    one-wave kernel (H % 256 != 0) or on the workgroup kernel with the LDS copy
    of the activation, GEMM2 likewise (I % 256 and H % 128), and both GEMMs in
    one launch where both workgroup forms apply (H % 256 == 0 and I % 256 == 0:
    GEMM2 weight preloads of 8 and 4 k-tiles, GEMM1 depths 8 and 4, and at
    I = 256 two output pairs a GEMM2 wave); two-launch pipeline depths 5
    (H/64), 3, 6 (I/64 = 12) and 8."""
    from oracle.layer import intermediate_amax
    wl = W.Workload(f"stream_{T}_{H}_{I}_{E}_{K}_{m}", T=T, H=H, I=I, E=E, K=K, tile_m=m, seed=5)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    a2 = float(np.float32(2688.0 / intermediate_amax(probe)))
    inp = W.make_inputs(wl, a2_gscale=a2)
    res = run_layer(inp)
    ref = o_layer(inp)
    _compare_layer(res, ref, wl.name, inp)


@pytest.mark.parametrize("tile_m", [32, 64, 256])
def test_layer_parity_other_tiles(inputs, tile_m):
    inp = inputs("decode_b8")
    res = run_layer(inp, tile_m=tile_m)
    ref = o_layer(inp, tile_m=tile_m)
    _compare_layer(res, ref, f"decode_b8 m={tile_m}", inp, tile_m)


def test_layer_parity_padding_tokens(inputs):
    inp = inputs("tiny")
    pad = np.array([False, True, False, False])
    res = run_layer(inp, is_padding=pad)
    ref = o_layer(inp, is_padding=pad)
    _compare_layer(res, ref, "tiny padded", inp)
    assert np.all(res["ids"][1] == -1) and np.all(F.bf16_to_f64(res["out"][1]) == 0)


@pytest.mark.slow
def test_layer_parity_decode_b64_zipf(inputs):
    inp = inputs("decode_b64_zipf")
    res = run_layer(inp)
    ref = o_layer(inp)
    _compare_layer(res, ref, "decode_b64_zipf", inp)
    counts = res["counts"]
    say(f"decode_b64_zipf: {int((counts > 0).sum())} experts touched, hottest {int(counts.max())} routes")


def _compare_sampled(res, inp, tokens, name):
    """The HIP layer's rows, intermediate and outputs for the given tokens against
    the oracle's sampled evaluation of the same tokens."""
    ref = layer_sampled(inp, tokens)
    e2p = res["exp2perm"][tokens]
    served = e2p >= 0
    assert np.array_equal(served, ref["served"])
    got_rows = F.bf16_to_f64(res["rows"][0][np.maximum(e2p, 0)])[served]
    want_rows = F.bf16_to_f64(ref["route_rows"])[served]
    rows_rel = rel_l2(got_rows, want_rows)
    out_rel = rel_l2(F.bf16_to_f64(res["out"][tokens]), F.bf16_to_f64(ref["out"]))
    say(f"{name}: sampled {len(tokens)} tokens, rows rel-L2 {rows_rel:.2e}, out rel-L2 {out_rel:.2e}")
    assert rows_rel < TOL and out_rel < TOL
    tt, kk = np.nonzero(served)
    _compare_requant(res, ref, inp, e2p[tt, kk], np.asarray(tokens)[tt], ref["ids"][tt, kk], name)
    return ref


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_layer_parity_prefill_all_tokens(inputs):
    """prefill_t4096 against the oracle's whole layer over all 4096 tokens (32768
    routes): routing, metadata and the quantizer bit-exact, the intermediate by
    the one-step rule, the rows of every routed 128-row block and the outputs
    within rel-L2 1e-2."""
    inp = inputs("prefill_t4096")
    res = run_layer(inp)
    say("prefill_t4096: oracle layer over all tokens")
    ref = o_layer(inp)
    _compare_layer(res, ref, "prefill_t4096", inp)


@pytest.mark.slow
def test_expert_tp_slices(inputs):
    """Expert TP on one GPU: 8 slices of all experts at I' = 256, each a byte view
    of the converted weights, give K-partial GEMM2 rows whose fp32 sum (one bf16
    rounding) matches the full-width rows; the finalize on the summed partials
    matches the oracle on all 32 tokens."""
    inp = inputs("expert_tp8_b32")
    wl = inp.wl
    w = upload_weights(inp)
    full = run_layer(inp, weights=w, tp=1)
    sliced = run_layer(inp, weights=w, tp=wl.tp)
    _check_sync_words(full)
    _check_sync_words(sliced)
    assert np.array_equal(full["exp2perm"], sliced["exp2perm"])
    p = np.nonzero(full["perm2tok"] >= 0)[0]
    part_sum = np.zeros((p.size, wl.H), np.float32)
    for r in range(wl.tp):
        part_sum = (part_sum + F.bf16_to_f64(sliced["rows"][r][p]).astype(np.float32)).astype(np.float32)
    summed = F.bf16_to_f64(F.f32_to_bf16(part_sum))
    probe = rel_l2(summed, F.bf16_to_f64(full["rows"][0][p]))
    out_rel = rel_l2(F.bf16_to_f64(sliced["out"]), F.bf16_to_f64(full["out"]))
    say(f"expert TP: slice-sum probe rel-L2 {probe:.2e}, finalize(partials) vs full {out_rel:.2e}")
    assert probe < TOL and out_rel < TOL
    tokens = np.arange(wl.T)
    ref = _compare_sampled(full, inp, tokens, "expert_tp8 full width")
    got = F.bf16_to_f64(sliced["out"][tokens])
    sliced_rel = rel_l2(got, F.bf16_to_f64(ref["out"]))
    say(f"expert TP: finalize(partials) vs oracle {sliced_rel:.2e}")
    assert sliced_rel < TOL


def _tiled_inputs():
    """Many routes per expert (the register-tiled form): T=256, H=512, I=256,
    E=4, top-2, 128-row tiles, the intermediate's global scale set from its amax."""
    from oracle.layer import intermediate_amax
    wl = W.Workload("tiled_256", T=256, H=512, I=256, E=4, K=2, tile_m=128, seed=3)
    probe = W.make_inputs(wl, a2_gscale=1.0)
    return W.make_inputs(wl, a2_gscale=float(np.float32(2688.0 / intermediate_amax(probe))))


@pytest.mark.parametrize("name,tile_m", [("decode_b8", 16), ("decode_b8", 64), ("tiny", 16), ("tiled_256", 128)])
def test_experts_repeated_calls_on_one_metadata(inputs, name, tile_m):
    """moe_experts_fwd called again and again on one routing (as a graph replay
    or the expert TP slices do), its intermediate and rows cleared in between:
    identical rows every time (decode_b8: the workgroup kernels with the LDS
    copy of the activation for both GEMMs; tiny: GEMM2 on the one-wave kernel,
    I/16 = 8 scale bytes per row; tiled_256: the persistent register-tiled
    kernel, whose work queues in the metadata must be back at 0 after every
    call)."""
    inp = _tiled_inputs() if name == "tiled_256" else inputs(name)
    wl = inp.wl
    w = upload_weights(inp)
    first = run_layer(inp, weights=w, tile_m=tile_m)
    shape = LY.LayerShape(wl.T, wl.H, wl.I, wl.E, wl.K, tile_m)
    bufs = LY.Buffers(shape, DEV)
    LY.run_layer(bufs, dev(inp.x_bf16), dev(inp.a1_gscale), dev(inp.logits), None, None, w,
                 dev(inp.norm_weight_bf16), wl.gain_center, wl.eps, bool(wl.weight_before_norm))
    valid = first["perm2tok"] >= 0
    say(f"repeated moe_experts_fwd {name} tile_m={tile_m}")
    L = bufs.layout
    for it in range(6):
        bufs.rows.fill_(0)
        bufs.inter_codes.fill_(0)
        bufs.inter_sf.fill_(0)
        N.moe_experts_fwd(bufs.a_codes, bufs.a_sf, bufs.meta, w, wl.T, wl.K, wl.E, wl.H, wl.I,
                          tile_m, bufs.inter_codes, bufs.inter_sf, bufs.rows[0], None)
        torch.cuda.synchronize()
        assert np.array_equal(host(bufs.rows)[0][valid], first["rows"][0][valid]), it
        meta = host(bufs.meta)
        assert meta[L.sync_status] == 0 and not np.any(sync_counters(meta, L)), it
        assert not np.any(queue_words(meta, L)), it


def test_layer_leaves_padding_rows_untouched_and_is_deterministic(inputs):
    inp = inputs("decode_b8")
    w = upload_weights(inp)
    a = run_layer(inp, weights=w, fill_rows=0x3F3F)
    b = run_layer(inp, weights=w, fill_rows=0x3F3F)
    pad = a["perm2tok"] < 0
    assert np.all(a["rows"][0][pad] == 0x3F3F)
    for k in ("rows", "out", "inter_codes", "inter_sf", "meta"):
        x, y = a[k], b[k]
        if k.startswith("inter"):
            x, y = x[~pad[:x.shape[0]]], y[~pad[:y.shape[0]]]
        assert np.array_equal(x, y), k

// moe_experts_fwd: the routed experts up to the GEMM2 rows -- the runner page,
// "MuseSparkTrtLlmNvFp4Experts.apply_routed" (TRT-LLM-gen op, do_finalize=False);
// the flashinfer_ops page, "routed_experts_from_metadata".
//
//   GEMM1  acc1 = A(t) . w13[e]^T       A: NVFP4 input row of token t
//   act    h = silu(acc_gate * g1_alphas[e]) * (acc_up * g1_scale_c[e]),
//          requantized to NVFP4 along I with global scale 1 (the intermediate's
//          global scale is folded into g1_scale_c: the runner page,
//          "process_weights_after_loading")
//   GEMM2  rows = bf16(hq . w2[e]^T * g2_alphas[e])
//
// Operands: every NVFP4 element e2m1 * e4m3 is exact in f16, so both GEMMs run
// v_mfma_f32_16x16x32_f16 with fp32 accumulation; both operands are decoded in
// registers from their codes (a pack-convert of 8 codes and one packed multiply
// by the block's e4m3 scale). Each lane of a wave owns whole 16-element blocks
// of K (lane (q, n) takes block q of every 64-wide k-tile, for row n of both
// operands), so one scale byte per operand and k-tile serves a lane, and the
// weight layout puts a lane's block of both row halves in one 16-byte slot.
//
// Decode is bound by the weight stream, so the kernels are built to keep HBM
// busy: one wave is one work unit, computes all of K on its own and writes its
// results itself -- no workgroup barrier, no cross-wave reduction. Units:
//   GEMM1 (16 routed rows, intermediate pair j): the 16 gate and 16 up weight
//     rows of intermediates [16j, 16j + 16) over K = H, so the SwiGLU and the
//     16-wide NVFP4 block of the requant complete in the wave;
//   GEMM2 (16 routed rows, output pair c): 32 output columns over K = I.
// A wave streams its unit's k-tiles through a D-stage register pipeline: the
// loads of k-tile c + D (16-byte weight slot, 2 weight scale bytes, 8 activation
// code bytes, 1 activation scale byte) are issued right after k-tile c is
// consumed, so D k-tiles of every wave are in flight at all times.
// Units are numbered row tile major; a unit finds its expert in the tile's
// metadata entry, which is -1 for every tile past the routed ones, so those
// waves exit at once. The expert kernels never read expert counts: a 16-row
// tile's padding rows have token -1 and are neither read nor written.
#include "experts.hpp"

namespace moe {

constexpr int kThreads = 256;              // 4 independent waves per workgroup
constexpr int kWavesPerBlock = kThreads / 64;

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One k-tile's operands of one lane.
struct Stage {
    uint4 w;        // weight slot: half 0 elements 0-7, 8-15, half 1 elements 0-7, 8-15
    uint32_t wsf;   // scale bytes of half 0 (bits 0-7) and half 1 (bits 8-15)
    uint2 a;        // activation block: elements 0-7, 8-15
    uint32_t asf;   // its scale byte
};

// Per-lane operand pointers of one unit; k-tile c is at +c * {1024, 128, 32, 4}.
// A lane whose activation row holds no route reads an in-bounds stand-in row:
// row m of an MFMA product depends on row m of A only, and such rows are never
// written, so their values do not matter (and nothing has to wait to mask them).
struct Streams {
    const uint8_t* wc;
    const uint8_t* ws;
    const uint8_t* ac;
    const uint8_t* as;
};

__device__ __forceinline__ void load_stage(Stage& st, const Streams& p, int c) {
    st.w = *reinterpret_cast<const uint4*>(p.wc + (int64_t)c * kSlotBytes);
    st.wsf = *reinterpret_cast<const uint16_t*>(p.ws + (int64_t)c * kSlotSfBytes);
    st.a = *reinterpret_cast<const uint2*>(p.ac + c * 32);
    st.asf = p.as[c * 4];
}

// acc0 += A . half0^T, acc1 += A . half1^T over one k-tile (two MFMA steps).
__device__ __forceinline__ void use_stage(const Stage& st, floatx4& acc0, floatx4& acc1) {
    const half2v ws = e4m3x2_to_f16(st.wsf);
    const half2v as = splat_lo(e4m3x2_to_f16(st.asf));
    const half2v s0 = splat_lo(ws), s1 = splat_hi(ws);
    {
        const half8 a = nvfp4x8_to_f16(st.a.x, as);
        acc0 = mfma16(a, nvfp4x8_to_f16(st.w.x, s0), acc0);
        acc1 = mfma16(a, nvfp4x8_to_f16(st.w.z, s1), acc1);
    }
    {
        const half8 a = nvfp4x8_to_f16(st.a.y, as);
        acc0 = mfma16(a, nvfp4x8_to_f16(st.w.y, s0), acc0);
        acc1 = mfma16(a, nvfp4x8_to_f16(st.w.w, s1), acc1);
    }
}

// All KT k-tiles of one unit through a D-deep pipeline (KT % D == 0, KT >= D).
template <int D>
__device__ __forceinline__ void stream_unit(const Streams& p, int KT, floatx4& acc0, floatx4& acc1) {
    Stage st[D];
    // Every stage's four loads issue together and in stage order, here and in
    // the loop, so that consuming stage d waits only for the loads issued before
    // it: vmcnt drains in issue order.
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_stage(st[d], p, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int c0 = 0; c0 + D < KT; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            use_stage(st[d], acc0, acc1);
            load_stage(st[d], p, c0 + D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        use_stage(st[d], acc0, acc1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The unit's 16-row tile: expert (-1: no unit) and the lane's row token.
struct RowTile {
    int e;
    int row0;
    int tok;                // token of row n (lane & 15), -1 for a padding row
    uint32_t vmask;         // bit m: row m holds a route
};

__device__ __forceinline__ RowTile row_tile(const ExpArgs& a, int sub, int n) {
    RowTile r;
    const int per_tile = a.tile_m >> 4;
    const int t = (int)((uint32_t)sub / (uint32_t)per_tile);
    // Both metadata loads go out before any decision: the tile index is clamped
    // so that they stay in bounds for units past the last tile.
    const int tc = min(t, (int)a.L.tiles_max - 1);
    r.row0 = tc * a.tile_m + (sub - t * per_tile) * 16;
    const int e = a.meta[a.L.tile_expert + tc];
    int tok = a.meta[a.L.perm2tok + r.row0 + n];
    if (tok >= a.T) tok = -1;
    r.tok = tok;
    r.vmask = (uint32_t)(__ballot(tok >= 0) & 0xFFFFull);
    r.e = (t < a.L.tiles_max && e >= 0 && e < a.E_local && r.vmask) ? e : -1;
    return r;
}

// ---------------------------------------------------------------- GEMM1 + SwiGLU + requant
template <int D>
__global__ void __launch_bounds__(kThreads) gemm1_kernel(ExpArgs a) {
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n1 = a.I >> 4;
    const int sub = (int)(unit / n1), j = (int)(unit - sub * n1);
    const RowTile rt = row_tile(a, sub, n);
    if (rt.e < 0) return;
    const int e = rt.e;
    Streams p;
    p.wc = a.w.w13 + e * a.w.w13_expert_stride_bytes + j * a.w.w13_pair_stride_bytes + lane * 16;
    p.ws = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + j * a.w.w13_sf_pair_stride_bytes + lane * 2;
    const int64_t tok = rt.tok >= 0 ? rt.tok : 0;
    p.ac = a.a_codes + tok * (a.H >> 1) + q * 8;
    p.as = a.a_sf + tok * (a.H >> 4) + q;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    stream_unit<D>(p, a.H >> 6, acc_g, acc_u);

    // lane (q, n) holds rows 4q + i of intermediate 16j + n
    const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const float g = acc_g[i] * ga;
        const float u = acc_u[i] * uc;
        const float h = g / (1.0f + expf(-g)) * u;
        const float amax = wave_max16(__builtin_fabsf(h));
        const BlockScale bs = nvfp4_block_scale(amax, 1.0f);
        const uint32_t code = nvfp4_code(h, bs);
        uint32_t b = code | (__shfl_xor(code, 1) << 4);      // even n: byte n/2
        b = b | (__shfl_xor(b, 2) << 8);                      // n % 4 == 0: 2 bytes
        b = b | (__shfl_xor(b, 4) << 16);                     // n % 8 == 0: 4 bytes
        if ((rt.vmask >> m) & 1u) {
            const int64_t row = rt.row0 + m;
            if ((n & 7) == 0)
                *reinterpret_cast<uint32_t*>(a.inter_codes + row * (a.I >> 1) + j * 8 + (n >> 1)) = b;
            if (n == 0) a.inter_sf[row * (a.I >> 4) + j] = (uint8_t)bs.byte;
        }
    }
}

// ---------------------------------------------------------------- GEMM2
template <int D>
__global__ void __launch_bounds__(kThreads) gemm2_kernel(ExpArgs a) {
    const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
    const uint32_t unit = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t n2 = a.H >> 5;
    const int sub = (int)(unit / n2), c = (int)(unit - sub * n2);
    const RowTile rt = row_tile(a, sub, n);
    if (rt.e < 0) return;
    const int e = rt.e;
    Streams p;
    p.wc = a.w.w2 + e * a.w.w2_expert_stride_bytes + c * a.w.w2_pair_stride_bytes + lane * 16;
    p.ws = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + c * a.w.w2_sf_pair_stride_bytes + lane * 2;
    const int64_t row = rt.row0 + n;   // the intermediate is in permuted row order
    p.ac = a.inter_codes + row * (a.I >> 1) + q * 8;
    p.as = a.inter_sf + row * (a.I >> 4) + q;
    floatx4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    stream_unit<D>(p, a.I >> 6, acc0, acc1);

    // lane (q, n) holds rows 4q + i of output columns 32c + n and 32c + 16 + n
    const float alpha = a.w.g2_alphas[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        if ((rt.vmask >> m) & 1u) {
            uint16_t* out = a.rows + (int64_t)(rt.row0 + m) * a.rows_stride + c * 32 + n;
            out[0] = (uint16_t)f32_to_bf16(acc0[i] * alpha);
            out[16] = (uint16_t)f32_to_bf16(acc1[i] * alpha);
        }
    }
}

// ---------------------------------------------------------------- launch
static int pipeline_depth(int kt) {
    const int depths[] = {8, 6, 4, 3, 2, 1};
    for (int d : depths)
        if (kt % d == 0) return d;
    return 1;
}

#define MOE_LAUNCH_DEPTHS(kernel)                                                         \
    static void launch_##kernel(int d, dim3 grid, hipStream_t s, const ExpArgs& a) {      \
        switch (d) {                                                                      \
            case 8: hipLaunchKernelGGL(kernel<8>, grid, dim3(kThreads), 0, s, a); break; \
            case 6: hipLaunchKernelGGL(kernel<6>, grid, dim3(kThreads), 0, s, a); break; \
            case 4: hipLaunchKernelGGL(kernel<4>, grid, dim3(kThreads), 0, s, a); break; \
            case 3: hipLaunchKernelGGL(kernel<3>, grid, dim3(kThreads), 0, s, a); break; \
            case 2: hipLaunchKernelGGL(kernel<2>, grid, dim3(kThreads), 0, s, a); break; \
            default: hipLaunchKernelGGL(kernel<1>, grid, dim3(kThreads), 0, s, a); break; \
        }                                                                                 \
    }
MOE_LAUNCH_DEPTHS(gemm1_kernel)
MOE_LAUNCH_DEPTHS(gemm2_kernel)
#undef MOE_LAUNCH_DEPTHS

}  // namespace moe

extern "C" int moe_experts_fwd(const uint8_t* a_codes, const uint8_t* a_sf, const int32_t* meta,
                               const moe_nvfp4_weights* w, int T, int K, int E_local, int H,
                               int I, int tile_m, uint8_t* inter_codes, uint8_t* inter_sf,
                               uint16_t* rows, int64_t rows_stride, void* stream) {
    using namespace moe;
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "moe_experts_fwd: T=%d K=%d E_local=%d out of range", T, K, E_local);
    if (H < 64 || H % 64 || I < 64 || I % 64)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: H=%d and I=%d must be multiples of 64", H, I);
    if (H > MOE_MAX_HIDDEN || I > MOE_MAX_HIDDEN)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: H=%d or I=%d above %d", H, I, MOE_MAX_HIDDEN);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: tile_m=%d must be a multiple of 16 in [16, 256]", tile_m);
    if (!w || !meta) return fail(MOE_EINVAL, "moe_experts_fwd: NULL weights or meta");
    if (T == 0) return MOE_OK;
    if (!a_codes || !a_sf || !inter_codes || !inter_sf || !rows || !w->w13 || !w->w13_sf ||
        !w->w2 || !w->w2_sf || !w->g1_alphas || !w->g1_scale_c || !w->g2_alphas)
        return fail(MOE_EINVAL, "moe_experts_fwd: NULL pointer");
    const void* ptrs[] = {a_codes, a_sf, meta, inter_codes, inter_sf, rows, w->w13, w->w13_sf,
                          w->w2, w->w2_sf, w->g1_alphas, w->g1_scale_c, w->g2_alphas};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return fail(MOE_EINVAL, "moe_experts_fwd: pointers must be 16-byte aligned");
    const int64_t kt1 = H / 64, kt2 = I / 64;
    if (w->w13_pair_stride_bytes < kt1 * kSlotBytes || w->w13_sf_pair_stride_bytes < kt1 * kSlotSfBytes ||
        w->w2_pair_stride_bytes < kt2 * kSlotBytes || w->w2_sf_pair_stride_bytes < kt2 * kSlotSfBytes ||
        w->w13_pair_stride_bytes % 16 || w->w13_sf_pair_stride_bytes % 16 ||
        w->w2_pair_stride_bytes % 16 || w->w2_sf_pair_stride_bytes % 16)
        return fail(MOE_EINVAL, "moe_experts_fwd: pair strides too small or not multiples of 16");
    if (w->w13_expert_stride_bytes < (int64_t)(I / 16) * w->w13_pair_stride_bytes ||
        w->w13_sf_expert_stride_bytes < (int64_t)(I / 16) * w->w13_sf_pair_stride_bytes ||
        w->w2_expert_stride_bytes < (int64_t)(H / 32) * w->w2_pair_stride_bytes ||
        w->w2_sf_expert_stride_bytes < (int64_t)(H / 32) * w->w2_sf_pair_stride_bytes ||
        w->w13_expert_stride_bytes % 16 || w->w13_sf_expert_stride_bytes % 16 ||
        w->w2_expert_stride_bytes % 16 || w->w2_sf_expert_stride_bytes % 16)
        return fail(MOE_EINVAL, "moe_experts_fwd: expert strides too small or not multiples of 16");
    if (rows_stride < H || rows_stride % 8)
        return fail(MOE_EINVAL, "moe_experts_fwd: rows_stride must be >= H and a multiple of 8");
    ExpArgs args;
    args.a_codes = a_codes; args.a_sf = a_sf; args.meta = meta;
    args.L = meta_layout(T, K, E_local, tile_m);
    args.w = *w; args.T = T; args.E_local = E_local; args.H = H; args.I = I; args.tile_m = tile_m;
    args.inter_codes = inter_codes; args.inter_sf = inter_sf; args.rows = rows;
    args.rows_stride = rows_stride;
    if (args.L.rows_max == 0) return MOE_OK;
    const int64_t subs = args.L.rows_max / 16;             // 16-row tiles, routed or not
    const int64_t units1 = subs * (I / 16), units2 = subs * (H / 32);
    const int64_t grid1 = (units1 + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t grid2 = (units2 + kWavesPerBlock - 1) / kWavesPerBlock;
    if (units1 > 0x7FFFFFFF || units2 > 0x7FFFFFFF)   // unit indices are 32-bit in the kernels
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: too many work units");
    hipStream_t s = (hipStream_t)stream;
    // Many routes per expert (on average a quarter of a 128-row block or more):
    // the GEMMs are MFMA-bound and take the register-tiled kernels.
    if (tiled_shape_ok(T, H, I, tile_m) && (int64_t)T * K >= (int64_t)32 * E_local) {
        launch_tiled(args, s);
        return check_launch("moe_experts_fwd (tiled)");
    }
    launch_gemm1_kernel(pipeline_depth((int)kt1), dim3((unsigned)grid1), s, args);
    int rc = check_launch("moe_experts_fwd (GEMM1)");
    if (rc) return rc;
    launch_gemm2_kernel(pipeline_depth((int)kt2), dim3((unsigned)grid2), s, args);
    return check_launch("moe_experts_fwd (GEMM2)");
}

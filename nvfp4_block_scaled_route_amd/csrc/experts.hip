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
// v_mfma_f32_16x16x32_f16 on decoded fragments with fp32 accumulation. One wave
// computes a 16-row M-subtile (16 permuted rows of one expert) against one
// 16-wide N group over the whole K; a lane decodes its own 8-element slices of
// both operands in registers. GEMM1's N group is 16 gate rows + the 16 up rows
// of the same intermediates (the converted layout's gated interleave), so the
// SwiGLU and the 16-wide NVFP4 block of the requant live in one wave.
#include "common.hpp"

namespace moe {

struct ExpArgs {
    const uint8_t* a_codes;
    const uint8_t* a_sf;
    const int32_t* meta;
    moe_meta_layout L;
    moe_nvfp4_weights w;
    int T, E_local, H, I, tile_m;
    uint8_t* inter_codes;
    uint8_t* inter_sf;
    uint16_t* rows;
    int64_t rows_stride;
};

constexpr int kWaves = 4;

// Rows that hold routes, from the metadata, never past the buffer bound: a
// metadata buffer from another call's shape cannot push an access out of bounds.
__device__ __forceinline__ int live_rows(const ExpArgs& a) {
    const int t = a.meta[a.L.total_rows];
    return t < (int)a.L.rows_max ? t : (int)a.L.rows_max;
}

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// GEMM1 + SwiGLU + requant. grid (ceil(I/16 / kWaves), rows_max / 16).
__global__ void __launch_bounds__(64 * kWaves) gemm1_swiglu_kernel(ExpArgs a) {
    const int row0 = blockIdx.y * 16;
    if (row0 + 16 > live_rows(a)) return;
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * kWaves + (threadIdx.x >> 6);   // intermediate group
    if (j >= a.I / 16) return;
    const int e = a.meta[a.L.tile_expert + row0 / a.tile_m];
    if (e < 0 || e >= a.E_local) return;
    const int n = lane & 15, q = lane >> 4;
    int tok = a.meta[a.L.perm2tok + row0 + n];                // A row m = n
    if (tok >= a.T) tok = -1;
    const int H = a.H;
    const uint8_t* acode = a.a_codes + (int64_t)(tok < 0 ? 0 : tok) * (H / 2);
    const uint8_t* asf = a.a_sf + (int64_t)(tok < 0 ? 0 : tok) * (H / 16);
    const uint8_t* wg = a.w.w13 + e * a.w.w13_expert_stride_bytes + (int64_t)(2 * j) * a.w.w13_group_stride_bytes;
    const uint8_t* wu = wg + a.w.w13_group_stride_bytes;
    const uint8_t* sg = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + (int64_t)(2 * j) * a.w.w13_sf_group_stride_bytes;
    const uint8_t* su = sg + a.w.w13_sf_group_stride_bytes;
    const int lane_code = lane * 8;
    const int lane_sf = ((q >> 1) * 16 + n) * 2;
    floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
    const int ktiles = H / 64;
    for (int c = 0; c < ktiles; ++c) {
        const uint2 cg = *reinterpret_cast<const uint2*>(wg + c * 512 + lane_code);
        const uint2 cu = *reinterpret_cast<const uint2*>(wu + c * 512 + lane_code);
        const uint32_t fg = *reinterpret_cast<const uint16_t*>(sg + c * 64 + lane_sf);
        const uint32_t fu = *reinterpret_cast<const uint16_t*>(su + c * 64 + lane_sf);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int k = c * 64 + s * 32 + q * 8;
            half8 av = {0, 0, 0, 0, 0, 0, 0, 0};
            if (tok >= 0)
                av = nvfp4x8_to_f16(*reinterpret_cast<const uint32_t*>(acode + k / 2), e4m3_to_f16(asf[k / 16]));
            const half8 bg = nvfp4x8_to_f16(s ? cg.y : cg.x, e4m3_to_f16((fg >> (8 * s)) & 0xFFu));
            const half8 bu = nvfp4x8_to_f16(s ? cu.y : cu.x, e4m3_to_f16((fu >> (8 * s)) & 0xFFu));
            acc_g = mfma16(av, bg, acc_g);
            acc_u = mfma16(av, bu, acc_u);
        }
    }
    // Epilogue: lane (q, n) holds rows 4q+i of intermediate 16j+n.
    const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const int p = row0 + m;
        const int ptok = __shfl(tok, m);
        const float g = acc_g[i] * ga;
        const float u = acc_u[i] * uc;
        const float h = g / (1.0f + expf(-g)) * u;
        const float amax = wave_max16(__builtin_fabsf(h));
        const BlockScale bs = nvfp4_block_scale(amax, 1.0f);
        const uint32_t code = nvfp4_code(h, bs);
        uint32_t b = code | (__shfl_xor(code, 1) << 4);         // even n: byte n/2
        b = b | (__shfl_xor(b, 2) << 8);                         // n % 4 == 0: 2 bytes
        b = b | (__shfl_xor(b, 4) << 16);                        // n % 8 == 0: 4 bytes
        if (ptok >= 0) {
            if ((n & 7) == 0)
                *reinterpret_cast<uint32_t*>(a.inter_codes + (int64_t)p * (a.I / 2) + j * 8 + (n >> 1)) = b;
            if (n == 0) a.inter_sf[(int64_t)p * (a.I / 16) + j] = (uint8_t)bs.byte;
        }
    }
}

// GEMM2. grid (ceil(H/16 / kWaves), rows_max / 16).
__global__ void __launch_bounds__(64 * kWaves) gemm2_kernel(ExpArgs a) {
    const int row0 = blockIdx.y * 16;
    if (row0 + 16 > live_rows(a)) return;
    const int lane = threadIdx.x & 63;
    const int g = blockIdx.x * kWaves + (threadIdx.x >> 6);   // output column group
    if (g >= a.H / 16) return;
    const int e = a.meta[a.L.tile_expert + row0 / a.tile_m];
    if (e < 0 || e >= a.E_local) return;
    const int n = lane & 15, q = lane >> 4;
    const int I = a.I;
    const int prow = row0 + n;
    const bool valid = a.meta[a.L.perm2tok + prow] >= 0;
    const uint8_t* hcode = a.inter_codes + (int64_t)prow * (I / 2);
    const uint8_t* hsf = a.inter_sf + (int64_t)prow * (I / 16);
    const uint8_t* wb = a.w.w2 + e * a.w.w2_expert_stride_bytes + (int64_t)g * a.w.w2_group_stride_bytes;
    const uint8_t* sb = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + (int64_t)g * a.w.w2_sf_group_stride_bytes;
    const int lane_code = lane * 8;
    const int lane_sf = ((q >> 1) * 16 + n) * 2;
    floatx4 acc = {0, 0, 0, 0};
    const int ktiles = I / 64;
    for (int c = 0; c < ktiles; ++c) {
        const uint2 cb = *reinterpret_cast<const uint2*>(wb + c * 512 + lane_code);
        const uint32_t fb = *reinterpret_cast<const uint16_t*>(sb + c * 64 + lane_sf);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int k = c * 64 + s * 32 + q * 8;
            half8 av = {0, 0, 0, 0, 0, 0, 0, 0};
            if (valid)
                av = nvfp4x8_to_f16(*reinterpret_cast<const uint32_t*>(hcode + k / 2), e4m3_to_f16(hsf[k / 16]));
            const half8 bv = nvfp4x8_to_f16(s ? cb.y : cb.x, e4m3_to_f16((fb >> (8 * s)) & 0xFFu));
            acc = mfma16(av, bv, acc);
        }
    }
    const float alpha = a.w.g2_alphas[e];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = row0 + 4 * q + i;
        const bool pv = __shfl((int)valid, 4 * q + i) != 0;
        if (pv) a.rows[(int64_t)p * a.rows_stride + g * 16 + n] = (uint16_t)f32_to_bf16(acc[i] * alpha);
    }
}

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
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: tile_m=%d must be a multiple of 16 in [16, 256]", tile_m);
    if (!w || !meta) return fail(MOE_EINVAL, "moe_experts_fwd: NULL weights or meta");
    if (T == 0) return MOE_OK;
    if (!a_codes || !a_sf || !inter_codes || !inter_sf || !rows || !w->w13 || !w->w13_sf ||
        !w->w2 || !w->w2_sf || !w->g1_alphas || !w->g1_scale_c || !w->g2_alphas)
        return fail(MOE_EINVAL, "moe_experts_fwd: NULL pointer");
    const void* ptrs[] = {a_codes, a_sf, meta, inter_codes, inter_sf, rows, w->w13, w->w13_sf,
                          w->w2, w->w2_sf, w->g1_alphas, w->g1_scale_c, w->g2_alphas};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(MOE_EINVAL, "moe_experts_fwd: pointers must be 16-byte aligned");
    const int64_t w13_gmin = (int64_t)(H / 64) * 512, w13s_gmin = (int64_t)(H / 64) * 64;
    const int64_t w2_gmin = (int64_t)(I / 64) * 512, w2s_gmin = (int64_t)(I / 64) * 64;
    if (w->w13_group_stride_bytes < w13_gmin || w->w13_sf_group_stride_bytes < w13s_gmin ||
        w->w2_group_stride_bytes < w2_gmin || w->w2_sf_group_stride_bytes < w2s_gmin ||
        w->w13_group_stride_bytes % 16 || w->w13_sf_group_stride_bytes % 16 ||
        w->w2_group_stride_bytes % 16 || w->w2_sf_group_stride_bytes % 16)
        return fail(MOE_EINVAL, "moe_experts_fwd: group strides too small or not multiples of 16");
    if (w->w13_expert_stride_bytes < (int64_t)(2 * I / 16) * w->w13_group_stride_bytes ||
        w->w13_sf_expert_stride_bytes < (int64_t)(2 * I / 16) * w->w13_sf_group_stride_bytes ||
        w->w2_expert_stride_bytes < (int64_t)(H / 16) * w->w2_group_stride_bytes ||
        w->w2_sf_expert_stride_bytes < (int64_t)(H / 16) * w->w2_sf_group_stride_bytes ||
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
    const int64_t subtiles = args.L.rows_max / 16;
    if (subtiles == 0) return MOE_OK;
    if (subtiles > 65535) return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: too many rows");
    hipStream_t s = (hipStream_t)stream;
    const int g1x = (I / 16 + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(gemm1_swiglu_kernel, dim3(g1x, (unsigned)subtiles), dim3(64 * kWaves), 0, s, args);
    int rc = check_launch("moe_experts_fwd (GEMM1)");
    if (rc) return rc;
    const int g2x = (H / 16 + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(gemm2_kernel, dim3(g2x, (unsigned)subtiles), dim3(64 * kWaves), 0, s, args);
    return check_launch("moe_experts_fwd (GEMM2)");
}

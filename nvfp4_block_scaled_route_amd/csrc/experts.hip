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
// v_mfma_f32_16x16x32_f16 with fp32 accumulation. The weights are decoded in
// registers (pack-convert of 8 codes + one packed multiply by the e4m3 scale);
// the activation side arrives already expanded to f16 -- the input by
// nvfp4_quant, the intermediate by GEMM1's epilogue -- so it is decoded once per
// element, not once per weight tile that meets it.
//
// Two persistent launches, GEMM1 then GEMM2 (the kernel boundary is what makes
// the intermediate written by one CU visible to the others: the 8 XCDs' L2
// caches are not coherent with each other inside a kernel, and agent-scope
// fences would write back or invalidate a whole L2 per unit). Work units:
//   GEMM1 unit (expert e, j): 16 gate rows + the 16 up rows of the same
//     intermediates (one gated-interleave row-group pair), all of K = H, so the
//     SwiGLU and the 16-wide NVFP4 block of the requant complete in the unit;
//   GEMM2 unit (expert e, 2 row groups = 32 output columns), all of K = I.
// Only experts with routes have units; every workgroup builds the same list of
// them from the metadata. A launch holds about as many workgroups as the chip
// keeps resident and workgroup b takes units b, b + grid, ... : consecutive
// workgroups stream neighbouring rows of one expert at the same time, and no
// workgroup is ever dispatched for an expert without routes.
// Inside a unit the waves split K; each wave issues all of its weight loads
// before any arithmetic; the expert's routes are then taken 16 rows (one MFMA
// M tile) at a time against the packed weights held in registers, so a unit
// streams its weights exactly once whatever the number of routes. K-split
// partial sums meet in LDS in a fixed order (deterministic results).
#include "common.hpp"

namespace moe {

struct ExpArgs {
    const uint16_t* a_dq;
    const int32_t* meta;
    moe_meta_layout L;
    moe_nvfp4_weights w;
    int T, E_local, H, I, tile_m;
    uint8_t* inter_codes;
    uint8_t* inter_sf;
    uint16_t* inter_dq;
    uint16_t* rows;
    int64_t rows_stride;
};

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kSplit1 = 8;                 // GEMM1: waves splitting K
constexpr int kGroups2 = 2, kSplit2 = 4;   // GEMM2: row groups x K parts
constexpr int kMaxKt = 16;                 // k-tiles per wave: H <= 8192, I <= 4096
constexpr int kWgPerCu = 2;

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Activation-side fragment of K step s of k-tile c: 8 f16 values of a row
// (lane (q, n) reads row n at column c*64 + s*32 + q*8); zeros without a route.
__device__ __forceinline__ half8 act_load(const uint16_t* row, bool valid, int c, int s, int q) {
    half8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (valid) v = *reinterpret_cast<const half8*>(row + c * 64 + s * 32 + q * 8);
    return v;
}

// Weight fragment of K step s from a lane's packed k-tile (codes of both steps,
// the two scale bytes).
__device__ __forceinline__ half8 w_frag(uint2 codes, uint32_t sf2, int s) {
    const half2v sc = e4m3x2_to_f16(sf2);
    return nvfp4x8_to_f16(s ? codes.y : codes.x, s ? splat_hi(sc) : splat_lo(sc));
}

// The expert's routed rows [begin, begin + count), checked against the buffer
// bound so that a metadata buffer of another shape cannot cause a stray access.
__device__ __forceinline__ bool expert_rows(const ExpArgs& a, int e, int& begin, int& count) {
    count = a.meta[a.L.expert_counts + e];
    begin = a.meta[a.L.expert_offsets + e];
    return count > 0 && begin >= 0 && (int64_t)begin + count <= a.L.rows_max;
}

// ---------------------------------------------------------------- GEMM1 + SwiGLU + requant unit
template <int KT>
__device__ void gemm1_unit(const ExpArgs& a, int e, int j, float (*red)[8][64]) {
    int begin, count;
    if (!expert_rows(a, e, begin, count)) return;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, q = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int H = a.H, ktiles = H / 64;
    const int per = (ktiles + kSplit1 - 1) / kSplit1;
    const int c0 = w * per;
    const int nk = max(0, min(per, ktiles - c0));
    const uint8_t* wg = a.w.w13 + e * a.w.w13_expert_stride_bytes + (int64_t)(2 * j) * a.w.w13_group_stride_bytes + c0 * 512 + lane * 8;
    const uint8_t* wu = wg + a.w.w13_group_stride_bytes;
    const uint8_t* sg = a.w.w13_sf + e * a.w.w13_sf_expert_stride_bytes + (int64_t)(2 * j) * a.w.w13_sf_group_stride_bytes + c0 * 64 + ((q >> 1) * 16 + n) * 2;
    const uint8_t* su = sg + a.w.w13_sf_group_stride_bytes;
    uint2 cg[KT], cu[KT];
    uint32_t fg[KT], fu[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        if (t < nk) {
            cg[t] = *reinterpret_cast<const uint2*>(wg + t * 512);
            cu[t] = *reinterpret_cast<const uint2*>(wu + t * 512);
            fg[t] = *reinterpret_cast<const uint16_t*>(sg + t * 64);
            fu[t] = *reinterpret_cast<const uint16_t*>(su + t * 64);
        } else {
            cg[t] = cu[t] = make_uint2(0, 0);
            fg[t] = fu[t] = 0;
        }
    }
    const float ga = a.w.g1_alphas[e], uc = a.w.g1_scale_c[e];
    for (int r0 = 0; r0 < count; r0 += 16) {
        const int row0 = begin + r0;
        int tok = r0 + n < count ? a.meta[a.L.perm2tok + row0 + n] : -1;   // A row m = n
        if (tok >= a.T) tok = -1;
        const bool valid = tok >= 0;
        const uint16_t* arow = a.a_dq + (int64_t)(valid ? tok : 0) * H;
        floatx4 acc_g = {0, 0, 0, 0}, acc_u = {0, 0, 0, 0};
        // the activation is read two k-tiles ahead of its use
        half8 av[KT][2];
#pragma unroll
        for (int t = 0; t < 2 && t < KT; ++t)
            if (t < nk) { av[t][0] = act_load(arow, valid, c0 + t, 0, q); av[t][1] = act_load(arow, valid, c0 + t, 1, q); }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (t < nk) {
                if (t + 2 < KT && t + 2 < nk) {
                    av[t + 2][0] = act_load(arow, valid, c0 + t + 2, 0, q);
                    av[t + 2][1] = act_load(arow, valid, c0 + t + 2, 1, q);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    acc_g = mfma16(av[t][s], w_frag(cg[t], fg[t], s), acc_g);
                    acc_u = mfma16(av[t][s], w_frag(cu[t], fu[t], s), acc_u);
                    __builtin_amdgcn_sched_barrier(0);   // decode one K step at a time
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[w][i][lane] = acc_g[i];
            red[w][4 + i][lane] = acc_u[i];
        }
        __syncthreads();
        if (w < 4) {
            // wave w finishes row 4q + w of the 16-row tile for intermediate 16j + n
            const int i = w;
            float g = 0.0f, u = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kSplit1; ++ww) {
                g += red[ww][i][lane];
                u += red[ww][4 + i][lane];
            }
            const int m = 4 * q + i;
            const int p = row0 + m;
            g *= ga;
            u *= uc;
            const float h = g / (1.0f + expf(-g)) * u;
            const float amax = wave_max16(__builtin_fabsf(h));
            const BlockScale bs = nvfp4_block_scale(amax, 1.0f);
            const uint32_t code = nvfp4_code(h, bs);
            uint32_t b = code | (__shfl_xor(code, 1) << 4);      // even n: byte n/2
            b = b | (__shfl_xor(b, 2) << 8);                      // n % 4 == 0: 2 bytes
            b = b | (__shfl_xor(b, 4) << 16);                     // n % 8 == 0: 4 bytes
            if (r0 + m < count) {
                if ((n & 7) == 0)
                    *reinterpret_cast<uint32_t*>(a.inter_codes + (int64_t)p * (a.I / 2) + j * 8 + (n >> 1)) = b;
                if (n == 0) a.inter_sf[(int64_t)p * (a.I / 16) + j] = (uint8_t)bs.byte;
                // the exact f16 expansion e2m1(code) * e4m3(scale): GEMM2's operand
                const _Float16 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(code, 1.0f, 0)[0] *
                                   e4m3x2_to_f16(bs.byte)[0];
                a.inter_dq[(int64_t)p * a.I + j * 16 + n] = *reinterpret_cast<const uint16_t*>(&v);
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- GEMM2 unit
template <int KT>
__device__ void gemm2_unit(const ExpArgs& a, int e, int gq, float (*red)[8][64]) {
    int begin, count;
    if (!expert_rows(a, e, begin, count)) return;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, q = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int gi = w % kGroups2, ks = w / kGroups2;
    const int g = gq * kGroups2 + gi;
    const bool gvalid = g < a.H / 16;
    const int I = a.I, ktiles = I / 64;
    const int per = (ktiles + kSplit2 - 1) / kSplit2;
    const int c0 = ks * per;
    const int nk = gvalid ? max(0, min(per, ktiles - c0)) : 0;
    const uint8_t* wb = a.w.w2 + e * a.w.w2_expert_stride_bytes + (int64_t)g * a.w.w2_group_stride_bytes + c0 * 512 + lane * 8;
    const uint8_t* sb = a.w.w2_sf + e * a.w.w2_sf_expert_stride_bytes + (int64_t)g * a.w.w2_sf_group_stride_bytes + c0 * 64 + ((q >> 1) * 16 + n) * 2;
    uint2 cb[KT];
    uint32_t fb[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        if (t < nk) {
            cb[t] = *reinterpret_cast<const uint2*>(wb + t * 512);
            fb[t] = *reinterpret_cast<const uint16_t*>(sb + t * 64);
        } else {
            cb[t] = make_uint2(0, 0);
            fb[t] = 0;
        }
    }
    const float alpha = a.w.g2_alphas[e];
    for (int r0 = 0; r0 < count; r0 += 16) {
        const int row0 = begin + r0;
        const bool valid = r0 + n < count;                       // A row m = n
        const uint16_t* hrow = a.inter_dq + (int64_t)(row0 + n) * I;
        floatx4 acc = {0, 0, 0, 0};
        half8 av[KT][2];
#pragma unroll
        for (int t = 0; t < 2 && t < KT; ++t)
            if (t < nk) { av[t][0] = act_load(hrow, valid, c0 + t, 0, q); av[t][1] = act_load(hrow, valid, c0 + t, 1, q); }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (t < nk) {
                if (t + 2 < KT && t + 2 < nk) {
                    av[t + 2][0] = act_load(hrow, valid, c0 + t + 2, 0, q);
                    av[t + 2][1] = act_load(hrow, valid, c0 + t + 2, 1, q);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    acc = mfma16(av[t][s], w_frag(cb[t], fb[t], s), acc);
                    __builtin_amdgcn_sched_barrier(0);   // decode one K step at a time
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][i][lane] = acc[i];
        __syncthreads();
        // wave w = (gi, ks) finishes rows 4q + i, i = ks * 4 / kSplit2 + ii, column 16g + n
#pragma unroll
        for (int ii = 0; ii < 4 / kSplit2; ++ii) {
            const int i = ks * (4 / kSplit2) + ii;
            float v = 0.0f;
#pragma unroll
            for (int kk = 0; kk < kSplit2; ++kk) v += red[kk * kGroups2 + gi][i][lane];
            const int m = 4 * q + i;
            if (gvalid && r0 + m < count)
                a.rows[(int64_t)(row0 + m) * a.rows_stride + g * 16 + n] = (uint16_t)f32_to_bf16(v * alpha);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- the persistent launches
// The experts with routes, ascending, into s_act (the same list in every
// workgroup); returns their number.
__device__ int active_experts(const ExpArgs& a, int* s_act, int* s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int El = a.E_local;
    const int per = (El + kThreads - 1) / kThreads;
    const int e0 = tid * per, e1 = min(El, e0 + per);
    int mine = 0;
    for (int e = e0; e < e1; ++e) mine += a.meta[a.L.expert_counts + e] > 0;
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) s_wave[w] = incl;
    __syncthreads();
    int base = 0, nact = 0;
    for (int ww = 0; ww < kWaves; ++ww) { if (ww < w) base += s_wave[ww]; nact += s_wave[ww]; }
    int pos = base + incl - mine;
    for (int e = e0; e < e1; ++e)
        if (a.meta[a.L.expert_counts + e] > 0) s_act[pos++] = e;
    __syncthreads();
    return nact;
}

template <int KT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KT <= 8 ? 4 : 2)))
gemm1_kernel(ExpArgs a) {
    __shared__ float red[kWaves][8][64];
    __shared__ int s_act[MOE_MAX_EXPERTS];
    __shared__ int s_wave[kWaves];
    const int nact = active_experts(a, s_act, s_wave);
    const int n1 = a.I / 16;
    for (int u = blockIdx.x; u < nact * n1; u += gridDim.x) gemm1_unit<KT>(a, s_act[u / n1], u % n1, red);
}

template <int KT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KT <= 8 ? 4 : 2)))
gemm2_kernel(ExpArgs a) {
    __shared__ float red[kWaves][8][64];
    __shared__ int s_act[MOE_MAX_EXPERTS];
    __shared__ int s_wave[kWaves];
    const int nact = active_experts(a, s_act, s_wave);
    const int n2 = (a.H / 16 + kGroups2 - 1) / kGroups2;
    for (int u = blockIdx.x; u < nact * n2; u += gridDim.x) gemm2_unit<KT>(a, s_act[u / n2], u % n2, red);
}

static int kt_bucket(int per) { return per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16; }

static void launch_gemm1(int kt, dim3 grid, hipStream_t s, const ExpArgs& a) {
    switch (kt) {
        case 2: hipLaunchKernelGGL(gemm1_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(gemm1_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL(gemm1_kernel<8>, grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL(gemm1_kernel<16>, grid, dim3(kThreads), 0, s, a); break;
    }
}

static void launch_gemm2(int kt, dim3 grid, hipStream_t s, const ExpArgs& a) {
    switch (kt) {
        case 2: hipLaunchKernelGGL(gemm2_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(gemm2_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL(gemm2_kernel<8>, grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL(gemm2_kernel<16>, grid, dim3(kThreads), 0, s, a); break;
    }
}

static int cu_count() {
    static thread_local int cached_dev = -1, cached = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached_dev = dev;
        cached = n;
    }
    return cached;
}

}  // namespace moe

extern "C" int moe_experts_fwd(const uint16_t* a_dq, const int32_t* meta,
                               const moe_nvfp4_weights* w, int T, int K, int E_local, int H,
                               int I, int tile_m, uint8_t* inter_codes, uint8_t* inter_sf,
                               uint16_t* inter_dq, uint16_t* rows, int64_t rows_stride,
                               void* stream) {
    using namespace moe;
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK || E_local < 1 || E_local > MOE_MAX_EXPERTS)
        return fail(MOE_EINVAL, "moe_experts_fwd: T=%d K=%d E_local=%d out of range", T, K, E_local);
    if (H < 64 || H % 64 || I < 64 || I % 64)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: H=%d and I=%d must be multiples of 64", H, I);
    if (H > 64 * kSplit1 * kMaxKt || I > 64 * kSplit2 * kMaxKt)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: H=%d (max %d) or I=%d (max %d) too large", H,
                    64 * kSplit1 * kMaxKt, I, 64 * kSplit2 * kMaxKt);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "moe_experts_fwd: tile_m=%d must be a multiple of 16 in [16, 256]", tile_m);
    if (!w || !meta) return fail(MOE_EINVAL, "moe_experts_fwd: NULL weights or meta");
    if (T == 0) return MOE_OK;
    if (!a_dq || !inter_codes || !inter_sf || !inter_dq || !rows || !w->w13 || !w->w13_sf ||
        !w->w2 || !w->w2_sf || !w->g1_alphas || !w->g1_scale_c || !w->g2_alphas)
        return fail(MOE_EINVAL, "moe_experts_fwd: NULL pointer");
    const void* ptrs[] = {a_dq, meta, inter_codes, inter_sf, inter_dq, rows, w->w13,
                          w->w13_sf, w->w2, w->w2_sf, w->g1_alphas, w->g1_scale_c, w->g2_alphas};
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
    args.a_dq = a_dq; args.meta = meta;
    args.L = meta_layout(T, K, E_local, tile_m);
    args.w = *w; args.T = T; args.E_local = E_local; args.H = H; args.I = I; args.tile_m = tile_m;
    args.inter_codes = inter_codes; args.inter_sf = inter_sf; args.inter_dq = inter_dq; args.rows = rows;
    args.rows_stride = rows_stride;
    if (args.L.rows_max == 0) return MOE_OK;
    // About as many workgroups as stay resident, never more than there can be units.
    const int64_t experts_max = min((int64_t)E_local, (int64_t)T * K);
    const int64_t resident = (int64_t)cu_count() * kWgPerCu;
    const int grid1 = (int)min(resident, experts_max * (I / 16));
    const int grid2 = (int)min(resident, experts_max * ((H / 16 + kGroups2 - 1) / kGroups2));
    hipStream_t s = (hipStream_t)stream;
    launch_gemm1(kt_bucket((H / 64 + kSplit1 - 1) / kSplit1), dim3(grid1), s, args);
    int rc = check_launch("moe_experts_fwd (GEMM1)");
    if (rc) return rc;
    launch_gemm2(kt_bucket((I / 64 + kSplit2 - 1) / kSplit2), dim3(grid2), s, args);
    return check_launch("moe_experts_fwd (GEMM2)");
}

// moe_router_logits / moe_router_route: the router's linear layer (fp32 input,
// fp32 weight with the output multiplier folded in, fp32 logits) and the full
// routing chain, logits then top-k routing -- the model page, "MuseSpark1xMoE"
// (GateLinear with fp32 parameters and output, "_load_router_weight",
// "wants_fp32_router_input") and "_route_topk_and_pool" (router, then
// "_compute_routing").
//
// Each logit is the fp32 rounding of the dot product accumulated in fp64: the
// products of two fp32 values are exact in fp64, so the only error before the
// final rounding is that of the fp64 sums (about 2^-53 relative per step).
//
// Up to 256 tokens, one wave computes 8 tokens x 1 expert over all of D: per round a lane loads
// 4 consecutive weights and the same 4 columns of the 8 token rows (16-byte
// loads, a wave covering 256 consecutive columns), four rounds' loads issued
// together (decode is bound by the latency of these loads, not their bytes),
// then the 8 sums are reduced across the wave. A workgroup's 4 waves take 4 consecutive experts of the same
// 8 tokens, so the token rows they all read are shared in the CU's cache. At
// decode sizes the weight ([E, D] fp32) is read once from memory.
#include "common.hpp"

namespace moe {

constexpr int kRlTokens = 8;                 // tokens per wave
constexpr int kRlThreads = 256;              // 4 experts per workgroup
constexpr int kRlWaves = kRlThreads / 64;
constexpr int kRlUnroll = 4;                 // rounds of 256 columns per batch of loads

struct RlArgs {
    const float* x;
    int64_t x_row_stride;
    const float* w;
    int T, D, E;
    float* logits;
};

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ double dot4(const float4& a, const float4& b, double acc) {
    acc = __dadd_rn(acc, __dmul_rn((double)a.x, (double)b.x));
    acc = __dadd_rn(acc, __dmul_rn((double)a.y, (double)b.y));
    acc = __dadd_rn(acc, __dmul_rn((double)a.z, (double)b.z));
    acc = __dadd_rn(acc, __dmul_rn((double)a.w, (double)b.w));
    return acc;
}

__global__ void __launch_bounds__(kRlThreads) router_logits_kernel(RlArgs a) {
    const int lane = threadIdx.x & 63;
    const int e = (int)blockIdx.y * kRlWaves + (threadIdx.x >> 6);
    const int t0 = (int)blockIdx.x * kRlTokens;
    if (e >= a.E) return;
    const int nt = min(kRlTokens, a.T - t0);
    double acc[kRlTokens];
#pragma unroll
    for (int i = 0; i < kRlTokens; ++i) acc[i] = 0.0;
    const float* wrow = a.w + (int64_t)e * a.D;
    const float* xrow = a.x + (int64_t)t0 * a.x_row_stride;
    // kRlUnroll rounds of 256 columns at a time: all their loads issue before
    // the first product, so a row of D columns costs D / 1024 memory round
    // trips rather than D / 256
    int d0 = 0;
    for (; d0 + 256 * kRlUnroll <= a.D; d0 += 256 * kRlUnroll) {
        float4 w4[kRlUnroll], x4[kRlUnroll][kRlTokens];
#pragma unroll
        for (int u = 0; u < kRlUnroll; ++u) {
            const int d = d0 + 256 * u + 4 * lane;
            w4[u] = *reinterpret_cast<const float4*>(wrow + d);
#pragma unroll
            for (int i = 0; i < kRlTokens; ++i)
                if (i < nt) x4[u][i] = *reinterpret_cast<const float4*>(xrow + (int64_t)i * a.x_row_stride + d);
        }
#pragma unroll
        for (int u = 0; u < kRlUnroll; ++u)
#pragma unroll
            for (int i = 0; i < kRlTokens; ++i)
                if (i < nt) acc[i] = dot4(x4[u][i], w4[u], acc[i]);
    }
    for (int d = d0 + 4 * lane; d < a.D; d += 256) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrow + d);
        float4 x4[kRlTokens];
#pragma unroll
        for (int i = 0; i < kRlTokens; ++i)
            if (i < nt) x4[i] = *reinterpret_cast<const float4*>(xrow + (int64_t)i * a.x_row_stride + d);
#pragma unroll
        for (int i = 0; i < kRlTokens; ++i)
            if (i < nt) acc[i] = dot4(x4[i], w4, acc[i]);
    }
    float mine = 0.0f;
#pragma unroll
    for (int i = 0; i < kRlTokens; ++i) {
        const double s = wave_sum_d(acc[i]);
        if (lane == i) mine = __double2float_rn(s);
    }
    if (lane < nt) a.logits[(int64_t)(t0 + lane) * a.E + e] = mine;
}

// Many tokens: an LDS-tiled product on the fp64 matrix instruction. A
// workgroup computes 16 tokens x 64 experts, a wave 16 x 16 with
// v_mfma_f64_16x16x4_f64; per 128-column step both operands are staged in LDS
// as fp32 and widened to fp64 as they are read (a product of two fp32 values
// is exact in fp64, so only the fp64 additions round). The next step's
// operands are loaded into registers while this step computes, so that the
// memory latency hides behind 128 columns of arithmetic. Rows are 132 floats
// apart: the 64 lanes of a read (16 rows x 4 columns) fall on 64 distinct
// banks.
constexpr int kTileT = 16, kTileE = 64, kTileK = 128, kTileRow = kTileK + 4;
typedef double doublex4 __attribute__((ext_vector_type(4)));
constexpr int kTileXVecs = kTileT * kTileK / 4 / 256;    // float4 of x a thread stages per step
constexpr int kTileWVecs = kTileE * kTileK / 4 / 256;    // float4 of w

struct RlTileRegs {
    float4 x[kTileXVecs];
    float4 w[kTileWVecs];
};

// Thread tid stages rows tid / 32 + 8 h of each operand tile, 4 columns at
// 4 (tid % 32): 32 threads read 512 contiguous bytes of a row. Out-of-range
// rows and columns read as zero (D % 4 == 0, so a float4 is in or out whole).
__device__ __forceinline__ void rl_tile_load(RlTileRegs& r, const RlArgs& a, int t0, int e0, int k0) {
    const int tid = threadIdx.x, c = (tid & 31) * 4, k = k0 + c;
#pragma unroll
    for (int h = 0; h < kTileXVecs; ++h) {
        const int t = t0 + (tid >> 5) + 8 * h;
        r.x[h] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < a.T && k < a.D) r.x[h] = *reinterpret_cast<const float4*>(a.x + (int64_t)t * a.x_row_stride + k);
    }
#pragma unroll
    for (int h = 0; h < kTileWVecs; ++h) {
        const int e = e0 + (tid >> 5) + 8 * h;
        r.w[h] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < a.E && k < a.D) r.w[h] = *reinterpret_cast<const float4*>(a.w + (int64_t)e * a.D + k);
    }
}

__device__ __forceinline__ void rl_tile_store(const RlTileRegs& r, float (*xs)[kTileRow], float (*ws)[kTileRow]) {
    const int tid = threadIdx.x, c = (tid & 31) * 4;
#pragma unroll
    for (int h = 0; h < kTileXVecs; ++h) *reinterpret_cast<float4*>(&xs[(tid >> 5) + 8 * h][c]) = r.x[h];
#pragma unroll
    for (int h = 0; h < kTileWVecs; ++h) *reinterpret_cast<float4*>(&ws[(tid >> 5) + 8 * h][c]) = r.w[h];
}

__global__ void __launch_bounds__(256) router_logits_tiled_kernel(RlArgs a) {
    __shared__ __align__(16) float xs[kTileT][kTileRow];
    __shared__ __align__(16) float ws[kTileE][kTileRow];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kTileT, e0 = blockIdx.y * kTileE;
    const int lane = tid & 63, n = lane & 15, q = lane >> 4;
    const int ew = 16 * (tid >> 6);                  // the wave's 16 experts: e0 + ew + [0, 16)
    doublex4 acc = {0, 0, 0, 0};
    RlTileRegs r;
    rl_tile_load(r, a, t0, e0, 0);
    rl_tile_store(r, xs, ws);
    __syncthreads();
    for (int k0 = 0; k0 < a.D; k0 += kTileK) {
        const bool more = k0 + kTileK < a.D;
        if (more) rl_tile_load(r, a, t0, e0, k0 + kTileK);
#pragma unroll 8
        for (int k = 0; k < kTileK; k += 4) {
            const double xv = xs[n][k + q], wv = ws[ew + n][k + q];
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xv, wv, acc, 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            rl_tile_store(r, xs, ws);
            __syncthreads();
        }
    }
    // lane (n, q) holds tokens q + 4 i of the tile, expert n of the wave's 16
    const int e = e0 + ew + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + q + 4 * i;
        if (e < a.E && t < a.T) a.logits[(int64_t)t * a.E + e] = __double2float_rn(acc[i]);
    }
}

static int logits_check(const float* x, int64_t x_row_stride, const float* w, int T, int D, int E,
                        const float* logits, const char* name) {
    if (T < 0 || D < 4 || D % 4 || D > (1 << 20) || E < 1 || E > MOE_MAX_EXPERTS)
        return fail(MOE_EUNSUPPORTED, "%s: T=%d D=%d E=%d (D a multiple of 4, E <= %d)", name, T, D, E,
                    MOE_MAX_EXPERTS);
    if (T == 0) return MOE_OK;
    if (!x || !w || !logits) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(x) || !aligned16(w) || !aligned16(logits))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if (x_row_stride < D || x_row_stride % 4)
        return fail(MOE_EINVAL, "%s: x row stride must be >= D and a multiple of 4", name);
    if ((int64_t)T > (int64_t)kRlTokens * 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too many tokens", name);
    return MOE_OK;
}

static void logits_launch(const float* x, int64_t x_row_stride, const float* w, int T, int D, int E,
                          float* logits, hipStream_t s) {
    RlArgs a;
    a.x = x; a.x_row_stride = x_row_stride; a.w = w; a.T = T; a.D = D; a.E = E; a.logits = logits;
    if (T > 256) {   // enough tokens to share each staged weight tile among 32 of them
        const dim3 grid((unsigned)((T + kTileT - 1) / kTileT), (unsigned)((E + kTileE - 1) / kTileE));
        hipLaunchKernelGGL(router_logits_tiled_kernel, grid, dim3(256), 0, s, a);
        return;
    }
    const dim3 grid((unsigned)((T + kRlTokens - 1) / kRlTokens), (unsigned)((E + kRlWaves - 1) / kRlWaves));
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kRlThreads), 0, s, a);
}

}  // namespace moe

extern "C" int moe_router_logits(const float* x, int64_t x_row_stride, const float* w_router, int T, int D,
                                 int E, float* logits, void* stream) {
    using namespace moe;
    const int rc = logits_check(x, x_row_stride, w_router, T, D, E, logits, "moe_router_logits");
    if (rc != MOE_OK || T == 0) return rc;
    logits_launch(x, x_row_stride, w_router, T, D, E, logits, (hipStream_t)stream);
    return check_launch("moe_router_logits");
}

extern "C" int moe_router_route(const float* x, int64_t x_row_stride, const float* w_router, int D,
                                const float* expert_bias, const uint8_t* is_padding, int T, int E, int K,
                                float route_scale, int tile_m, int local_expert_offset,
                                int local_num_experts, float* logits, int32_t* topk_ids,
                                float* topk_weights, int32_t* meta, void* stream) {
    using namespace moe;
    int rc = logits_check(x, x_row_stride, w_router, T, D, E, logits, "moe_router_route");
    if (rc != MOE_OK) return rc;
    // the routing's own checks run before either launch (T = 0 included)
    rc = moe_route_check(T, E, K, tile_m, local_expert_offset, local_num_experts, E, logits, topk_ids,
                         topk_weights, meta, "moe_router_route");
    if (rc != MOE_OK || T == 0) return rc;
    logits_launch(x, x_row_stride, w_router, T, D, E, logits, (hipStream_t)stream);
    rc = check_launch("moe_router_route (logits)");
    if (rc != MOE_OK) return rc;
    return moe_route(logits, E, expert_bias, is_padding, T, E, K, route_scale, tile_m, local_expert_offset,
                     local_num_experts, topk_ids, topk_weights, meta, stream);
}

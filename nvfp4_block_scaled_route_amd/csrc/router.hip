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
// Up to 256 tokens a workgroup computes 8 tokens x NE experts (NE = 1, 2 or 4
// as the tokens grow, rl_experts). Its 4 waves take every fourth 256-column
// round of D: per round a lane loads 4 consecutive weights of each expert and
// the same 4 columns of the 8 token rows (16-byte loads; each token column
// serves the NE experts), and a wave issues the loads of up to 4 of its rounds
// (2 at NE = 4) together, so that at D <= 4096 it waits for memory once or
// twice: decode is bound by that latency, not by the bytes. Each wave then
// folds its 8 sums of an expert across its lanes -- over lane bits 5, 4 and 3
// a lane keeps half of its token sums and adds its partner's, then bits 2, 1
// and 0 sum the one left: 10 exchanges for the 8 sums -- and wave 0 adds the 4
// waves' sums in wave order. The token rows are read by the E / NE workgroups
// of a token group from the cache; the weight ([E, D] fp32) once from memory,
// then by the other token groups from the cache.
#include "common.hpp"

namespace moe {

constexpr int kRlTokens = 8;                 // tokens per workgroup
constexpr int kRlThreads = 256;
constexpr int kRlWaves = kRlThreads / 64;    // waves splitting D

struct RlArgs {
    const float* x;
    int64_t x_row_stride;
    const float* w;
    int T, D, E;
    float* logits;
};

__device__ __forceinline__ double dot4(const float4& a, const float4& b, double acc) {
    acc = __dadd_rn(acc, __dmul_rn((double)a.x, (double)b.x));
    acc = __dadd_rn(acc, __dmul_rn((double)a.y, (double)b.y));
    acc = __dadd_rn(acc, __dmul_rn((double)a.z, (double)b.z));
    acc = __dadd_rn(acc, __dmul_rn((double)a.w, (double)b.w));
    return acc;
}

// Lane l holds, for tokens j and j + H of its 2H sums, its own and lane
// l ^ M's; it keeps token j + H where bit M is set and j elsewhere, adding
// the partner's sum of the token it keeps (fp64 addition commutes, so both
// lanes of a pair form the same sum).
template <int H>
__device__ __forceinline__ void fold(const double (&in)[2 * H], double (&out)[H], int lane, int mask) {
    const bool up = (lane & mask) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const double keep = up ? in[j + H] : in[j], give = up ? in[j] : in[j + H];
        out[j] = keep + __shfl_xor(give, mask);
    }
}

// NE experts (rows e0 .. e0 + NE - 1; past E they repeat row E - 1 and are not
// written), U of a wave's rounds per batch of loads.
template <int NE, int U>
__global__ void __launch_bounds__(kRlThreads) router_logits_kernel(RlArgs a) {
    __shared__ double part[kRlWaves][NE][kRlTokens];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e0 = (int)blockIdx.y * NE;
    const int t0 = (int)blockIdx.x * kRlTokens;
    const int nt = min(kRlTokens, a.T - t0);
    double acc[NE][kRlTokens];
#pragma unroll
    for (int j = 0; j < NE; ++j)
#pragma unroll
        for (int i = 0; i < kRlTokens; ++i) acc[j][i] = 0.0;
    const float* wrow[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) wrow[j] = a.w + (int64_t)min(e0 + j, a.E - 1) * a.D;
    const float* xrow = a.x + (int64_t)t0 * a.x_row_stride;
    const int nr = (a.D + 255) / 256;           // rounds; the last may be partial (D % 4 == 0)
    // The loads carry no lane-dependent branch (those made the compiler wait
    // for one round's loads before issuing the next): a lane past D in the
    // last round reads an in-bounds column and its products are dropped by a
    // select, and the rows of tokens past T repeat the last token's row (their
    // sums are never written).
    int64_t xo[kRlTokens];
#pragma unroll
    for (int i = 0; i < kRlTokens; ++i) xo[i] = (int64_t)min(i, nt - 1) * a.x_row_stride;
    for (int r0 = wave; r0 < nr; r0 += kRlWaves * U) {
        float4 w4[U][NE], x4[U][kRlTokens];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + kRlWaves * u >= nr) break;          // uniform
            const int d = min(256 * (r0 + kRlWaves * u) + 4 * lane, a.D - 4);
#pragma unroll
            for (int j = 0; j < NE; ++j) w4[u][j] = *reinterpret_cast<const float4*>(wrow[j] + d);
#pragma unroll
            for (int i = 0; i < kRlTokens; ++i) x4[u][i] = *reinterpret_cast<const float4*>(xrow + xo[i] + d);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + kRlWaves * u >= nr) break;
            const bool in = 256 * (r0 + kRlWaves * u) + 4 * lane < a.D;
#pragma unroll
            for (int j = 0; j < NE; ++j)
#pragma unroll
                for (int i = 0; i < kRlTokens; ++i) {
                    const double v = dot4(x4[u][i], w4[u][j], acc[j][i]);
                    acc[j][i] = in ? v : acc[j][i];
                }
        }
    }
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        double s4[4], s2[2], s1[1];
        fold<4>(acc[j], s4, lane, 32);
        fold<2>(s4, s2, lane, 16);
        fold<1>(s2, s1, lane, 8);
        double v = s1[0];                       // token lane >> 3, summed over lane bits 3-5
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 1);
        if ((lane & 7) == 0) part[wave][j][lane >> 3] = v;
    }
    __syncthreads();
    const int i = lane & 7, j = lane >> 3;      // wave 0: lane 8 j + i sums token i of expert e0 + j
    if (wave == 0 && j < NE && i < nt && e0 + j < a.E) {
        double sum = part[0][j][i];
#pragma unroll
        for (int w = 1; w < kRlWaves; ++w) sum += part[w][j][i];
        a.logits[(int64_t)(t0 + i) * a.E + e0 + j] = __double2float_rn(sum);
    }
}

// Experts a workgroup takes: more tokens share each expert's weight row among
// fewer token groups, and fewer workgroups then re-read the token rows.
static int rl_experts(int T) { return T <= 16 ? 1 : T <= 64 ? 2 : 4; }

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
    const int ne = rl_experts(T);
    const dim3 grid((unsigned)((T + kRlTokens - 1) / kRlTokens), (unsigned)((E + ne - 1) / ne));
    if (ne == 1) hipLaunchKernelGGL((router_logits_kernel<1, 4>), grid, dim3(kRlThreads), 0, s, a);
    else if (ne == 2) hipLaunchKernelGGL((router_logits_kernel<2, 4>), grid, dim3(kRlThreads), 0, s, a);
    else hipLaunchKernelGGL((router_logits_kernel<4, 2>), grid, dim3(kRlThreads), 0, s, a);
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

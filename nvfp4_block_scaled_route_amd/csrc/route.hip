// moe_route: MuseSpark1x top-k routing and the permutation metadata.
//   the runner page, "validate_deployment" (sigmoid + expert bias + sum
//   renormalize, no groups, route scale 1); the model page, "MuseSpark1xMoE"
//   (division eps 1e-15) and "_prepared_nvfp4_forward" (padding tokens -> -1);
//   the flashinfer_ops page, "FlashInferOps.slot" / "gemm2_rows" (metadata).
//
// Phase 1, top-k: one 64-wide wave per token; lane l holds experts l, l+64, ...
// Each of the K rounds takes the wave-wide best (key desc, index asc) among the
// experts not taken yet. Lane k keeps the k-th choice; the renormalizing sum runs
// over k in order.
// Phase 2, permutation: one workgroup. Routes are processed in chunks of 512 in
// expanded order; within a wave, routes of the same expert are matched with
// ballots over the expert index bits, giving each route its rank among earlier
// routes of its expert (a stable counting sort, no atomics, deterministic).
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 512;                 // 8 waves
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;  // 16

struct RouteArgs {
    const float* logits;
    int64_t logits_row_stride;
    const float* bias;
    const uint8_t* is_padding;
    int T, E, K;
    float route_scale;
    int tile_m, local_offset, local_num;
    int32_t* ids;
    float* weights;
    int32_t* meta;
    moe_meta_layout L;
};

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__device__ void topk_token(const RouteArgs& a, int t, int lane) {
    int32_t* ids = a.ids + (int64_t)t * a.K;
    float* wts = a.weights + (int64_t)t * a.K;
    if (a.is_padding && a.is_padding[t]) {
        if (lane < a.K) { ids[lane] = -1; wts[lane] = 0.0f; }
        return;
    }
    const float* row = a.logits + (int64_t)t * a.logits_row_stride;
    float key[kMaxPerLane], sc[kMaxPerLane];
    uint32_t alive = 0;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        key[j] = -__builtin_inff();
        sc[j] = 0.0f;
        if (e < a.E) {
            sc[j] = sigmoid32(row[e]);
            key[j] = a.bias ? __fadd_rn(sc[j], a.bias[e]) : sc[j];
            alive |= 1u << j;
        }
    }
    float total = 0.0f, my_s = 0.0f;
    int my_id = -1;
    for (int k = 0; k < a.K; ++k) {
        float bk = -__builtin_inff(), bs = 0.0f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            const int e = lane + 64 * j;
            if (((alive >> j) & 1u) && better(key[j], e, bk, bi)) { bk = key[j]; bi = e; bs = sc[j]; }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ok = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            const float os = __shfl_xor(bs, off);
            if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; bs = os; }
        }
        // bi, bs are now the same on every lane
        if ((bi & 63) == lane) alive &= ~(1u << (bi >> 6));
        if (lane == k) { my_id = bi; my_s = bs; }
        total = __fadd_rn(total, bs);
    }
    if (lane < a.K) {
        const float denom = __fadd_rn(total, 1e-15f);
        ids[lane] = my_id;
        wts[lane] = __fmul_rn(__fdiv_rn(my_s, denom), a.route_scale);
    }
}

__device__ void permute_block(const RouteArgs& a) {
    extern __shared__ int32_t lds[];
    const int El = a.local_num;
    int32_t* cnt = lds;                           // [kRouteWaves][El]
    int32_t* running = cnt + kRouteWaves * El;    // [El]
    int32_t* offs = running + El;                 // [El + 1]
    int32_t* scan = offs + El + 1;                // [kRouteWaves]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int R = a.T * a.K;
    int32_t* exp2perm = a.meta + a.L.exp2perm;
    int32_t* perm2tok = a.meta + a.L.perm2tok;
    int32_t* tile_expert = a.meta + a.L.tile_expert;
    const int m = a.tile_m;
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    for (int e = tid; e < El; e += kRouteThreads) running[e] = 0;
    for (int base = 0; base < R; base += kRouteThreads) {
        for (int i = tid; i < kRouteWaves * El; i += kRouteThreads) cnt[i] = 0;
        __syncthreads();
        const int r = base + tid;
        int e = -1;
        if (r < R) {
            const int id = a.ids[r];
            const int loc = id - a.local_offset;
            if (id >= 0 && loc >= 0 && loc < El) e = loc;
        }
        const bool valid = e >= 0;
        uint64_t match = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 10; ++bit) {
            const bool mine = (e >> bit) & 1;
            const uint64_t b = __ballot(mine);
            match &= mine ? b : ~b;
        }
        const int rank_in_wave = __popcll(match & lt_mask);
        if (valid && rank_in_wave == 0) cnt[w * El + e] = __popcll(match);
        __syncthreads();
        for (int x = tid; x < El; x += kRouteThreads) {
            int acc = running[x];
#pragma unroll
            for (int ww = 0; ww < kRouteWaves; ++ww) {
                const int c = cnt[ww * El + x];
                cnt[ww * El + x] = acc;
                acc += c;
            }
            running[x] = acc;
        }
        __syncthreads();
        if (r < R) exp2perm[r] = valid ? cnt[w * El + e] + rank_in_wave : -1;  // rank for now
        __syncthreads();
    }
    // Padded offsets: exclusive scan of ceil(count / m) * m over the local experts.
    int my_total = 0;
    {
        // each thread owns a contiguous run of experts
        const int per = (El + kRouteThreads - 1) / kRouteThreads;
        const int e0 = tid * per, e1 = min(El, e0 + per);
        for (int x = e0; x < e1; ++x) my_total += (running[x] + m - 1) / m * m;
        int incl = my_total;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        if (lane == 63) scan[w] = incl;
        __syncthreads();
        int wave_base = 0;
        for (int ww = 0; ww < w; ++ww) wave_base += scan[ww];
        int acc = wave_base + incl - my_total;
        for (int x = e0; x < e1; ++x) {
            offs[x] = acc;
            acc += (running[x] + m - 1) / m * m;
        }
        if (tid == kRouteThreads - 1) offs[El] = wave_base + incl;
    }
    __syncthreads();
    const int total_rows = offs[El];
    const int num_tiles = total_rows / m;
    for (int x = tid; x <= El; x += kRouteThreads) a.meta[a.L.expert_offsets + x] = offs[x];
    for (int x = tid; x < El; x += kRouteThreads) a.meta[a.L.expert_counts + x] = running[x];
    if (tid == 0) {
        a.meta[a.L.num_tiles] = num_tiles;
        a.meta[a.L.total_rows] = total_rows;
    }
    // tile -> expert, and -1 on every padding row (rows of a tile past its expert's
    // routes, and every row past the last tile).
    for (int tile = tid; tile < a.L.tiles_max; tile += kRouteThreads) {
        int ex = -1;
        if (tile < num_tiles) {
            const int row = tile * m;
            int lo = 0, hi = El - 1;                 // last expert with offs <= row
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (offs[mid] <= row) lo = mid; else hi = mid - 1;
            }
            ex = lo;
            // an expert with zero rows shares its offset with the next one
            while (ex + 1 < El && offs[ex + 1] <= row) ++ex;
        }
        tile_expert[tile] = ex;
        const int first_pad = ex >= 0 ? offs[ex] + running[ex] : 0;
        for (int i = 0; i < m; ++i) {
            const int row = tile * m + i;
            if (ex < 0 || row >= first_pad) perm2tok[row] = -1;
        }
    }
    // Scatter: the thread that wrote route r's rank above is this one (r % 512).
    for (int r = tid; r < R; r += kRouteThreads) {
        const int rank = exp2perm[r];
        if (rank < 0) continue;
        const int e = a.ids[r] - a.local_offset;
        const int pos = offs[e] + rank;
        exp2perm[r] = pos;
        perm2tok[pos] = r / a.K;
    }
}

__global__ void __launch_bounds__(kRouteThreads) route_kernel(RouteArgs a, int do_topk,
                                                              int do_permute) {
    if (do_topk) {
        const int lane = threadIdx.x & 63;
        const int wave = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
        const int nwaves = gridDim.x * kRouteWaves;
        for (int t = wave; t < a.T; t += nwaves) topk_token(a, t, lane);
    }
    if (do_permute) {
        __syncthreads();   // the top-k ids written above are read back below
        permute_block(a);
    }
}

}  // namespace moe

extern "C" int moe_route(const float* logits, int64_t logits_row_stride, const float* expert_bias,
                         const uint8_t* is_padding, int T, int E, int K, float route_scale,
                         int tile_m, int local_expert_offset, int local_num_experts,
                         int32_t* topk_ids, float* topk_weights, int32_t* meta, void* stream) {
    using namespace moe;
    if (T < 0) return fail(MOE_EINVAL, "moe_route: T=%d", T);
    if (E < 1 || E > MOE_MAX_EXPERTS)
        return fail(MOE_EUNSUPPORTED, "moe_route: E=%d outside [1, %d]", E, MOE_MAX_EXPERTS);
    if (K < 1 || K > E || K > MOE_MAX_TOPK)
        return fail(MOE_EUNSUPPORTED, "moe_route: K=%d outside [1, min(E, %d)]", K, MOE_MAX_TOPK);
    if (local_num_experts < 1 || local_num_experts > MOE_MAX_EXPERTS || local_expert_offset < 0)
        return fail(MOE_EINVAL, "moe_route: local experts [%d, +%d) invalid", local_expert_offset,
                    local_num_experts);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "moe_route: tile_m=%d must be a multiple of 16 in [16, 256]",
                    tile_m);
    if (logits_row_stride < E) return fail(MOE_EINVAL, "moe_route: logits row stride < E");
    if (!meta) return fail(MOE_EINVAL, "moe_route: meta is NULL");
    if (T > 0 && (!logits || !topk_ids || !topk_weights))
        return fail(MOE_EINVAL, "moe_route: NULL pointer");
    if (!aligned16(meta) || (T > 0 && (!aligned16(logits) || !aligned16(topk_ids) ||
                                        !aligned16(topk_weights))))
        return fail(MOE_EINVAL, "moe_route: pointers must be 16-byte aligned");
    if ((int64_t)T * K > 0x3FFFFFFF) return fail(MOE_EUNSUPPORTED, "moe_route: too many routes");
    RouteArgs a;
    a.logits = logits; a.logits_row_stride = logits_row_stride; a.bias = expert_bias;
    a.is_padding = is_padding; a.T = T; a.E = E; a.K = K; a.route_scale = route_scale;
    a.tile_m = tile_m; a.local_offset = local_expert_offset; a.local_num = local_num_experts;
    a.ids = topk_ids; a.weights = topk_weights; a.meta = meta;
    a.L = meta_layout(T, K, local_num_experts, tile_m);
    const size_t lds = sizeof(int32_t) * ((size_t)(kRouteWaves + 2) * local_num_experts + 1 + kRouteWaves);
    hipStream_t s = (hipStream_t)stream;
    if (T <= kRouteWaves) {
        hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, s, a, 1, 1);
    } else {
        const int grid = (int)((T + kRouteWaves - 1) / kRouteWaves < 8192 ? (T + kRouteWaves - 1) / kRouteWaves : 8192);
        hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(kRouteThreads), 0, s, a, 1, 0);
        int rc = check_launch("moe_route (top-k)");
        if (rc) return rc;
        hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, s, a, 0, 1);
    }
    return check_launch("moe_route");
}

// moe_route / moe_route_quant: MuseSpark1x top-k routing and the permutation
// metadata (and, fused into the same launch, the NVFP4 input quantizer).
//   the runner page, "validate_deployment" (sigmoid + expert bias + sum
//   renormalize, no groups, route scale 1); the model page, "MuseSpark1xMoE"
//   (division eps 1e-15) and "_prepared_nvfp4_forward" (padding tokens -> -1);
//   the flashinfer_ops page, "FlashInferOps.slot" / "gemm2_rows" (metadata).
//
// Top-k, one 64-wide wave per token. Selection keys are totally ordered by
// (key descending, expert index ascending), so every expert's place in the
// ranking is unique: for E <= 64 each lane counts, against the wave's keys in
// LDS (one 64-bit comparison per key), the experts that beat its own, and the
// experts with rank < K land in slot `rank` -- the K choices in key order with
// no serial rounds. Larger E takes K rounds of a wave-wide maximum of the
// 64-bit composite keys by DPP (registers only). The renormalizing sum then
// runs over the K choices in order.
// Permutation: routes per expert are counted, the padded offsets scanned, and
// a second pass gives every route its rank among the earlier routes of its
// expert (ballot matching over the expert index bits within a wave: a stable
// counting sort, no ordering atomics, deterministic) and scatters it at once.
// Up to 128 routes one wave counts and ranks them, chunk by chunk, while the
// workgroup's other waves write the per-row and per-tile fields; beyond, the
// whole workgroup does it (LDS atomics for the counts, a scan across its waves
// for the ranks; measured, moe_route_quant: decode_b64_zipf's 512 routes 13.8
// -> 9.4 µs, expert_tp8_b32's 256 15.5 -> 14.3, while decode_b8's 64 take
// 6.2 µs by one wave and 6.8 by the workgroup). Past 512 routes of more than
// 8 tokens the grid does it (below).
// Small batches run top-k and the permutation in one workgroup, the top-k ids
// staying in LDS; larger ones take a top-k grid, then the permutation.
// moe_route_quant appends the quantizer's workgroups to the first launch: they
// need nothing from the routing and run beside it.
#include "common.hpp"

namespace moe {

constexpr int kRouteThreads = 512;                 // 8 waves
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;  // 16
constexpr int kRankMaxExperts = 64;                // rank-count top-k up to here; the wave maximum beyond
// One workgroup routes up to a token a wave; more tokens take the top-k grid
// (a token a wave) and then the permutation, since a wave's K rounds for
// several tokens run one after another (expert_tp8_b32, 32 tokens: 14.3 µs in
// one workgroup, 8.9 µs in the two launches).
constexpr int kFusedMaxTokens = kRouteWaves;

enum RouteMode { kTopkOnly = 0, kPermuteOnly = 1, kFused = 2 };

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
    // fused quantizer (x == nullptr: none)
    const uint16_t* x;
    int64_t x_row_stride;
    const float* gscale;
    int H;
    uint8_t* codes;
    uint8_t* sf;
    int route_blocks;      // workgroups [0, route_blocks) route, the rest quantize
};

// fp32 -> uint32 with the same order (finite inputs; -0 is first made +0 so
// that it ties with +0 as the fp32 comparison does)
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(__fadd_rn(f, 0.0f));
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ int epad(int E) { return (E + 3) & ~3; }

// LDS of the top-k: per wave Epad 64-bit composite keys, then per wave K
// (expert, score) slots.
__device__ __forceinline__ uint64_t* topk_keys(int32_t* base) { return reinterpret_cast<uint64_t*>(base); }
__device__ __forceinline__ uint2* topk_slots(int32_t* base, int E) {
    return reinterpret_cast<uint2*>(base + 2 * kRouteWaves * epad(E));
}

// Writes token t's ids and weights (and its ids into s_ids when given).
__device__ __forceinline__ void emit(const RouteArgs& a, int t, int lane, int id, float wt,
                                     int32_t* s_ids) {
    a.ids[(int64_t)t * a.K + lane] = id;
    a.weights[(int64_t)t * a.K + lane] = wt;
    if (s_ids) s_ids[t * a.K + lane] = id;
}

// Rank-count top-k of token t by wave w (E <= kRankMaxExperts: one key a lane). Called by every
// thread of the workgroup (it holds two barriers); `active` is false for waves
// without a token this round. An expert's composite key is its ordered key in
// the high word and the complement of its index in the low word, so that one
// 64-bit comparison decides (key desc, index asc); its rank is the number of
// larger composites.
__device__ void topk_rank(const RouteArgs& a, int t, bool active, int lane, int w,
                          int32_t* lds_topk, int32_t* s_ids) {
    const int Ep = epad(a.E);
    uint64_t* key = topk_keys(lds_topk) + w * Ep;
    uint2* slot = topk_slots(lds_topk, a.E) + w * a.K;
    const bool live = active && !(a.is_padding && a.is_padding[t]);
    constexpr int kPer = kRankMaxExperts / 64;
    float sc[kPer];
    uint64_t kk[kPer];
    if (live) {
        const float* row = a.logits + (int64_t)t * a.logits_row_stride;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = lane + 64 * j;
            sc[j] = 0.0f;
            kk[j] = 0u;
            if (e < a.E) {
                sc[j] = sigmoid32(row[e]);
                const uint32_t ok = order_key(a.bias ? __fadd_rn(sc[j], a.bias[e]) : sc[j]);
                kk[j] = ((uint64_t)ok << 32) | (uint32_t)~(uint32_t)e;
                key[e] = kk[j];
            }
        }
        if (lane < Ep - a.E) key[a.E + lane] = 0u;   // padding keys: below every real key
    }
    __syncthreads();
    if (live) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = lane + 64 * j;
            if (e < a.E) {
                const uint64_t me = kk[j];
                int rank = 0;
#pragma unroll 4
                for (int i = 0; i < Ep; i += 2) {
                    const ulonglong2 q = *reinterpret_cast<const ulonglong2*>(key + i);
                    rank += (int)(q.x > me) + (int)(q.y > me);
                }
                if (rank < a.K) slot[rank] = make_uint2((uint32_t)e, __float_as_uint(sc[j]));
            }
        }
    }
    __syncthreads();
    if (active) {
        int id = -1;
        float wt = 0.0f;
        if (live) {
            const uint2 mine = slot[lane < a.K ? lane : 0];
            // the renormalizing sum over k in order, from the K lanes' scores
            float total = 0.0f;
            for (int k = 0; k < a.K; ++k)
                total = __fadd_rn(total, __int_as_float(__builtin_amdgcn_readlane((int)mine.y, k)));
            id = (int)mine.x;
            wt = __fmul_rn(__fdiv_rn(__uint_as_float(mine.y), __fadd_rn(total, 1e-15f)), a.route_scale);
        }
        if (lane < a.K) emit(a, t, lane, id, wt, s_ids);
    }
}

__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }

// v[idx] for a wave-uniform idx < N, by a tree of selects on idx's bits (an
// index loop would be lowered to a stack array and a load).
template <int N>
__device__ __forceinline__ float pick(const float* v, int idx) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        const float lo = pick<N / 2>(v, idx), hi = pick<N - N / 2>(v + N / 2, idx - N / 2);
        return idx >= N / 2 ? hi : lo;
    }
}

// The largest u32 over the wave, uniform: the maximum over each row of 16
// lanes by DPP, then over the four rows' lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowMirror, 0xF, 0xF, true));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// The largest 64-bit value over the wave, uniform: the largest high word, then
// the largest low word among the lanes that hold it (two 32-bit maxima, each
// step one DPP instruction, instead of a 64-bit comparison per step).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// Top-k of token t by one wave, any E up to 64 kPer: K rounds of a wave-wide
// maximum of the composite keys (the ordered key in the high word, the
// complement of the expert index in the low word: one 64-bit comparison
// decides key descending, index ascending), taking the winner out of its lane
// after each round. The K choices come out by key descending and the
// renormalizing sum runs over them in that order, as in the rank-count form.
// Registers and DPP only: no LDS, no barrier.
// Expert e's selection key and score from its logit: the ordered key in the
// high word, the complement of the index in the low word (one 64-bit
// comparison decides key descending, index ascending).
__device__ __forceinline__ void topk_key(const RouteArgs& a, int e, float logit, uint64_t& kk, float& sc) {
    sc = sigmoid32(logit);
    const uint32_t ok = order_key(a.bias ? __fadd_rn(sc, a.bias[e]) : sc);
    kk = ((uint64_t)ok << 32) | (uint32_t)~(uint32_t)e;
}

// The K rounds of token t over the keys the wave holds (kk[j], sc[j]: expert
// lane + 64 j; 0 below every real composite, whose high word is non-zero).
template <int kPer>
__device__ __forceinline__ void topk_rounds(const RouteArgs& a, int t, int lane, int32_t* s_ids,
                                            uint64_t (&kk)[kPer], const float (&sc)[kPer]) {
    float total = 0.0f, my_s = 0.0f;
    int my_id = -1;
    for (int k = 0; k < a.K; ++k) {
        uint64_t best = kk[0];
#pragma unroll
        for (int j = 1; j < kPer; ++j) best = max_u64(best, kk[j]);
        best = wave_max_u64(best);
        const int e = (int)~(uint32_t)best;       // uniform
        const int owner = e & 63, slot = e >> 6;
        const float s_own = pick<kPer>(sc, slot);
        const float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_own), owner));
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j == slot && lane == owner) kk[j] = 0u;
        if (lane == k) { my_id = e; my_s = bs; }
        total = __fadd_rn(total, bs);
    }
    if (lane < a.K)
        emit(a, t, lane, my_id,
             __fmul_rn(__fdiv_rn(my_s, __fadd_rn(total, 1e-15f)), a.route_scale), s_ids);
}

// One token, its logits loaded here (the form for many experts a lane).
template <int kPer>
__device__ void topk_max(const RouteArgs& a, int t, int lane, int32_t* s_ids) {
    if (a.is_padding && a.is_padding[t]) {
        if (lane < a.K) emit(a, t, lane, -1, 0.0f, s_ids);
        return;
    }
    const float* row = a.logits + (int64_t)t * a.logits_row_stride;
    uint64_t kk[kPer];
    float sc[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = lane + 64 * j;
        kk[j] = 0u;
        sc[j] = 0.0f;
        if (e < a.E) topk_key(a, e, row[e], kk[j], sc[j]);
    }
    topk_rounds<kPer>(a, t, lane, s_ids, kk, sc);
}

// The K-round form for a wave's tokens first + w, + step, ... (up to 4
// experts a lane): the logits of up to kPre of them load together before
// their rounds, so that a wave with several tokens waits for one memory
// latency instead of one per token.
template <int kPer>
__device__ __forceinline__ void topk_max_tokens(const RouteArgs& a, int first, int step, int lane, int w,
                                                int32_t* s_ids) {
    constexpr int kPre = kPer <= 2 ? 4 : 2;
    for (int base = first; base < a.T; base += kPre * step) {
        float lg[kPre][kPer];
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int t = base + q * step + w;
            const float* row = a.logits + (int64_t)t * a.logits_row_stride;
#pragma unroll
            for (int j = 0; j < kPer; ++j) lg[q][j] = t < a.T && lane + 64 * j < a.E ? row[lane + 64 * j] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int t = base + q * step + w;
            if (t >= a.T) continue;                // uniform over the wave
            if (a.is_padding && a.is_padding[t]) {
                if (lane < a.K) emit(a, t, lane, -1, 0.0f, s_ids);
                continue;
            }
            uint64_t kk[kPer];
            float sc[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int e = lane + 64 * j;
                kk[j] = 0u;
                sc[j] = 0.0f;
                if (e < a.E) topk_key(a, e, lg[q][j], kk[j], sc[j]);
            }
            topk_rounds<kPer>(a, t, lane, s_ids, kk, sc);
        }
    }
}

// Top-k of tokens [first, T) with stride `step`, one token per wave: the
// rank count up to 64 experts (every thread of the workgroup takes part in
// every round: it holds barriers), the K-round wave maximum beyond (measured,
// moe_route_quant back to back: decode_b8 (E = 64) 6.4 µs by rank count, 6.7
// by rounds; E = 128: expert_tp8_b32 (32 tokens, one workgroup) 26.2 µs by
// rank count, 17.5 by rounds, 15.5 with the logits loaded ahead and the
// 64-bit maximum as two 32-bit ones; decode_b64_zipf 17.5 -> 15.3 -> 14.5;
// prefill_t4096 32.6 -> 29.2 -> 26.2, with the scan's batched loads).
__device__ __forceinline__ void topk_tokens(const RouteArgs& a, int first, int step, int32_t* lds_topk,
                            int32_t* s_ids) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (a.E <= kRankMaxExperts) {
        for (int base = first; base < a.T; base += step) {
            const int t = base + w;
            topk_rank(a, t, t < a.T, lane, w, lds_topk, s_ids);
        }
    } else if (a.E <= 128) {
        topk_max_tokens<2>(a, first, step, lane, w, s_ids);
    } else if (a.E <= 256) {
        topk_max_tokens<4>(a, first, step, lane, w, s_ids);
    } else {
        for (int base = first; base < a.T; base += step) {
            const int t = base + w;
            if (t < a.T) topk_max<kMaxPerLane>(a, t, lane, s_ids);   // uniform over the wave
        }
    }
}

__device__ __forceinline__ int local_expert(const RouteArgs& a, int id) {
    const int loc = id - a.local_offset;
    return (id >= 0 && loc >= 0 && loc < a.local_num) ? loc : -1;
}

// Lanes of the wave whose route goes to the same local expert (e < 0: none).
__device__ __forceinline__ uint64_t same_expert_lanes(int e) {
    uint64_t match = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const bool mine = (e >> bit) & 1;
        const uint64_t b = __ballot(mine);
        match &= mine ? b : ~b;
    }
    return match;
}


// The expert step's sync words start at zero: its status, the two counters
// of every 16-row tile (moe_experts_fwd's one-launch form), the tiled form's
// work queues and the per-token counters of the finalize in the launch.
__device__ __forceinline__ void clear_sync(const RouteArgs& a, int i, int step) {
    int32_t* sync = a.meta + a.L.sub_sync;
    for (int64_t x = i; x < 2 * a.L.subs_max; x += step) sync[(x >> 1) * kSubSyncStride + (x & 1)] = 0;
    int32_t* tok = a.meta + a.L.tok_sync;
    for (int64_t x = i; x < 3 * a.T; x += step) tok[(x / 3) * kTokSyncStride + x % 3] = 0;
    if (i == 0) a.meta[a.L.sync_status] = 0;
    if (i < kQueueWords) a.meta[a.L.queue + i] = 0;
}

// The permutation metadata for up to 128 routes, by one workgroup. Wave 0
// counts the routes per expert (chunks of 64 routes, one per lane; experts in
// runs of ceil(El / 64) per lane) and scans the padded offsets. Then, while wave
// 0 ranks the routes and scatters them, the other waves write the per-row and
// per-tile fields -- tile -> expert, -1 on padding rows and past the last tile,
// the cleared sync words -- as coalesced strided stores, each row's expert read
// from an LDS copy of the tile map.
constexpr int kWaveMaxRoutes = 128;

__device__ __forceinline__ void permute_small(const RouteArgs& a, const int32_t* ids, int32_t* lds) {
    const int El = a.local_num;
    int32_t* count = lds;                          // [El]
    int32_t* offs = count + El;                    // [El + 1]
    int32_t* running = offs + El + 1;              // [El]
    int32_t* tile_e = running + El;                // [tiles_max]: tile -> expert, -1 past the last tile
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int R = a.T * a.K;
    const int m = a.tile_m;
    const int tiles_max = (int)a.L.tiles_max, rows_max = (int)a.L.rows_max;
    int32_t* exp2perm = a.meta + a.L.exp2perm;
    int32_t* perm2tok = a.meta + a.L.perm2tok;
    int32_t* tile_expert = a.meta + a.L.tile_expert;
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    // wave 0's local experts of routes 64 c + lane, loaded once for both passes
    // (in flight together: from global memory each chunk's load would
    // otherwise wait a memory latency, twice)
    constexpr int kChunks = kWaveMaxRoutes / 64;
    int re[kChunks];
    if (w == 0) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int r = 64 * c + lane;
            re[c] = r < R ? local_expert(a, ids[r]) : -1;
        }
        for (int x = lane; x < El; x += 64) count[x] = 0;
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (64 * c >= R) break;
            const int e = re[c];
            const uint64_t match = same_expert_lanes(e);
            if (e >= 0 && (match & lt_mask) == 0) count[e] += __popcll(match);   // one lane per expert
            wave_lds_sync();
        }
        // padded offsets
        const int per = (El + 63) >> 6;
        const int x0 = lane * per, x1 = min(El, x0 + per);
        int mine = 0;
        for (int x = x0; x < x1; ++x) mine += (count[x] + m - 1) / m * m;
        const int incl = wave_inclusive_scan(mine);
        const int total_rows = __builtin_amdgcn_readlane(incl, 63);
        int acc = incl - mine;
        for (int x = x0; x < x1; ++x) {
            offs[x] = acc;
            running[x] = acc;
            acc += (count[x] + m - 1) / m * m;
        }
        if (lane == 0) offs[El] = total_rows;
        wave_lds_sync();
        for (int x = lane; x <= El; x += 64) a.meta[a.L.expert_offsets + x] = offs[x];
        for (int x = lane; x < El; x += 64) a.meta[a.L.expert_counts + x] = count[x];
        if (lane == 0) {
            a.meta[a.L.num_tiles] = total_rows / m;
            a.meta[a.L.total_rows] = total_rows;
        }
    }
    __syncthreads();
    const int total_rows = offs[El];
    const int num_tiles = total_rows / m;
    for (int x = tid; x < El; x += kRouteThreads)
        for (int tile = offs[x] / m; tile < offs[x + 1] / m; ++tile) tile_e[tile] = x;
    for (int tile = num_tiles + tid; tile < tiles_max; tile += kRouteThreads) tile_e[tile] = -1;
    __syncthreads();
    if (w == 0) {
        // stable ranks, chunk by chunk, scattered at once
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (64 * c >= R) break;
            const int r = 64 * c + lane;
            const int e = re[c];
            const uint64_t match = same_expert_lanes(e);
            const int pos = e >= 0 ? running[e] + __popcll(match & lt_mask) : -1;
            wave_lds_sync();
            if (e >= 0 && (match & lt_mask) == 0) running[e] += __popcll(match);
            wave_lds_sync();
            if (r < R) {
                exp2perm[r] = pos;
                if (pos >= 0) perm2tok[pos] = r / a.K;
            }
        }
    } else {
        const int i = tid - 64, step = kRouteThreads - 64;
        for (int tile = i; tile < tiles_max; tile += step) tile_expert[tile] = tile_e[tile];
        for (int row = i; row < rows_max; row += step) {
            const int e = tile_e[row / m];
            if (e < 0 || row - offs[e] >= count[e]) perm2tok[row] = -1;   // padding: no route lands here
        }
        clear_sync(a, i, step);
    }
}

// The permutation metadata from the top-k ids (global or LDS). One workgroup.
__device__ __forceinline__ void permute_block(const RouteArgs& a, const int32_t* ids, int32_t* lds) {
    const int El = a.local_num;
    int32_t* cnt = lds;                           // [kRouteWaves][El]
    int32_t* count = cnt + kRouteWaves * El;      // [El]  routes per expert
    int32_t* running = count + El;                // [El]  next free row of each expert
    int32_t* offs = running + El;                 // [El + 1]
    int32_t* scan = offs + El + 1;                // [kRouteWaves]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int R = a.T * a.K;
    const int m = a.tile_m;
    int32_t* exp2perm = a.meta + a.L.exp2perm;
    int32_t* perm2tok = a.meta + a.L.perm2tok;
    int32_t* tile_expert = a.meta + a.L.tile_expert;

    // pass 1: routes per local expert
    for (int e = tid; e < El; e += kRouteThreads) count[e] = 0;
    __syncthreads();
    for (int r = tid; r < R; r += kRouteThreads) {
        const int e = local_expert(a, ids[r]);
        if (e >= 0) atomicAdd(&count[e], 1);
    }
    __syncthreads();
    // padded offsets: exclusive scan of ceil(count / m) * m; each thread owns a
    // contiguous run of experts
    {
        const int per = (El + kRouteThreads - 1) / kRouteThreads;
        const int e0 = tid * per, e1 = min(El, e0 + per);
        int my_total = 0;
        for (int x = e0; x < e1; ++x) my_total += (count[x] + m - 1) / m * m;
        const int incl = wave_inclusive_scan(my_total);
        if (lane == 63) scan[w] = incl;
        __syncthreads();
        int wave_base = 0;
        for (int ww = 0; ww < w; ++ww) wave_base += scan[ww];
        int acc = wave_base + incl - my_total;
        for (int x = e0; x < e1; ++x) {
            offs[x] = acc;
            running[x] = acc;
            acc += (count[x] + m - 1) / m * m;
        }
        if (tid == kRouteThreads - 1) offs[El] = wave_base + incl;
    }
    __syncthreads();
    const int total_rows = offs[El];
    const int num_tiles = total_rows / m;
    for (int x = tid; x <= El; x += kRouteThreads) a.meta[a.L.expert_offsets + x] = offs[x];
    for (int x = tid; x < El; x += kRouteThreads) a.meta[a.L.expert_counts + x] = count[x];
    if (tid == 0) {
        a.meta[a.L.num_tiles] = num_tiles;
        a.meta[a.L.total_rows] = total_rows;
    }
    // tile -> expert and -1 on the padding rows of each expert's range (the
    // expert's own thread), then -1 past the last tile
    for (int x = tid; x < El; x += kRouteThreads) {
        for (int tile = offs[x] / m; tile < offs[x + 1] / m; ++tile) tile_expert[tile] = x;
        for (int row = offs[x] + count[x]; row < offs[x + 1]; ++row) perm2tok[row] = -1;
    }
    for (int tile = num_tiles + tid; tile < a.L.tiles_max; tile += kRouteThreads) tile_expert[tile] = -1;
    for (int row = total_rows + tid; row < a.L.rows_max; row += kRouteThreads) perm2tok[row] = -1;
    clear_sync(a, tid, kRouteThreads);
    // pass 2: stable rank within the expert, in chunks of one route per thread
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int base = 0; base < R; base += kRouteThreads) {
        for (int i = tid; i < kRouteWaves * El; i += kRouteThreads) cnt[i] = 0;
        __syncthreads();
        const int r = base + tid;
        const int e = r < R ? local_expert(a, ids[r]) : -1;
        const bool valid = e >= 0;
        const uint64_t match = same_expert_lanes(e);
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
        if (r < R) {
            if (valid) {
                const int pos = cnt[w * El + e] + rank_in_wave;
                exp2perm[r] = pos;
                perm2tok[pos] = r / a.K;
            } else {
                exp2perm[r] = -1;
            }
        }
        __syncthreads();   // cnt is cleared for the next chunk
    }
}

__global__ void __launch_bounds__(kRouteThreads) route_kernel(RouteArgs a, int mode) {
    extern __shared__ int32_t lds[];
    if ((int)blockIdx.x >= a.route_blocks) {       // the fused quantizer's workgroups
        const int bpr = a.H >> 4;
        const int64_t blk = (int64_t)(blockIdx.x - a.route_blocks) * kRouteThreads + threadIdx.x;
        if (blk < (int64_t)a.T * bpr)
            quantize_block16(a.x, a.x_row_stride, *a.gscale, a.H, (int)(blk / bpr),
                             (int)(blk % bpr), a.codes, a.sf);
        return;
    }
    if (mode == kTopkOnly) {
        topk_tokens(a, blockIdx.x * kRouteWaves, a.route_blocks * kRouteWaves, lds, nullptr);
    } else if (mode == kPermuteOnly) {
        if (a.T * a.K > kWaveMaxRoutes) permute_block(a, a.ids, lds);
        else permute_small(a, a.ids, lds);
    } else {
        // ids of all routes first, then the region top-k and permutation share
        int32_t* s_ids = lds;
        int32_t* work = lds + ((a.T * a.K + 3) & ~3);
        topk_tokens(a, 0, kRouteWaves, work, s_ids);
        __syncthreads();
        if (a.T * a.K > kWaveMaxRoutes) permute_block(a, s_ids, work);
        else permute_small(a, s_ids, work);
    }
}

// ---------------------------------------------------------------- many routes
// The same metadata as permute_block, by the whole grid: a stable counting
// sort in three launches over chunks of 512 consecutive routes.
//   count:   per chunk, the routes of each local expert (LDS atomics; counts do
//            not depend on their order) -> meta's perm_counts [chunk][expert]
//   scan:    one workgroup: per-expert totals, padded offsets, each chunk's
//            first row in each expert (in place), the tile map
//   scatter: per chunk, each route's rank among the chunk's earlier routes of
//            its expert (ballot matching within a wave, a prefix over the
//            chunk's waves in LDS), added to the chunk's first row; and a
//            share of the padding rows and of the sync words per workgroup
constexpr int kChunk = kRouteThreads;
constexpr int kGridPermMinRoutes = 512;           // more routes than this: the grid-wide permutation

__global__ void __launch_bounds__(kRouteThreads) perm_count_kernel(RouteArgs a) {
    extern __shared__ int32_t lds[];                   // [El]
    const int El = a.local_num, R = a.T * a.K, tid = threadIdx.x;
    for (int x = tid; x < El; x += kRouteThreads) lds[x] = 0;
    __syncthreads();
    const int r = blockIdx.x * kChunk + tid;
    if (r < R) {
        const int e = local_expert(a, a.ids[r]);
        if (e >= 0) atomicAdd(&lds[e], 1);
    }
    __syncthreads();
    int32_t* cnt = a.meta + a.L.perm_counts + (int64_t)blockIdx.x * El;
    for (int x = tid; x < El; x += kRouteThreads) cnt[x] = lds[x];
}

__global__ void __launch_bounds__(kRouteThreads) perm_scan_kernel(RouteArgs a, int nchunks) {
    extern __shared__ int32_t lds[];
    const int El = a.local_num, m = a.tile_m;
    const int tiles_max = (int)a.L.tiles_max;
    int32_t* count = lds;                          // [El]
    int32_t* offs = count + El;                    // [El + 1]
    int32_t* scan = offs + El + 1;                 // [kRouteWaves]
    int32_t* tile_e = scan + kRouteWaves;          // [tiles_max]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t* cnt = a.meta + a.L.perm_counts;
    int32_t* tile_expert = a.meta + a.L.tile_expert;
    // each thread owns a contiguous run of experts. Its chunk counts load
    // kScanBatch at a time, all in flight together (a chunk's counts of
    // consecutive experts are adjacent: the wave's loads coalesce); up to
    // kScanBatch chunks they stay in registers for the in-place pass below.
    constexpr int kScanBatch = 64;
    const int per = (El + kRouteThreads - 1) / kRouteThreads;
    const int e0 = tid * per, e1 = min(El, e0 + per);
    const bool held = per == 1 && nchunks <= kScanBatch;
    int v[kScanBatch];
    int my_total = 0;
    for (int x = e0; x < e1; ++x) {
        int c = 0;
        for (int b0 = 0; b0 < nchunks; b0 += kScanBatch) {
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) v[i] = b0 + i < nchunks ? cnt[(int64_t)(b0 + i) * El + x] : 0;
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) c += v[i];
        }
        count[x] = c;
        my_total += (c + m - 1) / m * m;
    }
    const int incl = wave_inclusive_scan(my_total);
    if (lane == 63) scan[w] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int ww = 0; ww < w; ++ww) wave_base += scan[ww];
    int acc = wave_base + incl - my_total;
    for (int x = e0; x < e1; ++x) {
        offs[x] = acc;
        int base = acc;                            // the chunks' first rows, in place
        for (int b0 = 0; b0 < nchunks; b0 += kScanBatch) {
            if (!held) {
#pragma unroll
                for (int i = 0; i < kScanBatch; ++i) v[i] = b0 + i < nchunks ? cnt[(int64_t)(b0 + i) * El + x] : 0;
            }
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i)
                if (b0 + i < nchunks) {
                    cnt[(int64_t)(b0 + i) * El + x] = base;
                    base += v[i];
                }
        }
        acc += (count[x] + m - 1) / m * m;
    }
    if (tid == kRouteThreads - 1) offs[El] = wave_base + incl;
    __syncthreads();
    const int total_rows = offs[El], num_tiles = total_rows / m;
    for (int x = tid; x <= El; x += kRouteThreads) a.meta[a.L.expert_offsets + x] = offs[x];
    for (int x = tid; x < El; x += kRouteThreads) a.meta[a.L.expert_counts + x] = count[x];
    if (tid == 0) {
        a.meta[a.L.num_tiles] = num_tiles;
        a.meta[a.L.total_rows] = total_rows;
    }
    for (int x = tid; x < El; x += kRouteThreads)
        for (int tile = offs[x] / m; tile < offs[x + 1] / m; ++tile) tile_e[tile] = x;
    for (int tile = num_tiles + tid; tile < tiles_max; tile += kRouteThreads) tile_e[tile] = -1;
    __syncthreads();
    for (int tile = tid; tile < tiles_max; tile += kRouteThreads) tile_expert[tile] = tile_e[tile];
}

__global__ void __launch_bounds__(kRouteThreads) perm_scatter_kernel(RouteArgs a) {
    extern __shared__ int32_t lds[];                   // [kRouteWaves][El]
    const int El = a.local_num, R = a.T * a.K;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int32_t* first = a.meta + a.L.perm_counts + (int64_t)blockIdx.x * El;
    int32_t* exp2perm = a.meta + a.L.exp2perm;
    int32_t* perm2tok = a.meta + a.L.perm2tok;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int i = tid; i < kRouteWaves * El; i += kRouteThreads) lds[i] = 0;
    __syncthreads();
    const int r = blockIdx.x * kChunk + tid;
    const int e = r < R ? local_expert(a, a.ids[r]) : -1;
    const uint64_t match = same_expert_lanes(e);
    const int rank_in_wave = __popcll(match & lt_mask);
    if (e >= 0 && rank_in_wave == 0) lds[w * El + e] = __popcll(match);
    __syncthreads();
    for (int x = tid; x < El; x += kRouteThreads) {   // exclusive prefix over the chunk's waves
        int acc = first[x];
#pragma unroll
        for (int ww = 0; ww < kRouteWaves; ++ww) {
            const int c = lds[ww * El + x];
            lds[ww * El + x] = acc;
            acc += c;
        }
    }
    __syncthreads();
    if (r < R) {
        if (e >= 0) {
            const int pos = lds[w * El + e] + rank_in_wave;
            exp2perm[r] = pos;
            perm2tok[pos] = r / a.K;
        } else {
            exp2perm[r] = -1;
        }
    }
    // this workgroup's share of the padding rows (-1: no route lands there) and
    // of the sync words; the tile map, offsets and counts are the scan's
    const int rows_max = (int)a.L.rows_max, m = a.tile_m;
    const int share = (rows_max + gridDim.x - 1) / gridDim.x;
    const int row0 = blockIdx.x * share, row1 = min(rows_max, row0 + share);
    const int32_t* tile_expert = a.meta + a.L.tile_expert;
    const int32_t* offs = a.meta + a.L.expert_offsets;
    const int32_t* counts = a.meta + a.L.expert_counts;
    for (int row = row0 + tid; row < row1; row += kRouteThreads) {
        const int ex = tile_expert[row / m];
        if (ex < 0 || row - offs[ex] >= counts[ex]) perm2tok[row] = -1;
    }
    const int64_t words = 2 * a.L.subs_max, wshare = (words + gridDim.x - 1) / gridDim.x;
    int32_t* sync = a.meta + a.L.sub_sync;
    for (int64_t x = blockIdx.x * wshare + tid; x < min(words, (blockIdx.x + 1) * wshare); x += kRouteThreads)
        sync[(x >> 1) * kSubSyncStride + (x & 1)] = 0;
    const int64_t tshare = (a.T + gridDim.x - 1) / gridDim.x;
    int32_t* tok = a.meta + a.L.tok_sync;
    for (int64_t x = blockIdx.x * tshare + tid; x < min((int64_t)a.T, (blockIdx.x + 1) * tshare); x += kRouteThreads) {
        tok[x * kTokSyncStride] = 0;
        tok[x * kTokSyncStride + 1] = 0;
        tok[x * kTokSyncStride + 2] = 0;
    }
    if (blockIdx.x == 0 && tid == 0) a.meta[a.L.sync_status] = 0;
    if (blockIdx.x == 0 && tid < kQueueWords) a.meta[a.L.queue + tid] = 0;
}

static size_t topk_lds_bytes(int E, int K) {
    if (E > kRankMaxExperts) return 0;
    return sizeof(int32_t) * ((size_t)2 * kRouteWaves * ((E + 3) & ~3) + (size_t)kRouteWaves * K * 2);
}

static size_t permute_lds_bytes(int El, int64_t tiles_max) {
    const size_t block = (size_t)(kRouteWaves + 3) * El + 1 + kRouteWaves;   // permute_block
    const size_t small = (size_t)3 * El + 1 + (size_t)tiles_max;              // permute_small
    return sizeof(int32_t) * (block > small ? block : small);
}

int moe_route_check(int T, int E, int K, int tile_m, int local_expert_offset, int local_num_experts,
                    int64_t logits_row_stride, const float* logits, const int32_t* topk_ids,
                    const float* topk_weights, const int32_t* meta, const char* name) {
    if (T < 0) return fail(MOE_EINVAL, "%s: T=%d", name, T);
    if (E < 1 || E > MOE_MAX_EXPERTS)
        return fail(MOE_EUNSUPPORTED, "%s: E=%d outside [1, %d]", name, E, MOE_MAX_EXPERTS);
    if (K < 1 || K > E || K > MOE_MAX_TOPK)
        return fail(MOE_EUNSUPPORTED, "%s: K=%d outside [1, min(E, %d)]", name, K, MOE_MAX_TOPK);
    if (local_num_experts < 1 || local_num_experts > MOE_MAX_EXPERTS || local_expert_offset < 0)
        return fail(MOE_EINVAL, "%s: local experts [%d, +%d) invalid", name, local_expert_offset,
                    local_num_experts);
    if (tile_m < 16 || tile_m > 256 || tile_m % 16)
        return fail(MOE_EUNSUPPORTED, "%s: tile_m=%d must be a multiple of 16 in [16, 256]", name,
                    tile_m);
    if (logits_row_stride < E) return fail(MOE_EINVAL, "%s: logits row stride < E", name);
    if (!meta) return fail(MOE_EINVAL, "%s: meta is NULL", name);
    if (T > 0 && (!logits || !topk_ids || !topk_weights))
        return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(meta) || (T > 0 && (!aligned16(logits) || !aligned16(topk_ids) ||
                                        !aligned16(topk_weights))))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if ((int64_t)T * K > 0x3FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too many routes", name);
    return MOE_OK;
}

static int route_launch(const float* logits, int64_t logits_row_stride, const float* expert_bias,
                        const uint8_t* is_padding, int T, int E, int K, float route_scale,
                        int tile_m, int local_expert_offset, int local_num_experts,
                        int32_t* topk_ids, float* topk_weights, int32_t* meta,
                        const uint16_t* x, int64_t x_row_stride, const float* gscale, int H,
                        uint8_t* codes, uint8_t* sf, void* stream, const char* name) {
    const int rc = moe_route_check(T, E, K, tile_m, local_expert_offset, local_num_experts, logits_row_stride,
                                   logits, topk_ids, topk_weights, meta, name);
    if (rc != MOE_OK) return rc;
    RouteArgs a;
    a.logits = logits; a.logits_row_stride = logits_row_stride; a.bias = expert_bias;
    a.is_padding = is_padding; a.T = T; a.E = E; a.K = K; a.route_scale = route_scale;
    a.tile_m = tile_m; a.local_offset = local_expert_offset; a.local_num = local_num_experts;
    a.ids = topk_ids; a.weights = topk_weights; a.meta = meta;
    a.L = meta_layout(T, K, local_num_experts, tile_m);
    a.x = x; a.x_row_stride = x_row_stride; a.gscale = gscale; a.H = H; a.codes = codes; a.sf = sf;
    const int64_t qblocks = x ? ((int64_t)T * (H / 16) + kRouteThreads - 1) / kRouteThreads : 0;
    if (qblocks > 0x3FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too large", name);
    const size_t topk_lds = topk_lds_bytes(E, K), perm_lds = permute_lds_bytes(local_num_experts, a.L.tiles_max);
    // more than 512 routes of more than 8 tokens: the grid-wide permutation,
    // as long as its scan's LDS (tile map included) fits; else one workgroup
    const int64_t R = (int64_t)T * K;
    const size_t scan_lds =
        sizeof(int32_t) * ((size_t)2 * local_num_experts + 1 + kRouteWaves + (size_t)a.L.tiles_max);
    const bool grid_perm = T > kFusedMaxTokens && R > kGridPermMinRoutes && scan_lds <= 64 * 1024;
    hipStream_t s = (hipStream_t)stream;
    if (T <= kFusedMaxTokens) {
        const size_t lds = sizeof(int32_t) * (((size_t)T * K + 3) & ~(size_t)3) +
                           (topk_lds > perm_lds ? topk_lds : perm_lds);
        a.route_blocks = 1;
        hipLaunchKernelGGL(route_kernel, dim3((unsigned)(1 + qblocks)), dim3(kRouteThreads), lds, s,
                           a, (int)kFused);
    } else {
        const int64_t tb = (T + kRouteWaves - 1) / kRouteWaves;
        a.route_blocks = (int)(tb < 4096 ? tb : 4096);
        hipLaunchKernelGGL(route_kernel, dim3((unsigned)(a.route_blocks + qblocks)),
                           dim3(kRouteThreads), topk_lds, s, a, (int)kTopkOnly);
        int rc = check_launch(name);
        if (rc) return rc;
        a.route_blocks = 1;
        a.x = nullptr;
        if (!grid_perm) {
            hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), perm_lds, s, a,
                               (int)kPermuteOnly);
        } else {
            const int nchunks = (int)((R + kChunk - 1) / kChunk);
            const int El = local_num_experts;
            hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nchunks), dim3(kRouteThreads),
                               sizeof(int32_t) * El, s, a);
            rc = check_launch(name);
            if (rc) return rc;
            hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(kRouteThreads), scan_lds, s, a, nchunks);
            rc = check_launch(name);
            if (rc) return rc;
            hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)nchunks), dim3(kRouteThreads),
                               sizeof(int32_t) * kRouteWaves * El, s, a);
        }
    }
    return check_launch(name);
}

}  // namespace moe

extern "C" int moe_route(const float* logits, int64_t logits_row_stride, const float* expert_bias,
                         const uint8_t* is_padding, int T, int E, int K, float route_scale,
                         int tile_m, int local_expert_offset, int local_num_experts,
                         int32_t* topk_ids, float* topk_weights, int32_t* meta, void* stream) {
    return moe::route_launch(logits, logits_row_stride, expert_bias, is_padding, T, E, K,
                             route_scale, tile_m, local_expert_offset, local_num_experts, topk_ids,
                             topk_weights, meta, nullptr, 0, nullptr, 0, nullptr, nullptr, stream,
                             "moe_route");
}

extern "C" int moe_route_quant(const float* logits, int64_t logits_row_stride,
                               const float* expert_bias, const uint8_t* is_padding, int T, int E,
                               int K, float route_scale, int tile_m, int local_expert_offset,
                               int local_num_experts, int32_t* topk_ids, float* topk_weights,
                               int32_t* meta, const uint16_t* x, int64_t x_row_stride,
                               const float* gscale, int H, uint8_t* codes, uint8_t* sf,
                               void* stream) {
    using namespace moe;
    const int rc = quant_check(x, x_row_stride, gscale, T, H, codes, sf, "moe_route_quant");
    if (rc != MOE_OK) return rc;
    const bool quant = T > 0 && H > 0;
    return route_launch(logits, logits_row_stride, expert_bias, is_padding, T, E, K, route_scale,
                        tile_m, local_expert_offset, local_num_experts, topk_ids, topk_weights,
                        meta, quant ? x : nullptr, x_row_stride, gscale, H, codes, sf, stream,
                        "moe_route_quant");
}

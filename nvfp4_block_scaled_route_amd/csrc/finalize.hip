// moe_finalize: gather each route's GEMM2 row, per-route RMSNorm with an fp32
// output, fp32 top-k weighted sum, bf16 out -- the runner page,
// "MusePostExpertFinalize", "_finalize_native", "_finalize_chunk",
// "_effective_weight". Tensor-parallel K-partial rows are summed in fp32 and
// rounded once to bf16 before the norm (the expert_tp page, "probe_rel_l2").
//
// One workgroup per token; a thread owns C 8-column chunks (C = 1, or 2 above
// 8192 columns). Routes go in batches of 8 whose row loads issue together: the
// sum of squares of each route (a fixed-order wave reduction, then the waves
// in order), then sum_k w_k * y_k in fp32, k ascending, from the rows still in
// registers (batches past the first 8 routes are read again). Every order is
// fixed: the output is deterministic.
#include "common.hpp"

namespace moe {

constexpr int kFinBatch = 8;
constexpr int kFinMaxThreads = 1024;

struct FinArgs {
    const uint16_t* rows;
    int64_t rows_stride;
    int n_partials;
    int64_t partial_stride;
    const int32_t* exp2perm;
    const float* weights;
    const uint16_t* norm_weight;
    float gain_center, eps;
    int weight_before_norm;
    int T, K, H;
    uint16_t* out;
};

__device__ __forceinline__ void unpack8(const uint4& q, float v[8]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu); v[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
}

// Route row p at columns [8c, 8c + 8) as 8 bf16 values: with several partials
// their fp32 sum in order, rounded once to bf16.
__device__ __forceinline__ uint4 load_row8(const FinArgs& a, int p, int c) {
    const uint16_t* base = a.rows + (int64_t)p * a.rows_stride + 8 * c;
    uint4 q = *reinterpret_cast<const uint4*>(base);
    if (a.n_partials == 1) return q;
    float v[8];
    unpack8(q, v);
    for (int part = 1; part < a.n_partials; ++part) {
        float u[8];
        unpack8(*reinterpret_cast<const uint4*>(base + part * a.partial_stride), u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __fadd_rn(v[i], u[i]);
    }
    q.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    q.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    q.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
    q.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
    return q;
}

__device__ __forceinline__ void gamma8(const FinArgs& a, int c, float g[8]) {
    if (a.norm_weight) {
        unpack8(*reinterpret_cast<const uint4*>(a.norm_weight + 8 * c), g);
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = __fadd_rn(g[i], a.gain_center);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = __fadd_rn(1.0f, a.gain_center);
    }
}

// The rows of routes [k0, k0 + 8) at the thread's chunks (zeros where absent).
template <int C>
__device__ __forceinline__ void load_batch(const FinArgs& a, const int32_t* ep, int k0, int tid,
                                           int nthreads, int nchunks, uint4 raw[C][kFinBatch]) {
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
        const int k = k0 + kk;
        const int p = k < a.K ? ep[k] : -1;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int chunk = tid + c * nthreads;
            raw[c][kk] = make_uint4(0u, 0u, 0u, 0u);
            if (p >= 0 && chunk < nchunks) raw[c][kk] = load_row8(a, p, chunk);
        }
    }
}

template <int C>
__global__ void __launch_bounds__(kFinMaxThreads) finalize_kernel(FinArgs a) {
    __shared__ float s_part[kFinMaxThreads / 64][kFinBatch];
    __shared__ float s_inv[MOE_MAX_TOPK];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nthreads = blockDim.x, nwaves = nthreads >> 6;
    const int nchunks = a.H >> 3;
    const int32_t* ep = a.exp2perm + (int64_t)t * a.K;
    const float* wp = a.weights + (int64_t)t * a.K;
    float g[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (tid + c * nthreads < nchunks) gamma8(a, tid + c * nthreads, g[c]);
    uint4 raw[C][kFinBatch];

    // sums of squares, batch by batch
    for (int k0 = 0; k0 < a.K; k0 += kFinBatch) {
        load_batch<C>(a, ep, k0, tid, nthreads, nchunks, raw);
        float ss[kFinBatch];
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk) {
            ss[kk] = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (tid + c * nthreads >= nchunks) continue;
                float v[8];
                unpack8(raw[c][kk], v);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float z = a.weight_before_norm ? __fmul_rn(g[c][i], v[i]) : v[i];
                    ss[kk] = __fadd_rn(ss[kk], __fmul_rn(z, z));
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) ss[kk] = __fadd_rn(ss[kk], __shfl_xor(ss[kk], off));
        }
        if (lane < kFinBatch) {
            float mine = ss[0];
#pragma unroll
            for (int kk = 1; kk < kFinBatch; ++kk) mine = lane == kk ? ss[kk] : mine;
            s_part[wv][lane] = mine;
        }
        __syncthreads();
        if (tid < kFinBatch && k0 + tid < a.K) {
            float total = 0.0f;
            for (int w = 0; w < nwaves; ++w) total = __fadd_rn(total, s_part[w][tid]);
            s_inv[k0 + tid] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(total, (float)a.H), a.eps)));
        }
        __syncthreads();
    }

    // weighted sum over the routes, k ascending
    float acc[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += kFinBatch) {
        if (a.K > kFinBatch) load_batch<C>(a, ep, k0, tid, nthreads, nchunks, raw);
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk) {
            const int k = k0 + kk;
            if (k >= a.K || ep[k] < 0) continue;     // a missing row normalizes to zero
            const float wk = wp[k], inv = s_inv[k];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                float v[8];
                unpack8(raw[c][kk], v);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float y = a.weight_before_norm ? __fmul_rn(__fmul_rn(g[c][i], v[i]), inv)
                                                         : __fmul_rn(g[c][i], __fmul_rn(v[i], inv));
                    acc[c][i] = __fadd_rn(acc[c][i], __fmul_rn(y, wk));
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int chunk = tid + c * nthreads;
        if (chunk >= nchunks) continue;
        uint4 o;
        o.x = f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16);
        o.y = f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16);
        o.z = f32_to_bf16(acc[c][4]) | (f32_to_bf16(acc[c][5]) << 16);
        o.w = f32_to_bf16(acc[c][6]) | (f32_to_bf16(acc[c][7]) << 16);
        *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.H + 8 * chunk) = o;
    }
}

}  // namespace moe

extern "C" int moe_finalize(const uint16_t* rows, int64_t rows_stride, int n_partials,
                            int64_t partial_stride, const int32_t* exp2perm,
                            const float* topk_weights, const uint16_t* norm_weight,
                            float gain_center, float eps, int weight_before_norm, int T, int K,
                            int H, uint16_t* out, void* stream) {
    using namespace moe;
    if (T < 0 || K < 1 || K > MOE_MAX_TOPK)
        return fail(MOE_EINVAL, "moe_finalize: T=%d K=%d out of range", T, K);
    if (H < 8 || H % 8 || H > MOE_MAX_HIDDEN)
        return fail(MOE_EUNSUPPORTED, "moe_finalize: H=%d must be a multiple of 8 in [8, %d]", H,
                    MOE_MAX_HIDDEN);
    if (n_partials < 1 || n_partials > 16)
        return fail(MOE_EUNSUPPORTED, "moe_finalize: n_partials=%d outside [1, 16]", n_partials);
    if (T == 0) return MOE_OK;
    if (!rows || !exp2perm || !topk_weights || !out) return fail(MOE_EINVAL, "moe_finalize: NULL pointer");
    if (!aligned16(rows) || !aligned16(exp2perm) || !aligned16(topk_weights) || !aligned16(out) ||
        (norm_weight && !aligned16(norm_weight)))
        return fail(MOE_EINVAL, "moe_finalize: pointers must be 16-byte aligned");
    if (rows_stride < H || rows_stride % 8 || (n_partials > 1 && partial_stride % 8))
        return fail(MOE_EINVAL, "moe_finalize: strides must be multiples of 8, rows_stride >= H");
    FinArgs a;
    a.rows = rows; a.rows_stride = rows_stride; a.n_partials = n_partials;
    a.partial_stride = partial_stride; a.exp2perm = exp2perm; a.weights = topk_weights;
    a.norm_weight = norm_weight; a.gain_center = gain_center; a.eps = eps;
    a.weight_before_norm = weight_before_norm ? 1 : 0; a.T = T; a.K = K; a.H = H; a.out = out;
    // threads: every 8-column chunk owned once, at most 1024 threads of 1 or 2 chunks
    const int nchunks = H / 8;
    const int C = nchunks > kFinMaxThreads ? 2 : 1;
    const int threads = ((nchunks + C - 1) / C + 63) / 64 * 64;
    if (C == 1)
        hipLaunchKernelGGL(finalize_kernel<1>, dim3(T), dim3(threads), 0, (hipStream_t)stream, a);
    else
        hipLaunchKernelGGL(finalize_kernel<2>, dim3(T), dim3(threads), 0, (hipStream_t)stream, a);
    return check_launch("moe_finalize");
}

// moe_finalize: gather each route's GEMM2 row, per-route RMSNorm with an fp32
// output, fp32 top-k weighted sum, bf16 out -- the runner page,
// "MusePostExpertFinalize", "_finalize_native", "_finalize_chunk",
// "_effective_weight". Tensor-parallel K-partial rows are summed in fp32 and
// rounded once to bf16 before the norm (the expert_tp page, "probe_rel_l2").
//
// One 512-thread workgroup (8 waves) per token. Pass 1: wave w forms the sum of
// squares of routes k = w, w + 8, ... (a lane walks 8-column chunks lane,
// lane + 64, ...; then a fixed-order wave reduction), so no block-wide
// reduction is needed. Pass 2: a thread owns 8-column chunks tid, tid + 512, ...
// and accumulates sum_k w_k * y_k in fp32, k ascending. Rows are re-read in
// pass 2 (cache hits). Every order is fixed: the output is deterministic.
#include "common.hpp"

namespace moe {

constexpr int kFinThreads = 512;
constexpr int kFinWaves = kFinThreads / 64;

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

// 8 values of route row p at columns [8c, 8c + 8): partials summed in fp32 in
// order, rounded once to bf16 when there is more than one.
__device__ __forceinline__ void load_row8(const FinArgs& a, int p, int c, float v[8]) {
    const uint16_t* base = a.rows + (int64_t)p * a.rows_stride + 8 * c;
    uint4 q = *reinterpret_cast<const uint4*>(base);
    {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu); v[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
    }
    if (a.n_partials > 1) {
        for (int part = 1; part < a.n_partials; ++part) {
            q = *reinterpret_cast<const uint4*>(base + part * a.partial_stride);
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __fadd_rn(v[2 * i], bf16_to_f32(u[i] & 0xFFFFu));
                v[2 * i + 1] = __fadd_rn(v[2 * i + 1], bf16_to_f32(u[i] >> 16));
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(f32_to_bf16(v[i]));
    }
}

__device__ __forceinline__ void gamma8(const FinArgs& a, int c, float g[8]) {
    if (a.norm_weight) {
        const uint4 q = *reinterpret_cast<const uint4*>(a.norm_weight + 8 * c);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g[2 * i] = __fadd_rn(bf16_to_f32(w[i] & 0xFFFFu), a.gain_center);
            g[2 * i + 1] = __fadd_rn(bf16_to_f32(w[i] >> 16), a.gain_center);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = __fadd_rn(1.0f, a.gain_center);
    }
}

__global__ void __launch_bounds__(kFinThreads) finalize_kernel(FinArgs a) {
    __shared__ int s_perm[MOE_MAX_TOPK];
    __shared__ float s_w[MOE_MAX_TOPK];
    __shared__ float s_inv[MOE_MAX_TOPK];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nchunks = a.H >> 3;
    if (tid < a.K) {
        s_perm[tid] = a.exp2perm[(int64_t)t * a.K + tid];
        s_w[tid] = a.weights[(int64_t)t * a.K + tid];
    }
    __syncthreads();
    // pass 1: one wave per route
    for (int k = wv; k < a.K; k += kFinWaves) {
        const int p = s_perm[k];
        float ss = 0.0f;
        if (p >= 0) {
            for (int c = lane; c < nchunks; c += 64) {
                float v[8], g[8];
                load_row8(a, p, c, v);
                if (a.weight_before_norm) gamma8(a, c, g);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float z = a.weight_before_norm ? __fmul_rn(g[i], v[i]) : v[i];
                    ss = __fadd_rn(ss, __fmul_rn(z, z));
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss = __fadd_rn(ss, __shfl_xor(ss, off));
        if (lane == 0) s_inv[k] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(ss, (float)a.H), a.eps)));
    }
    __syncthreads();
    // pass 2: weighted sum over routes
    for (int c = tid; c < nchunks; c += kFinThreads) {
        float g[8];
        gamma8(a, c, g);
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = 0; k < a.K; ++k) {
            const int p = s_perm[k];
            if (p < 0) continue;            // a zero row normalizes to zero
            const float wk = s_w[k], inv = s_inv[k];
            float v[8];
            load_row8(a, p, c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float y = a.weight_before_norm ? __fmul_rn(__fmul_rn(g[i], v[i]), inv)
                                                     : __fmul_rn(g[i], __fmul_rn(v[i], inv));
                acc[i] = __fadd_rn(acc[i], __fmul_rn(y, wk));
            }
        }
        uint4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        *reinterpret_cast<uint4*>(a.out + (int64_t)t * a.H + 8 * c) = o;
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
    hipLaunchKernelGGL(finalize_kernel, dim3(T), dim3(kFinThreads), 0, (hipStream_t)stream, a);
    return check_launch("moe_finalize");
}

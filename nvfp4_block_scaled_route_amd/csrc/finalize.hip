// moe_finalize: gather each route's GEMM2 row, per-route RMSNorm with an fp32
// output, fp32 top-k weighted sum, bf16 out -- the runner page,
// "MusePostExpertFinalize", "_finalize_native", "_finalize_chunk",
// "_effective_weight". Tensor-parallel K-partial rows are summed in fp32 and
// rounded once to bf16 before the norm (the expert_tp page, "probe_rel_l2").
//
// One workgroup of up to 1024 threads per token, a thread owning W consecutive
// columns (W = 2, 4 or 8 by H, T and the partial count: fin_w; C = 2 column
// groups per thread only above 8192 columns), so that little serial work falls
// on any one wave. Routes go in batches of 8 whose row loads issue together: the sum
// of squares of each route (a DPP wave reduction in fixed order, then the
// waves' partials in a fixed-order 16-lane reduction), then sum_k w_k * y_k in
// fp32, k ascending, from the rows still in registers (batches past the first
// 8 routes are read again). Every order is fixed: the output is deterministic.
// With tensor-parallel partials the 4-column form loads a route's partials 4
// at a time before adding them in order: in the layer, where the partial rows
// come from other XCDs' writes, expert_tp8_b32's layer 384.2 -> 376.0 µs (8
// partials; the finalize about 26 -> 18 µs).
#include "finalize.hpp"

namespace moe {

// The rows of routes [k0, k0 + 8) at the thread's columns (zeros where absent),
// with the routes' permuted rows and weights (uniform values, loaded first).
template <int W, int C>
__device__ __forceinline__ void load_batch(const FinArgs& a, int t, int k0, int tid, int nthreads,
                                           int ngroups, Cols<W> raw[C][kFinBatch],
                                           int perm[kFinBatch], float wk[kFinBatch]) {
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
        const int k = k0 + kk;
        perm[kk] = k < a.K ? a.exp2perm[(int64_t)t * a.K + k] : -1;
        wk[kk] = k < a.K ? a.weights[(int64_t)t * a.K + k] : 0.0f;
    }
#pragma unroll
    for (int kk = 0; kk < kFinBatch; ++kk) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int grp = tid + c * nthreads;
#pragma unroll
            for (int i = 0; i < W / 2; ++i) raw[c][kk].w[i] = 0u;
            if (perm[kk] >= 0 && grp < ngroups) raw[c][kk] = load_row<W, W == 4 ? 4 : 1>(a, perm[kk], grp);
        }
    }
}

template <int W, int C>
__global__ void __launch_bounds__(kFinMaxThreads) finalize_kernel(FinArgs a) {
    __shared__ float s_part[kFinBatch][kFinMaxWaves];
    __shared__ float s_inv[MOE_MAX_TOPK];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nthreads = blockDim.x, nwaves = nthreads >> 6;
    const int ngroups = a.H / W;
    float g[C][W];
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (tid + c * nthreads < ngroups) gamma_cols<W>(a, tid + c * nthreads, g[c]);
    Cols<W> raw[C][kFinBatch];
    int perm[kFinBatch];
    float wk[kFinBatch];

    // sums of squares, batch by batch
    for (int k0 = 0; k0 < a.K; k0 += kFinBatch) {
        load_batch<W, C>(a, t, k0, tid, nthreads, ngroups, raw, perm, wk);
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk) {
            float ss = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (tid + c * nthreads >= ngroups) continue;
                float v[W];
                unpack<W>(raw[c][kk], v);
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    const float z = a.weight_before_norm ? __fmul_rn(g[c][i], v[i]) : v[i];
                    ss = __fadd_rn(ss, __fmul_rn(z, z));
                }
            }
            ss = wave_sum(ss);
            if (lane == 0) s_part[kk][wv] = ss;
        }
        __syncthreads();
        fin_inv_tree(a, k0, tid, nthreads, nwaves, s_part, s_inv);
        __syncthreads();
    }

    // weighted sum over the routes, k ascending
    float acc[C][W];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int i = 0; i < W; ++i) acc[c][i] = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += kFinBatch) {
        if (a.K > kFinBatch) load_batch<W, C>(a, t, k0, tid, nthreads, ngroups, raw, perm, wk);
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk) {
            if (k0 + kk >= a.K || perm[kk] < 0) continue;   // a missing row normalizes to zero
            const float inv = s_inv[k0 + kk];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                float v[W];
                unpack<W>(raw[c][kk], v);
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    const float y = a.weight_before_norm ? __fmul_rn(__fmul_rn(g[c][i], v[i]), inv)
                                                         : __fmul_rn(g[c][i], __fmul_rn(v[i], inv));
                    acc[c][i] = __fadd_rn(acc[c][i], __fmul_rn(y, wk[kk]));
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int grp = tid + c * nthreads;
        if (grp >= ngroups) continue;
        store_cols<W>(a.out + (int64_t)t * a.H + W * grp, pack<W>(acc[c]));
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
    const int W = fin_w(H, T, n_partials), C = fin_c(H, T, n_partials), threads = fin_threads(H, T, n_partials);
    hipStream_t s = (hipStream_t)stream;
    if (W == 2)
        hipLaunchKernelGGL((finalize_kernel<2, 1>), dim3(T), dim3(threads), 0, s, a);
    else if (W == 4)
        hipLaunchKernelGGL((finalize_kernel<4, 1>), dim3(T), dim3(threads), 0, s, a);
    else if (C == 1)
        hipLaunchKernelGGL((finalize_kernel<8, 1>), dim3(T), dim3(threads), 0, s, a);
    else
        hipLaunchKernelGGL((finalize_kernel<8, 2>), dim3(T), dim3(threads), 0, s, a);
    return check_launch("moe_finalize");
}

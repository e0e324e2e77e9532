// moe_finalize: gather each route's GEMM2 row, per-route RMSNorm with an fp32
// output, fp32 top-k weighted sum, bf16 out -- the runner page,
// "MusePostExpertFinalize", "_finalize_native", "_finalize_chunk",
// "_effective_weight". Tensor-parallel K-partial rows are summed in fp32 and
// rounded once to bf16 before the norm (the expert_tp page, "probe_rel_l2").
//
// One workgroup of up to 1024 threads per token, a thread owning W consecutive
// columns (W = 2, 4 or 8: the smallest that fits; C = 2 column groups per
// thread only above 8192 columns), so that little serial work falls on any
// one wave. Routes go in batches of 8 whose row loads issue together: the sum
// of squares of each route (a DPP wave reduction in fixed order, then the
// waves' partials in a fixed-order 16-lane reduction), then sum_k w_k * y_k in
// fp32, k ascending, from the rows still in registers (batches past the first
// 8 routes are read again). Every order is fixed: the output is deterministic.
#include "common.hpp"

namespace moe {

constexpr int kFinBatch = 8;
constexpr int kFinMaxThreads = 1024;
constexpr int kFinMaxWaves = kFinMaxThreads / 64;   // 16: one DPP row

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

// W bf16 values (W / 2 words)
template <int W>
struct Cols {
    uint32_t w[W / 2];
};

template <int W>
__device__ __forceinline__ Cols<W> load_cols(const uint16_t* p) {
    Cols<W> c;
    if constexpr (W == 8) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        c.w[0] = q.x; c.w[1] = q.y; c.w[2] = q.z; c.w[3] = q.w;
    } else if constexpr (W == 4) {
        const uint2 q = *reinterpret_cast<const uint2*>(p);
        c.w[0] = q.x; c.w[1] = q.y;
    } else {
        c.w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    return c;
}

template <int W>
__device__ __forceinline__ void unpack(const Cols<W>& c, float v[W]) {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) { v[2 * i] = bf16_to_f32(c.w[i] & 0xFFFFu); v[2 * i + 1] = bf16_to_f32(c.w[i] >> 16); }
}

template <int W>
__device__ __forceinline__ Cols<W> pack(const float v[W]) {
    Cols<W> c;
#pragma unroll
    for (int i = 0; i < W / 2; ++i) c.w[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
    return c;
}

// Route row p at columns [W*c, W*c + W): with several partials their fp32 sum
// in order, rounded once to bf16.
template <int W>
__device__ __forceinline__ Cols<W> load_row(const FinArgs& a, int p, int c) {
    const uint16_t* base = a.rows + (int64_t)p * a.rows_stride + W * c;
    Cols<W> q = load_cols<W>(base);
    if (a.n_partials == 1) return q;
    float v[W];
    unpack<W>(q, v);
    for (int part = 1; part < a.n_partials; ++part) {
        float u[W];
        unpack<W>(load_cols<W>(base + part * a.partial_stride), u);
#pragma unroll
        for (int i = 0; i < W; ++i) v[i] = __fadd_rn(v[i], u[i]);
    }
    return pack<W>(v);
}

template <int W>
__device__ __forceinline__ void gamma_cols(const FinArgs& a, int c, float g[W]) {
    if (a.norm_weight) {
        unpack<W>(load_cols<W>(a.norm_weight + W * c), g);
#pragma unroll
        for (int i = 0; i < W; ++i) g[i] = __fadd_rn(g[i], a.gain_center);
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) g[i] = __fadd_rn(1.0f, a.gain_center);
    }
}

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
            if (perm[kk] >= 0 && grp < ngroups) raw[c][kk] = load_row<W>(a, perm[kk], grp);
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
        for (int idx = tid; idx < kFinBatch * kFinMaxWaves; idx += nthreads) {   // whole waves
            // lane (k, w) of a 16-lane row: wave w's partial of route k0 + k
            const int k = idx >> 4, w = idx & 15;
            float v = w < nwaves ? s_part[k][w] : 0.0f;
            v = __fadd_rn(v, dpp_f<kDppQuadXor1>(v));
            v = __fadd_rn(v, dpp_f<kDppQuadXor2>(v));
            v = __fadd_rn(v, dpp_f<kDppRowHalfMirror>(v));
            v = __fadd_rn(v, dpp_f<kDppRowMirror>(v));
            if (w == 0 && k0 + k < a.K)
                s_inv[k0 + k] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)a.H), a.eps)));
        }
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
        const Cols<W> o = pack<W>(acc[c]);
        uint16_t* dst = a.out + (int64_t)t * a.H + W * grp;
        if constexpr (W == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(o.w[0], o.w[1], o.w[2], o.w[3]);
        else if constexpr (W == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(o.w[0], o.w[1]);
        else *reinterpret_cast<uint32_t*>(dst) = o.w[0];
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
    // columns per thread: the fewest that fit 1024 threads (two groups of 8
    // above 8192 columns)
    const int W = H <= 2048 ? 2 : H <= 4096 ? 4 : 8;
    const int C = H / W > kFinMaxThreads ? 2 : 1;
    const int threads = ((H / W + C - 1) / C + 63) / 64 * 64;
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

// The post-expert finalize's arithmetic, shared by moe_finalize
// (finalize.hip) and the finalize run inside the one-launch expert kernel
// (experts.hip, moe_experts_finalize): the runner page, "MusePostExpertFinalize",
// "_finalize_native", "_finalize_chunk", "_effective_weight". Both take every
// sum in the same order, so their outputs agree bit for bit:
//   * a virtual thread vt of N_v = ceil(ceil(H/W)/C / 64) * 64 owns the W
//     consecutive columns W (vt + c N_v), c < C;
//   * a route's sum of squares runs over its thread's columns (c, then i),
//     then over the 64 lanes of its virtual wave (wave_sum), then over the
//     virtual waves in a fixed 16-lane tree;
//   * the weighted sum runs over k ascending, per column.
// moe_finalize has one real thread per virtual thread; the expert kernel's 256
// threads each play N_v / 256 of them in turn.
#pragma once
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
    if constexpr (W == 16) {
        const uint4 q0 = reinterpret_cast<const uint4*>(p)[0], q1 = reinterpret_cast<const uint4*>(p)[1];
        c.w[0] = q0.x; c.w[1] = q0.y; c.w[2] = q0.z; c.w[3] = q0.w;
        c.w[4] = q1.x; c.w[5] = q1.y; c.w[6] = q1.z; c.w[7] = q1.w;
    } else if constexpr (W == 8) {
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
// in order, rounded once to bf16. With B > 1 the partials' loads go out B at
// a time before their additions, instead of each waiting for the one before.
template <int W, int B = 1>
__device__ __forceinline__ Cols<W> load_row(const FinArgs& a, int p, int c) {
    const uint16_t* base = a.rows + (int64_t)p * a.rows_stride + W * c;
    Cols<W> q = load_cols<W>(base);
    if (a.n_partials == 1) return q;
    float v[W];
    unpack<W>(q, v);
    for (int part0 = 1; part0 < a.n_partials; part0 += B) {
        Cols<W> u[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (part0 + j < a.n_partials) u[j] = load_cols<W>(base + (part0 + j) * a.partial_stride);
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (part0 + j >= a.n_partials) break;
            float f[W];
            unpack<W>(u[j], f);
#pragma unroll
            for (int i = 0; i < W; ++i) v[i] = __fadd_rn(v[i], f[i]);
        }
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


// buffer-load cache policy: agent-coherent (sc1), for rows another XCD wrote
// in the same launch with agent-coherent stores
constexpr int kCoherentLoad = 16;

template <int W>
__device__ __forceinline__ void store_cols(uint16_t* dst, const Cols<W>& o) {
    if constexpr (W == 16) {
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(o.w[0], o.w[1], o.w[2], o.w[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(o.w[4], o.w[5], o.w[6], o.w[7]);
    } else if constexpr (W == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(o.w[0], o.w[1], o.w[2], o.w[3]);
    else if constexpr (W == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(o.w[0], o.w[1]);
    else *reinterpret_cast<uint32_t*>(dst) = o.w[0];
}

// The virtual waves' partial sums of squares of routes [k0, k0 + 8), reduced
// in a fixed 16-lane tree (lane (k, w) of a DPP row holds virtual wave w's
// partial of route k0 + k), into the routes' 1 / rms. Run by threads
// [0, 128) of the workgroup: whole waves.
__device__ __forceinline__ void fin_inv_tree(const FinArgs& a, int k0, int tid, int nreal, int nwaves_v,
                                             float (*s_part)[kFinMaxWaves], float* s_inv) {
    for (int idx = tid; idx < kFinBatch * kFinMaxWaves; idx += nreal) {
        const int k = idx >> 4, w = idx & 15;
        float v = w < nwaves_v ? s_part[k][w] : 0.0f;
        v = __fadd_rn(v, dpp_f<kDppQuadXor1>(v));
        v = __fadd_rn(v, dpp_f<kDppQuadXor2>(v));
        v = __fadd_rn(v, dpp_f<kDppRowHalfMirror>(v));
        v = __fadd_rn(v, dpp_f<kDppRowMirror>(v));
        if (w == 0 && k0 + k < a.K)
            s_inv[k0 + k] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(v, (float)a.H), a.eps)));
    }
}

// Columns per thread and column groups of the finalize of T tokens x H
// columns with n_partials partial rows per route, and the (virtual) thread
// count. Wider threads issue fewer, larger loads (16 bytes at W = 8): measured
// on prefill_t4096 (T = 4096, H = 4096) 61 µs at W = 8 against 68 at W = 4,
// decode_b8 (H = 2048) 5.0 µs at W = 4 against 5.6 at W = 2. Where few tokens
// spread over few workgroups (or several partials are summed per route) the
// narrower form keeps more loads in flight per token (expert_tp8_b32: 16.1 µs
// at W = 4, 16.9 at W = 8), and the finalize inside the expert launch takes W
// up to 4 only (its registers are the GEMM workgroups' too). Two groups of 8
// columns a thread above 8192 columns.
__host__ __device__ constexpr int fin_w(int H, int T, int n_partials) {
    return H <= 1024 ? 2 : H <= 2048 ? 4 : (H > 4096 || (n_partials == 1 && T >= 512)) ? 8 : 4;
}
__host__ __device__ constexpr int fin_c(int H, int T, int n_partials) {
    return H / fin_w(H, T, n_partials) > kFinMaxThreads ? 2 : 1;
}
__host__ __device__ constexpr int fin_threads(int H, int T, int n_partials) {
    const int w = fin_w(H, T, n_partials), c = fin_c(H, T, n_partials);
    return ((H / w + c - 1) / c + 63) / 64 * 64;
}

// A route row's W columns at column group grp, with several partials summed
// in fp32 and rounded once, read with agent-coherent loads (rows another XCD
// wrote in the same launch). p is uniform over the workgroup.
template <int W>
__device__ __forceinline__ Cols<W> load_row_coherent(const FinArgs& a, int p, int grp) {
    float v[W];
    Cols<W> q;
    for (int part = 0; part < a.n_partials; ++part) {
        const uint16_t* base = a.rows + part * a.partial_stride + (int64_t)p * a.rows_stride;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
        const int off = grp * W * 2;
        if constexpr (W == 16) {
            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentLoad);
            const u32x4v y = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kCoherentLoad);
            q.w[0] = x[0]; q.w[1] = x[1]; q.w[2] = x[2]; q.w[3] = x[3];
            q.w[4] = y[0]; q.w[5] = y[1]; q.w[6] = y[2]; q.w[7] = y[3];
        } else if constexpr (W == 8) {
            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentLoad);
            q.w[0] = x[0]; q.w[1] = x[1]; q.w[2] = x[2]; q.w[3] = x[3];
        } else if constexpr (W == 4) {
            typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
            const u32x2v x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherentLoad);
            q.w[0] = x[0]; q.w[1] = x[1];
        } else {
            q.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherentLoad);
        }
        if (a.n_partials == 1) return q;
        float u[W];
        unpack<W>(q, u);
        if (part == 0) {
#pragma unroll
            for (int i = 0; i < W; ++i) v[i] = u[i];
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) v[i] = __fadd_rn(v[i], u[i]);
        }
    }
    return pack<W>(v);
}

// Token t's output row by the workgroup's nreal threads (a multiple of 64),
// as moe_finalize computes it: real thread tid plays virtual threads
// tid + j nreal below fin_threads(H, T, n_partials), whole waves at a time. s_part
// [kFinBatch][kFinMaxWaves] and s_inv [MOE_MAX_TOPK] are the workgroup's LDS.
// Row loads are agent-coherent. Ends with a barrier.
template <int W, int C>
__device__ void finalize_token(const FinArgs& a, int t, int tid, int nreal, float (*s_part)[kFinMaxWaves],
                               float* s_inv) {
    const int lane = tid & 63;
    const int nthreads_v = fin_threads(a.H, a.T, a.n_partials), nwaves_v = nthreads_v >> 6;
    const int V = (nthreads_v + nreal - 1) / nreal;
    const int ngroups = a.H / W;
    // sums of squares, batch by batch
    for (int k0 = 0; k0 < a.K; k0 += kFinBatch) {
        int perm[kFinBatch];
#pragma unroll
        for (int kk = 0; kk < kFinBatch; ++kk)
            perm[kk] = k0 + kk < a.K ? a.exp2perm[(int64_t)t * a.K + k0 + kk] : -1;
        for (int j = 0; j < V; ++j) {
            const int vt = tid + j * nreal;
            if (vt >= nthreads_v) break;                 // uniform over the wave
            float ss[kFinBatch];
#pragma unroll
            for (int kk = 0; kk < kFinBatch; ++kk) ss[kk] = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int grp = vt + c * nthreads_v;
                if (grp >= ngroups) continue;
                float g[W];
                gamma_cols<W>(a, grp, g);
#pragma unroll
                for (int kk = 0; kk < kFinBatch; ++kk) {
                    if (perm[kk] < 0) continue;
                    float v[W];
                    unpack<W>(load_row_coherent<W>(a, perm[kk], grp), v);
#pragma unroll
                    for (int i = 0; i < W; ++i) {
                        const float z = a.weight_before_norm ? __fmul_rn(g[i], v[i]) : v[i];
                        ss[kk] = __fadd_rn(ss[kk], __fmul_rn(z, z));
                    }
                }
            }
#pragma unroll
            for (int kk = 0; kk < kFinBatch; ++kk) {
                const float r = wave_sum(ss[kk]);
                if (lane == 0) s_part[kk][vt >> 6] = r;
            }
        }
        __syncthreads();
        fin_inv_tree(a, k0, tid, nreal, nwaves_v, s_part, s_inv);
        __syncthreads();
    }
    // weighted sum over the routes, k ascending
    for (int j = 0; j < V; ++j) {
        const int vt = tid + j * nreal;
        if (vt >= nthreads_v) break;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int grp = vt + c * nthreads_v;
            if (grp >= ngroups) continue;
            float g[W], acc[W];
            gamma_cols<W>(a, grp, g);
#pragma unroll
            for (int i = 0; i < W; ++i) acc[i] = 0.0f;
            for (int k = 0; k < a.K; ++k) {
                const int p = a.exp2perm[(int64_t)t * a.K + k];
                if (p < 0) continue;                 // a missing row normalizes to zero
                const float inv = s_inv[k], wk = a.weights[(int64_t)t * a.K + k];
                float v[W];
                unpack<W>(load_row_coherent<W>(a, p, grp), v);
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    const float y = a.weight_before_norm ? __fmul_rn(__fmul_rn(g[i], v[i]), inv)
                                                         : __fmul_rn(g[i], __fmul_rn(v[i], inv));
                    acc[i] = __fadd_rn(acc[i], __fmul_rn(y, wk));
                }
            }
            store_cols<W>(a.out + (int64_t)t * a.H + W * grp, pack<W>(acc));
        }
    }
    __syncthreads();
}

}  // namespace moe

// nvfp4_norm_quant: the pre-expert RMSNorm run inside the NVFP4 input
// quantizer -- the model page, "MuseSpark1xMoE" (pre_expert_norm: weight,
// zero-centred gain, eps; "norm_fuses_into_nvfp4_quant": the weight applies
// after normalizing) and "_prepared_nvfp4_forward" (norm_quant_trtllm_nvfp4:
// pooled rows, norm weight, eps, fused gain centre, input global scale ->
// NVFP4 codes and block scales).
//
// Per row of H values (bf16 x, each step one correctly rounded operation):
//   s  = sum_j x_j^2  in fp64 (the squares are exact)
//   ms = fp32(s / H);  r = 1 / sqrt(ms + eps)  (fp32)
//   y_j = (x_j * r) * gamma_j,  gamma_j = fp32(w_j) + gain_center
//   y -> NVFP4 with the input global scale, as nvfp4_quant does with x.
// The normalized row is not rounded to bf16: it goes to the quantizer in fp32.
//
// HBM-bound (2H bytes in, 9H/16 out per row). One wave per row: lane l takes
// the 16-value blocks l, l + 64, ..., so a wave's loads of one round are 2 KB
// of consecutive bytes. Up to H = 4096 the row stays in registers between the
// sum of squares and the quantization (the row is read once); wider rows are
// read a second time, from the cache.
#include "common.hpp"

namespace moe {

constexpr int kNqThreads = 256;   // four rows per workgroup

struct NqArgs {
    const uint16_t* x;
    int64_t x_row_stride;
    const uint16_t* norm_weight;
    float gain_center, eps;
    const float* gscale;
    int T, H;
    uint8_t* codes;
    uint8_t* sf;
};

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

struct Block16 {
    uint4 lo, hi;   // 16 bf16 values
};

__device__ __forceinline__ Block16 load_block(const uint16_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    return Block16{q[0], q[1]};
}

__device__ __forceinline__ void unpack16(const Block16& b, float v[16]) {
    const uint32_t w[8] = {b.lo.x, b.lo.y, b.lo.z, b.lo.w, b.hi.x, b.hi.y, b.hi.z, b.hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

__device__ __forceinline__ double sum_squares(const Block16& b) {
    float v[16];
    unpack16(b, v);
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double d = (double)v[i];
        s = __dadd_rn(s, __dmul_rn(d, d));
    }
    return s;
}

// y = (x * r) * gamma over one block, then its NVFP4 codes and scale.
__device__ __forceinline__ void norm_quant_block(const NqArgs& a, int64_t t, int b, const Block16& xb, float r,
                                                 float gs) {
    float v[16], g[16];
    unpack16(xb, v);
    if (a.norm_weight) {
        unpack16(load_block(a.norm_weight + b * 16), g);
#pragma unroll
        for (int i = 0; i < 16; ++i) g[i] = __fadd_rn(g[i], a.gain_center);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) g[i] = __fadd_rn(1.0f, a.gain_center);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = __fmul_rn(__fmul_rn(v[i], r), g[i]);
        amax = fmaxf(amax, __builtin_fabsf(v[i]));
    }
    const BlockScale bs = nvfp4_block_scale(amax, gs);
    const uint32_t lo = nvfp4_codes8<true>(v, bs), hi = nvfp4_codes8<true>(v + 8, bs);
    *reinterpret_cast<uint2*>(a.codes + t * (a.H >> 1) + b * 8) = make_uint2(lo, hi);
    a.sf[t * (a.H >> 4) + b] = (uint8_t)bs.byte;
}

// NB > 0: each lane holds its (at most NB) blocks in registers; NB == 0: the
// row is read twice.
template <int NB>
__global__ void __launch_bounds__(kNqThreads) norm_quant_kernel(NqArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * (kNqThreads / 64) + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int nblk = a.H >> 4;
    const uint16_t* row = a.x + t * a.x_row_stride;
    double ss = 0.0;
    Block16 held[NB > 0 ? NB : 1];
    if constexpr (NB > 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + 64 * i;
            if (b < nblk) held[i] = load_block(row + b * 16);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (lane + 64 * i < nblk) ss = __dadd_rn(ss, sum_squares(held[i]));
    } else {
        for (int b = lane; b < nblk; b += 64) ss = __dadd_rn(ss, sum_squares(load_block(row + b * 16)));
    }
    ss = wave_sum_f64(ss);
    const float ms = __double2float_rn(__ddiv_rn(ss, (double)a.H));
    const float r = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(ms, a.eps)));
    const float gs = *a.gscale;
    if constexpr (NB > 0) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = lane + 64 * i;
            if (b < nblk) norm_quant_block(a, t, b, held[i], r, gs);
        }
    } else {
        for (int b = lane; b < nblk; b += 64) norm_quant_block(a, t, b, load_block(row + b * 16), r, gs);
    }
}

}  // namespace moe

extern "C" int nvfp4_norm_quant(const uint16_t* x, int64_t x_row_stride, const uint16_t* norm_weight,
                                float gain_center, float eps, const float* gscale, int T, int H,
                                uint8_t* codes, uint8_t* sf, void* stream) {
    using namespace moe;
    const int rc = quant_check(x, x_row_stride, gscale, T, H, codes, sf, "nvfp4_norm_quant");
    if (rc != MOE_OK) return rc;
    if (H > MOE_MAX_HIDDEN) return fail(MOE_EUNSUPPORTED, "nvfp4_norm_quant: H=%d above %d", H, MOE_MAX_HIDDEN);
    if (!(eps > 0.0f) || eps > 1.0f || !(gain_center == gain_center))
        return fail(MOE_EINVAL, "nvfp4_norm_quant: eps must be in (0, 1] and the gain centre a number");
    if (norm_weight && !aligned16(norm_weight))
        return fail(MOE_EINVAL, "nvfp4_norm_quant: norm_weight must be 16-byte aligned");
    if (T == 0 || H == 0) return MOE_OK;
    NqArgs a;
    a.x = x; a.x_row_stride = x_row_stride; a.norm_weight = norm_weight; a.gain_center = gain_center;
    a.eps = eps; a.gscale = gscale; a.T = T; a.H = H; a.codes = codes; a.sf = sf;
    const int64_t grid = ((int64_t)T + kNqThreads / 64 - 1) / (kNqThreads / 64);
    if (grid > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "nvfp4_norm_quant: too many rows");
    hipStream_t s = (hipStream_t)stream;
    const dim3 g((unsigned)grid), b(kNqThreads);
    if (H <= 1024) hipLaunchKernelGGL(norm_quant_kernel<1>, g, b, 0, s, a);
    else if (H <= 2048) hipLaunchKernelGGL(norm_quant_kernel<2>, g, b, 0, s, a);
    else if (H <= 4096) hipLaunchKernelGGL(norm_quant_kernel<4>, g, b, 0, s, a);
    else hipLaunchKernelGGL(norm_quant_kernel<0>, g, b, 0, s, a);
    return check_launch("nvfp4_norm_quant");
}

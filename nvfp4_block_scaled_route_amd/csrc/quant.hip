// nvfp4_quant: NVFP4 quantization of the expert input (one global scale,
// row-major e4m3 block scales) -- the model page, "_prepared_nvfp4_forward".
// HBM-bound: one thread owns one 16-value block (32 bytes in, 8 + 1 out).
#include "common.hpp"

namespace moe {

__global__ void __launch_bounds__(256) nvfp4_quant_kernel(const uint16_t* __restrict__ x,
                                                          int64_t x_row_stride,
                                                          const float* __restrict__ gscale_p,
                                                          int T, int H, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ sf) {
    const int blocks_per_row = H >> 4;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= (int64_t)T * blocks_per_row) return;
    const int t = (int)(blk / blocks_per_row);
    const int b = (int)(blk - (int64_t)t * blocks_per_row);
    const uint4* src = reinterpret_cast<const uint4*>(x + t * x_row_stride + b * 16);
    const uint4 p0 = src[0], p1 = src[1];
    const uint32_t w[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        amax = fmaxf(amax, fmaxf(__builtin_fabsf(v[2 * i]), __builtin_fabsf(v[2 * i + 1])));
    }
    const BlockScale bs = nvfp4_block_scale(amax, *gscale_p);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= nvfp4_code(v[i], bs) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= nvfp4_code(v[8 + i], bs) << (4 * i);
    *reinterpret_cast<uint2*>(codes + (int64_t)t * (H >> 1) + b * 8) = make_uint2(lo, hi);
    sf[(int64_t)t * blocks_per_row + b] = (uint8_t)bs.byte;
}

}  // namespace moe

extern "C" int nvfp4_quant(const uint16_t* x, int64_t x_row_stride, const float* gscale, int T,
                           int H, uint8_t* codes, uint8_t* sf, void* stream) {
    using namespace moe;
    if (T < 0 || H < 0) return fail(MOE_EINVAL, "nvfp4_quant: negative size T=%d H=%d", T, H);
    if (H % 16) return fail(MOE_EUNSUPPORTED, "nvfp4_quant: H=%d is not a multiple of 16", H);
    if (T == 0 || H == 0) return MOE_OK;
    if (!x || !gscale || !codes || !sf) return fail(MOE_EINVAL, "nvfp4_quant: NULL pointer");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(sf) || !aligned16(gscale))
        return fail(MOE_EINVAL, "nvfp4_quant: pointers must be 16-byte aligned");
    if (x_row_stride < H || x_row_stride % 8)
        return fail(MOE_EINVAL, "nvfp4_quant: row stride %lld must be >= H and a multiple of 8",
                    (long long)x_row_stride);
    const int64_t blocks = (int64_t)T * (H / 16);
    const int64_t grid = (blocks + 255) / 256;
    if (grid > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "nvfp4_quant: too large");
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, x,
                       x_row_stride, gscale, T, H, codes, sf);
    return check_launch("nvfp4_quant");
}

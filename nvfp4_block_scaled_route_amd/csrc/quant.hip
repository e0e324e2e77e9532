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
    quantize_block16(x, x_row_stride, *gscale_p, H, t, b, codes, sf);
}

// Host-side checks shared with moe_route_quant.
int quant_check(const uint16_t* x, int64_t x_row_stride, const float* gscale, int T, int H,
                uint8_t* codes, uint8_t* sf, const char* name) {
    if (T < 0 || H < 0) return fail(MOE_EINVAL, "%s: negative size T=%d H=%d", name, T, H);
    if (H % 16) return fail(MOE_EUNSUPPORTED, "%s: H=%d is not a multiple of 16", name, H);
    if (T == 0 || H == 0) return MOE_OK;
    if (!x || !gscale || !codes || !sf) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(x) || !aligned16(codes) || !aligned16(sf) || !aligned16(gscale))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    if (x_row_stride < H || x_row_stride % 8)
        return fail(MOE_EINVAL, "%s: row stride %lld must be >= H and a multiple of 8", name,
                    (long long)x_row_stride);
    if ((int64_t)T * (H / 16) > ((int64_t)1 << 40)) return fail(MOE_EUNSUPPORTED, "%s: too large", name);
    return MOE_OK;
}

}  // namespace moe

extern "C" int nvfp4_quant(const uint16_t* x, int64_t x_row_stride, const float* gscale, int T,
                           int H, uint8_t* codes, uint8_t* sf, void* stream) {
    using namespace moe;
    const int rc = quant_check(x, x_row_stride, gscale, T, H, codes, sf, "nvfp4_quant");
    if (rc != MOE_OK || T == 0 || H == 0) return rc;
    const int64_t blocks = (int64_t)T * (H / 16);
    const int64_t grid = (blocks + 255) / 256;
    if (grid > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "nvfp4_quant: too large");
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, x,
                       x_row_stride, gscale, T, H, codes, sf);
    return check_launch("nvfp4_quant");
}

// moe_pack_w13 / moe_pack_w2: logical NVFP4 expert weights -> the converted
// layout the expert kernels read (moe_nvfp4.h, "weights"). Run once at load,
// like the weight conversion of the runner page,
// "MuseSparkModelOptNvFp4FusedMoE.process_weights_after_loading".
//
// Both layouts keep elements 2j and 2j+1 of a row in one byte (low nibble
// first), so the conversion permutes whole bytes: one thread writes 4
// consecutive converted code bytes (elements k..k+7 of one row) and, for the
// scales, one thread writes one converted scale byte.
#include "common.hpp"

namespace moe {

// converted row -> logical row (w13: the gated interleave; w2: identity)
__device__ __forceinline__ int64_t logical_row(int64_t rho, int interleave_half) {
    if (interleave_half == 0) return rho;
    const int64_t c = rho >> 5, w = rho & 31;
    return w < 16 ? 16 * c + w : interleave_half + 16 * c + (w - 16);
}

// out_codes: E * (N/16) * (K/64) tiles of 512 bytes; thread -> one u32 of a tile
__global__ void __launch_bounds__(256) pack_codes_kernel(const uint8_t* __restrict__ in, int E,
                                                         int N, int K, int interleave_half,
                                                         uint32_t* __restrict__ out) {
    const int64_t total = (int64_t)E * N * K / 8;          // u32 words out
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int tiles_k = K / 64;
    const int64_t tile = i >> 7;                           // 128 words per tile
    const int word = (int)(i & 127);                       // = (q*16 + n)*2 + s
    const int s = word & 1, n = (word >> 1) & 15, q = word >> 5;
    const int64_t e = tile / ((int64_t)(N / 16) * tiles_k);
    const int64_t rem = tile - e * (N / 16) * tiles_k;
    const int64_t g = rem / tiles_k;
    const int t = (int)(rem - g * tiles_k);
    const int64_t row = logical_row(g * 16 + n, interleave_half);
    const int k = t * 64 + s * 32 + q * 8;                 // 8 elements = 4 bytes
    const uint8_t* src = in + (e * N + row) * (int64_t)(K / 2) + k / 2;
    out[i] = *reinterpret_cast<const uint32_t*>(src);
}

// out_sf: E * (N/16) * (K/64) tiles of 64 bytes; thread -> one byte
__global__ void __launch_bounds__(256) pack_scales_kernel(const uint8_t* __restrict__ in, int E,
                                                          int N, int K, int interleave_half,
                                                          uint8_t* __restrict__ out) {
    const int64_t total = (int64_t)E * N * K / 16;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int tiles_k = K / 64;
    const int64_t tile = i >> 6;
    const int byte = (int)(i & 63);                        // = ((b%2)*16 + n)*2 + b/2
    const int bhi = byte & 1, n = (byte >> 1) & 15, blo = byte >> 5;
    const int b = bhi * 2 + blo;
    const int64_t e = tile / ((int64_t)(N / 16) * tiles_k);
    const int64_t rem = tile - e * (N / 16) * tiles_k;
    const int64_t g = rem / tiles_k;
    const int t = (int)(rem - g * tiles_k);
    const int64_t row = logical_row(g * 16 + n, interleave_half);
    out[i] = in[(e * N + row) * (int64_t)(K / 16) + t * 4 + b];
}

static int pack(const char* name, const uint8_t* codes, const uint8_t* sf, int E, int N, int K,
                int interleave_half, uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    if (E < 0 || N < 0 || K < 0) return fail(MOE_EINVAL, "%s: negative size", name);
    if (N % 16 || K % 64) return fail(MOE_EUNSUPPORTED, "%s: rows %d must be a multiple of 16 and columns %d of 64", name, N, K);
    if ((int64_t)E * N * K == 0) return MOE_OK;
    if (!codes || !sf || !out_codes || !out_sf) return fail(MOE_EINVAL, "%s: NULL pointer", name);
    if (!aligned16(codes) || !aligned16(sf) || !aligned16(out_codes) || !aligned16(out_sf))
        return fail(MOE_EINVAL, "%s: pointers must be 16-byte aligned", name);
    const int64_t words = (int64_t)E * N * K / 8, sbytes = (int64_t)E * N * K / 16;
    if ((words + 255) / 256 > 0x7FFFFFFF) return fail(MOE_EUNSUPPORTED, "%s: too large", name);
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                       codes, E, N, K, interleave_half, reinterpret_cast<uint32_t*>(out_codes));
    int rc = check_launch(name);
    if (rc) return rc;
    hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((sbytes + 255) / 256)), dim3(256), 0, s,
                       sf, E, N, K, interleave_half, out_sf);
    return check_launch(name);
}

}  // namespace moe

extern "C" int moe_pack_w13(const uint8_t* codes, const uint8_t* sf, int E, int I, int H,
                            uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    if (I % 16) return moe::fail(MOE_EUNSUPPORTED, "moe_pack_w13: I=%d is not a multiple of 16", I);
    return moe::pack("moe_pack_w13", codes, sf, E, 2 * I, H, I, out_codes, out_sf, stream);
}

extern "C" int moe_pack_w2(const uint8_t* codes, const uint8_t* sf, int E, int H, int I,
                           uint8_t* out_codes, uint8_t* out_sf, void* stream) {
    return moe::pack("moe_pack_w2", codes, sf, E, H, I, 0, out_codes, out_sf, stream);
}
